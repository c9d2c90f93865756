// HIP kernels of the decode attention block for CDNA4 (gfx950), wave64.
//
// Steps and their source (docs.rs turbospark-runtime 0.3.0):
//   gemv_bf16_kernel     -- the fused q_k_v_proj GEMV with the g_proj rows
//                           appended, and the o_proj GEMV
//                           ([attn.rs] `encode_attention_block`, GEMV steps)
//   attn_partial_kernel  -- the split into the cache slot, per-class NeoX RoPE
//                           of q and k, and split-K decode attention over the
//                           window/ring ([attn.rs] split, RoPE, window and
//                           attention steps; [kv_write.rs] `kv_write_target`,
//                           `encode_attention_any`)
//   attn_combine_kernel  -- merge of the split-K partials and the headwise
//                           sigmoid gate ([attn.rs] gate step, before o_proj)
//   rms_norm_kernel, residual_add_kernel -- the layer loop around the block
//                           ([mod.rs] `produce_real_spark_inner`)
//
// All of it is HBM-bandwidth bound (about 1-4 flop per byte): the kernels are
// built to keep many 16-byte loads in flight per wave and to read every weight
// and every attended K/V byte exactly once.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gqa_internal.h"

namespace gqa {
namespace {

// ---------------------------------------------------------------------------
// wave-level helpers
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Buffer loads: 32-bit byte offsets from a per-buffer resource.  An offset at
// or past the resource's size returns zeros without a memory access, which is
// how rows and columns that must not be read are skipped without branches.
// ---------------------------------------------------------------------------
constexpr unsigned kOutOfRange = 0x80000000u;   // every buffer here is < 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

__device__ __forceinline__ float dot8_bf16(uint4 q, float4 xa, float4 xb, float a) {
  a = fmaf(bf16_lo(q.x), xa.x, a);
  a = fmaf(bf16_hi(q.x), xa.y, a);
  a = fmaf(bf16_lo(q.y), xa.z, a);
  a = fmaf(bf16_hi(q.y), xa.w, a);
  a = fmaf(bf16_lo(q.z), xb.x, a);
  a = fmaf(bf16_hi(q.z), xb.y, a);
  a = fmaf(bf16_lo(q.w), xb.z, a);
  a = fmaf(bf16_hi(q.w), xb.w, a);
  return a;
}

// ---------------------------------------------------------------------------
// GEMV: y[b][r] = sum_c W[r][c] x[b][c], bf16 W, fp32 x/y/accumulation.
//
// One wave owns R consecutive rows.  Lane l reads columns
// [(it*64 + l)*8, +8) for it < NIT, so each 16-byte load instruction covers
// 1 KiB of one row contiguously; all R*NIT loads are issued before the first
// FMA so a wave keeps R*NIT KiB in flight.  The weights stay in registers
// while the batch is walked MB rows at a time, so W is read once per call.
// ---------------------------------------------------------------------------
template <int R, int NIT, int MB>
__global__ __launch_bounds__(kThreads) void gemv_bf16_kernel(const GemvParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int total = p.rows0 + p.rows1;
  const int row0 = wave * R;
  if (row0 >= total) return;
  const unsigned row_bytes = (unsigned)p.cols * 2u;
  const __amdgpu_buffer_rsrc_t r0 = make_rsrc(p.w0, (unsigned)p.rows0 * row_bytes);
  const __amdgpu_buffer_rsrc_t r1 = make_rsrc(p.w1, (unsigned)p.rows1 * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (unsigned)((size_t)p.batch * p.ldx * 4u));

  uint4 w[R][NIT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    const bool first = row < p.rows0;
    const unsigned base = first ? (unsigned)row * row_bytes : (unsigned)(row - p.rows0) * row_bytes;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int col = (it * 64 + lane) * 8;
      const unsigned off = (row < total && col < p.cols) ? base + (unsigned)col * 2u : kOutOfRange;
      w[r][it] = first ? buf_load16(r0, off) : buf_load16(r1, off);
    }
  }

  for (int b0 = 0; b0 < p.batch; b0 += MB) {
    float acc[R][MB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[r][m] = 0.f;

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int col = (it * 64 + lane) * 8;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const unsigned xo = (col < p.cols && b0 + m < p.batch)
                                ? (unsigned)(((size_t)(b0 + m) * p.ldx + col) * 4u)
                                : kOutOfRange;
        const float4 xa = __builtin_bit_cast(float4, buf_load16(rx, xo));
        const float4 xb = __builtin_bit_cast(float4, buf_load16(rx, xo == kOutOfRange ? xo : xo + 16u));
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][m] = dot8_bf16(w[r][it], xa, xb, acc[r][m]);
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const float s = wave_sum(acc[r][m]);
        if (lane == r * MB + m && row < total && b0 + m < p.batch) {
          if (row < p.rows0)
            p.y0[(size_t)(b0 + m) * p.ldy0 + row] = s;
          else
            p.y1[(size_t)(b0 + m) * p.ldy1 + (row - p.rows0)] = s;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV.  NIT is exactly ceil(cols/512), so no registers hold loads
// that would only return zeros; x (the lane's 8*NIT columns) stays in
// registers for the wave's R rows.  Fewer registers than the batched kernel
// means more resident waves per CU and more bytes in flight.
// ---------------------------------------------------------------------------
template <int R, int NIT>
__global__ __launch_bounds__(kThreads) void gemv1_bf16_kernel(const GemvParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int total = p.rows0 + p.rows1;
  const int row0 = wave * R;
  if (row0 >= total) return;
  const unsigned row_bytes = (unsigned)p.cols * 2u;
  const __amdgpu_buffer_rsrc_t r0 = make_rsrc(p.w0, (unsigned)p.rows0 * row_bytes);
  const __amdgpu_buffer_rsrc_t r1 = make_rsrc(p.w1, (unsigned)p.rows1 * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (unsigned)p.cols * 4u);

  uint4 w[R][NIT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    const bool first = row < p.rows0;
    const unsigned base = first ? (unsigned)row * row_bytes : (unsigned)(row - p.rows0) * row_bytes;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int col = (it * 64 + lane) * 8;
      const unsigned off = (row < total && col < p.cols) ? base + (unsigned)col * 2u : kOutOfRange;
      w[r][it] = first ? buf_load16(r0, off) : buf_load16(r1, off);
    }
  }
  float4 xa[NIT], xb[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int col = (it * 64 + lane) * 8;
    const unsigned xo = col < p.cols ? (unsigned)col * 4u : kOutOfRange;
    xa[it] = __builtin_bit_cast(float4, buf_load16(rx, xo));
    xb[it] = __builtin_bit_cast(float4, buf_load16(rx, xo + 16u));
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float a = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) a = dot8_bf16(w[r][it], xa[it], xb[it], a);
    const float s = wave_sum(a);
    const int row = row0 + r;
    if (lane == r && row < total) {
      if (row < p.rows0)
        p.y0[row] = s;
      else
        p.y1[row - p.rows0] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention, split-K over the window.
//
// Grid (total_chunks, Hk).  Workgroup (chunk c of sequence b, KV head g)
// owns logical positions [t0, t1) of that sequence and the 4 query heads
// 4g..4g+3 that read KV head g, so every K/V byte is read from HBM once and
// used for 4 heads.  Each of the 4 waves owns a contiguous quarter of the
// chunk and runs its own online softmax over it in tiles of RPT rows, with no
// workgroup barrier in the loop: while a wave computes tile i, the K and V
// loads of tile i+1 are already in flight (ping-pong register buffers).  K and
// V are read with buffer loads (32-bit offsets; a row that must not be read
// gets an offset past the end of the buffer, which returns zeros without an
// HBM access).
//
//   prologue  RoPE table (fp64 angle reduction), q of the 4 heads rotated and
//             scaled by scale*log2(e) into LDS.  The chunk that ends at this
//             token also rotates k, rounds k and v to fp16 once, writes both
//             to the cache slot, keeps the rounded row in LDS and scores it:
//             the kernel never reads back what it wrote.
//   per tile  scores: 16 lanes per row (lane owns dims 8s..8s+7 and
//             128+8s..+7), 4 rows per load, fp16 K straight into v_fma_mix,
//             DPP row sum.  Softmax: one (row, head) score per lane, per-head
//             max and sum by DPP/shuffles, one exp2 per lane.  P.V: lane owns
//             4 dims of a whole row (512 B per load), probabilities read back
//             from a wave-private LDS slot.
//   end       the 4 waves' (max, sum, acc) are merged in LDS and written as
//             this chunk's partial per head.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_seq(const AttnParams &p, int chunk_id) {
  int s = 0;
  for (int i = 1; i < p.nseq; ++i)
    if (chunk_id >= p.seq[i].chunk_begin) s = i;
  return s;
}

// max / sum over the lanes that hold the same head (same lane & 3)
__device__ __forceinline__ float head_max(float v) {
  v = fmaxf(v, dpp<0x124>(v));   // row_ror:4
  v = fmaxf(v, dpp<0x128>(v));   // row_ror:8
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float head_sum(float v) {
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <int RPT>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(const AttnParams p) {
  static_assert(RPT % 4 == 0 && RPT <= 16, "a tile is 1..4 groups of 4 rows");
  constexpr int kQuads = RPT / 4;
  __shared__ float s_cos[kHeadDim / 2];
  __shared__ float s_sin[kHeadDim / 2];
  __shared__ float s_q[kGroup][kHeadDim];
  __shared__ float s_kcur[kHeadDim];
  __shared__ float s_vcur[kHeadDim];
  __shared__ float s_cur[kGroup];                 // scores of this token's own row
  __shared__ float4 s_pw[4][RPT];                 // per-wave probabilities [row] x 4 heads
  __shared__ float4 s_acc[4][kGroup][kHeadDim / 4];
  __shared__ float s_mw[4][kGroup];
  __shared__ float s_lw[4][kGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
  const int g = blockIdx.y;
  const int cid = blockIdx.x;
  const int b = find_seq(p, cid);
  const SeqDesc sd = p.seq[b];
  const int Hk = p.num_kv_heads;
  const int Hq = Hk * kGroup;
  const int t0 = sd.kv_start + (cid - sd.chunk_begin) * p.chunk;
  const int seq_len = sd.kv_start + sd.n;
  const int t1 = min(t0 + p.chunk, seq_len);
  const int nrows = t1 - t0;
  const bool has_cur = (t1 == seq_len);
  const int cur_rel = seq_len - 1 - t0;          // meaningful when has_cur
  const unsigned row_bytes = (unsigned)Hk * kHeadDim * 2u;
  const int ring = sd.ring;
  const int p0 = ring ? (t0 % ring) : t0;        // physical row of t0; a chunk wraps at most once
  const int per_wave = p.chunk >> 2;
  const int wr0 = w * per_wave;                  // first row of this wave, relative to t0
  const int wrows = max(0, min(per_wave, nrows - wr0));
  const int ntiles = (wrows + RPT - 1) / RPT;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(sd.k, sd.cache_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(sd.v, sd.cache_bytes);
  const unsigned head_off = (unsigned)g * kHeadDim * 2u;

  // byte offset of row `rel` (relative to t0) of this KV head, or out of range
  // (this token's own row is never read back: it is taken from LDS)
  auto row_off = [&](int rel) -> unsigned {
    if (rel >= nrows || rel >= wr0 + wrows || (has_cur && rel == cur_rel)) return kOutOfRange;
    int ph = p0 + rel;
    if (ring && ph >= ring) ph -= ring;
    return (unsigned)ph * row_bytes + head_off;
  };
  const int sub = lane & 15;
  const int quad = lane >> 4;
  const unsigned k_lane_off = (unsigned)sub * 16u;   // lane's 16 bytes in each half row
  const unsigned v_lane_off = (unsigned)lane * 8u;   // lane's 8 bytes of a row

  uint4 kA[kQuads][2], kB[kQuads][2];
  uint2 vA[RPT], vB[RPT];
  auto load_tile = [&](uint4 (&kb)[kQuads][2], uint2 (&vb)[RPT], int it) {
    const int r0 = wr0 + it * RPT;
#pragma unroll
    for (int qi = 0; qi < kQuads; ++qi) {
      const unsigned off = row_off(r0 + qi * 4 + quad) + k_lane_off;
      kb[qi][0] = buf_load16(krs, off);
      kb[qi][1] = buf_load16(krs, off + kHeadDim);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) vb[j] = buf_load8(vrs, row_off(r0 + j) + v_lane_off);
  };
  if (ntiles > 0) load_tile(kA, vA, 0);   // HBM traffic starts before the prologue

  // ---- prologue: RoPE table, q, and this token's k/v ----
  const int rdim = p.rotary_dim;
  const int rhalf = rdim >> 1;
  if (tid < rhalf) {
    // angle = position * theta^(-2i/r), formed and reduced mod 2*pi in fp64
    // (an fp32 angle at position 32767 would be off by ~4e-3 rad); the
    // reduced angle is in [-pi, pi], where fp32 sin/cos are accurate.
    const double inv = exp2(-(2.0 * (double)tid / (double)rdim) * p.log2_theta);
    const double ang = (double)sd.position * inv;
    const double k = rint(ang * 0.15915494309189535);          // 1 / (2 pi)
    double red = fma(-k, 6.283185307179586, ang);               // 2 pi, high part
    red = fma(-k, 2.4492935982947064e-16, red);                 // 2 pi, low part
    float sn, cs;
    sincosf((float)red, &sn, &cs);
    s_cos[tid] = cs;
    s_sin[tid] = sn;
  }
  __syncthreads();

  const float *row_in = p.qkv + (size_t)b * p.ld_qkv;
  {
    const int d = tid;   // one dim of each of the 4 heads
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float *qh = row_in + (size_t)(g * kGroup + i) * kHeadDim;
      float val = qh[d];
      if (d < rdim) {
        const bool lo = d < rhalf;
        const int j = lo ? d : d - rhalf;
        const float other = lo ? qh[d + rhalf] : qh[d - rhalf];
        val = lo ? val * s_cos[j] - other * s_sin[j] : val * s_cos[j] + other * s_sin[j];
      }
      s_q[i][d] = val * p.qscale;
    }
    if (has_cur) {
      const float *kh = row_in + (size_t)Hq * kHeadDim + (size_t)g * kHeadDim;
      const float *vh = row_in + (size_t)(Hq + Hk) * kHeadDim + (size_t)g * kHeadDim;
      float kv = kh[d];
      if (d < rdim) {
        const bool lo = d < rhalf;
        const int j = lo ? d : d - rhalf;
        const float other = lo ? kh[d + rhalf] : kh[d - rhalf];
        kv = lo ? kv * s_cos[j] - other * s_sin[j] : kv * s_cos[j] + other * s_sin[j];
      }
      const _Float16 k16 = (_Float16)kv;
      const _Float16 v16 = (_Float16)vh[d];
      const size_t off = (size_t)sd.slot * Hk * kHeadDim + (size_t)g * kHeadDim + d;
      sd.k[off] = k16;
      sd.v[off] = v16;
      s_kcur[d] = (float)k16;
      s_vcur[d] = (float)v16;
    }
  }
  __syncthreads();
  if (has_cur) {   // wave w scores this token's row for head w
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(s_q[w][lane * 4 + e], s_kcur[lane * 4 + e], s);
    s = wave_sum(s);
    if (lane == 0) s_cur[w] = s;
  }
  float qreg[kGroup][16];
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qreg[i][e] = s_q[i][sub * 8 + e];
      qreg[i][8 + e] = s_q[i][kHeadDim / 2 + sub * 8 + e];
    }
  __syncthreads();

  // ---- per-wave online softmax over this wave's rows ----
  const int h_l = lane & 3;               // head of the score this lane holds
  const int q_l = (lane >> 2) & 3;        // row group of the score this lane holds
  const int r_l = 4 * q_l + quad;         // row (within the tile) of that score
  float m_run = -INFINITY;                // per head h_l
  float l_run = 0.f;
  float acc[kGroup][4];
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
  float4 *pw = s_pw[w];
  float *pwf = reinterpret_cast<float *>(pw);

  auto process = [&](const uint4 (&kb)[kQuads][2], const uint2 (&vb)[RPT], int it) {
    const int r0 = wr0 + it * RPT;
    float my_s = -INFINITY;
#pragma unroll
    for (int qi = 0; qi < kQuads; ++qi) {
      const _Float16 *k0 = reinterpret_cast<const _Float16 *>(&kb[qi][0]);
      const _Float16 *k1 = reinterpret_cast<const _Float16 *>(&kb[qi][1]);
      float a[kGroup] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ka = (float)k0[e];
        const float kc = (float)k1[e];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          a[i] = fmaf(ka, qreg[i][e], a[i]);
          a[i] = fmaf(kc, qreg[i][8 + e], a[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) a[i] = row_sum16(a[i]);
      const float sel = h_l == 0 ? a[0] : h_l == 1 ? a[1] : h_l == 2 ? a[2] : a[3];
      if (q_l == qi) my_s = sel;
    }
    const int rel = r0 + r_l;
    const bool cur_here = has_cur && rel == cur_rel;
    if (cur_here) my_s = s_cur[h_l];
    if (q_l >= kQuads || rel >= wr0 + wrows) my_s = -INFINITY;

    const float m_new = fmaxf(m_run, head_max(my_s));
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float pr = my_s == -INFINITY ? 0.f : exp2f(my_s - m_new);
    l_run = fmaf(l_run, alpha, head_sum(pr));
    m_run = m_new;
    if (q_l < kQuads) pwf[r_l * 4 + h_l] = pr;
    float al[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) al[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] *= al[i];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const float4 pp = pw[j];
      const _Float16 *vh = reinterpret_cast<const _Float16 *>(&vb[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vv = (float)vh[e];
        acc[0][e] = fmaf(vv, pp.x, acc[0][e]);
        acc[1][e] = fmaf(vv, pp.y, acc[1][e]);
        acc[2][e] = fmaf(vv, pp.z, acc[2][e]);
        acc[3][e] = fmaf(vv, pp.w, acc[3][e]);
      }
    }
    const int jc = cur_rel - r0;   // this token's row: its V comes from LDS
    if (has_cur && jc >= 0 && jc < RPT) {
      const float4 pp = pw[jc];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vv = s_vcur[lane * 4 + e];
        acc[0][e] = fmaf(vv, pp.x, acc[0][e]);
        acc[1][e] = fmaf(vv, pp.y, acc[1][e]);
        acc[2][e] = fmaf(vv, pp.z, acc[2][e]);
        acc[3][e] = fmaf(vv, pp.w, acc[3][e]);
      }
    }
  };

  for (int it = 0; it < ntiles; it += 2) {
    if (it + 1 < ntiles) load_tile(kB, vB, it + 1);
    process(kA, vA, it);
    if (it + 1 >= ntiles) break;
    if (it + 2 < ntiles) load_tile(kA, vA, it + 2);
    process(kB, vB, it + 1);
  }

  // ---- merge the 4 waves, write this chunk's partials ----
  if (lane < kGroup) {
    s_mw[w][lane] = m_run;
    s_lw[w][lane] = l_run;
  }
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
    s_acc[w][i][lane] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  __syncthreads();
  {
    const float *red = reinterpret_cast<const float *>(s_acc);
    const int d = tid;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_mw[ww][i]);
      float o = 0.f, L = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = s_mw[ww][i];
        const float wgt = mw == -INFINITY ? 0.f : exp2f(mw - M);
        o = fmaf(wgt, red[(ww * kGroup + i) * kHeadDim + d], o);
        L = fmaf(wgt, s_lw[ww][i], L);
      }
      p.part_o[((size_t)cid * Hq + g * kGroup + i) * kHeadDim + d] = o;
      if (d == 0) {
        float *ml = p.part_ml + ((size_t)cid * Hq + g * kGroup + i) * 2;
        ml[0] = M;
        ml[1] = L;
      }
    }
  }
}

// Merge of the split-K partials and the headwise gate.
// Grid (Hq * kCombineSplit, nseq).  Workgroup (h, part) owns head h and dims
// [part*64, part*64 + 64).  Thread (cg, dq): dq = tid % 16 owns 4 dims, chunk
// group cg = tid / 16 takes chunks cg, cg + 16, ...; each thread issues all
// of its loads (up to 8 at a time) before using any.
constexpr int kCombineSplit = 4;
constexpr int kCombineDims = kHeadDim / kCombineSplit;   // 64
constexpr int kCombineQuads = kCombineDims / 4;           // 16 threads per chunk row
constexpr int kCombineGroups = kThreads / kCombineQuads;  // 16 chunk groups
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const AttnParams p) {
  __shared__ float s_red[kThreads / 64];
  __shared__ float4 s_acc[kCombineGroups][kCombineQuads];
  __shared__ float s_lsum[kCombineGroups];

  const int tid = threadIdx.x;
  const int h = blockIdx.x / kCombineSplit;
  const int part = blockIdx.x % kCombineSplit;
  const int b = blockIdx.y;
  const SeqDesc sd = p.seq[b];
  const int Hq = p.num_kv_heads * kGroup;
  const int nchunks = (sd.n + p.chunk - 1) / p.chunk;
  const int f0 = sd.chunk_begin;

  // global max of the chunk maxima
  float m = -INFINITY;
  for (int c = tid; c < nchunks; c += kThreads)
    m = fmaxf(m, p.part_ml[((size_t)(f0 + c) * Hq + h) * 2]);
  m = wave_max(m);
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  const int cg = tid / kCombineQuads;
  const int dq = tid % kCombineQuads;
  const int dim0 = part * kCombineDims + dq * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
  for (int c0 = cg; c0 < nchunks; c0 += kCombineGroups * kCombineBatch) {
    float4 o[kCombineBatch];
    float2 ml[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int c = c0 + u * kCombineGroups;
      if (c < nchunks) {
        const size_t base = (size_t)(f0 + c) * Hq + h;
        ml[u] = *reinterpret_cast<const float2 *>(p.part_ml + base * 2);
        o[u] = *reinterpret_cast<const float4 *>(p.part_o + base * kHeadDim + dim0);
      } else {
        ml[u] = make_float2(-INFINITY, 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float wgt = exp2f(ml[u].x - M);   // 0 for padding entries
      lsum = fmaf(wgt, ml[u].y, lsum);
      acc.x = fmaf(wgt, o[u].x, acc.x);
      acc.y = fmaf(wgt, o[u].y, acc.y);
      acc.z = fmaf(wgt, o[u].z, acc.z);
      acc.w = fmaf(wgt, o[u].w, acc.w);
    }
  }
  s_acc[cg][dq] = acc;
  if (dq == 0) s_lsum[cg] = lsum;
  __syncthreads();
  if (tid < kCombineQuads) {
    float4 t = s_acc[0][tid];
    float L = s_lsum[0];
#pragma unroll
    for (int k = 1; k < kCombineGroups; ++k) {
      const float4 u = s_acc[k][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
      L += s_lsum[k];
    }
    const float gl = p.gate[(size_t)b * p.ld_gate + h];
    const float gate = 1.0f / (1.0f + expf(-gl));
    const float sc = gate / L;
    float4 r;
    r.x = t.x * sc;
    r.y = t.y * sc;
    r.z = t.z * sc;
    r.w = t.w * sc;
    *reinterpret_cast<float4 *>(p.out + (size_t)b * p.ld_out + (size_t)h * kHeadDim + part * kCombineDims +
                                tid * 4) = r;
  }
}

// ---------------------------------------------------------------------------
// RMSNorm with a bf16 weight: one workgroup per row.
// ---------------------------------------------------------------------------
// `out` may equal `h`: each thread reads h[c] before it writes out[c].
__global__ __launch_bounds__(kThreads) void rms_norm_kernel(const float *h, const uint16_t *w,
                                                            float *out, int hidden, float eps) {
  __shared__ float s_part[kThreads / 64];
  const float *row = h + (size_t)blockIdx.x * hidden;
  float ss = 0.f;
  for (int c = threadIdx.x; c < hidden; c += kThreads) ss = fmaf(row[c], row[c], ss);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)hidden + eps);
  float *o = out + (size_t)blockIdx.x * hidden;
  for (int c = threadIdx.x; c < hidden; c += kThreads)
    o[c] = row[c] * inv * __uint_as_float((uint32_t)w[c] << 16);
}

__global__ __launch_bounds__(kThreads) void residual_add_kernel(float *h, const float *o, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) h[i] += o[i];
}

template <int R, int NIT>
hipError_t gemv_dispatch_mb(const GemvParams &p, int waves, hipStream_t stream) {
  const int blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((gemv_bf16_kernel<R, NIT, 4>), dim3(blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int R>
hipError_t gemv_dispatch_nit(const GemvParams &p, int waves, hipStream_t stream) {
  const int nit = (p.cols + 511) / 512;
  if (nit <= 2) return gemv_dispatch_mb<R, 2>(p, waves, stream);
  if (nit <= 4) return gemv_dispatch_mb<R, 4>(p, waves, stream);
  if (nit <= 8) return gemv_dispatch_mb<R, 8>(p, waves, stream);
  return gemv_dispatch_mb<R, 16>(p, waves, stream);
}

template <int R, int NIT>
hipError_t gemv1_launch(const GemvParams &p, hipStream_t stream) {
  const int rows = p.rows0 + p.rows1;
  const int waves = (rows + R - 1) / R;
  hipLaunchKernelGGL((gemv1_bf16_kernel<R, NIT>), dim3((waves + 3) / 4), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Two rows per wave while that still gives >= 2048 waves, else one.
template <int NIT>
hipError_t gemv1_rows(const GemvParams &p, hipStream_t stream) {
  if (p.rows0 + p.rows1 >= 4096) return gemv1_launch<2, NIT>(p, stream);
  return gemv1_launch<1, NIT>(p, stream);
}

hipError_t gemv1_dispatch(const GemvParams &p, hipStream_t stream) {
  switch ((p.cols + 511) / 512) {
    case 1: return gemv1_rows<1>(p, stream);
    case 2: return gemv1_rows<2>(p, stream);
    case 3: return gemv1_rows<3>(p, stream);
    case 4: return gemv1_rows<4>(p, stream);
    case 5: return gemv1_rows<5>(p, stream);
    case 6: return gemv1_rows<6>(p, stream);
    case 7: return gemv1_rows<7>(p, stream);
    case 8: return gemv1_rows<8>(p, stream);
    case 9: case 10: return gemv1_rows<10>(p, stream);
    case 11: case 12: return gemv1_rows<12>(p, stream);
    default: return gemv1_rows<16>(p, stream);
  }
}

}  // namespace

hipError_t launch_gemv(const GemvParams &p, hipStream_t stream) {
  if (p.batch == 1) return gemv1_dispatch(p, stream);
  const int rows = p.rows0 + p.rows1;
  if (rows >= 4 * 1024) return gemv_dispatch_nit<4>(p, (rows + 3) / 4, stream);
  if (rows >= 2 * 1024) return gemv_dispatch_nit<2>(p, (rows + 1) / 2, stream);
  return gemv_dispatch_nit<1>(p, rows, stream);
}

hipError_t launch_attention(const AttnParams &p, int num_heads, hipStream_t stream) {
  const dim3 grid(p.total_chunks, p.num_kv_heads);
  hipLaunchKernelGGL(attn_partial_kernel<8>, grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(num_heads * kCombineSplit, p.nseq), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_rms_norm(const float *h, const uint16_t *w, float *out, int rows, int hidden,
                           float eps, hipStream_t stream) {
  hipLaunchKernelGGL(rms_norm_kernel, dim3(rows), dim3(kThreads), 0, stream, h, w, out, hidden, eps);
  return hipGetLastError();
}

hipError_t launch_residual_add(float *h, const float *o, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, h, o, n);
  return hipGetLastError();
}

}  // namespace gqa
