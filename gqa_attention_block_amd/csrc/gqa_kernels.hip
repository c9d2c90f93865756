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
// Attention, split-K over the window.
//
// Grid (total_chunks, Hk).  Workgroup (chunk c of sequence b, KV head g)
// owns logical positions [t0, t1) of that sequence and the 4 query heads
// 4g..4g+3 that read KV head g, so every K/V byte is read from HBM once and
// used for 4 heads.  The chunk is walked in tiles of 4*rpw rows; wave w owns
// rows [w*rpw, (w+1)*rpw) of each tile.  K and V are read with buffer loads
// (32-bit offsets; a row that must not be read gets an offset past the end
// of the buffer, which the hardware returns as zeros without touching HBM).
//
//   phase 0  RoPE table (fp64 angles), q of the 4 heads rotated and scaled
//            by scale*log2(e) into LDS.  The chunk that ends at this token
//            also rotates k, rounds k and v to fp16 once, writes both to the
//            cache slot, and keeps the rounded row in LDS: the kernel never
//            reads back what it wrote.
//   per tile:
//   scores   16 lanes per row (lane owns dims 8s..8s+7 and 128+8s..+7),
//            4 rows per load; fp16 K enters v_fma_mix directly; a DPP row
//            sum reduces.  The V loads of this tile and the K loads of the
//            next tile are issued before the barrier.
//   softmax  wave h updates head h's running (max, sum) over the tile and
//            turns the tile's scores into exp2(s - max).
//   P.V      lane owns 4 dims of a whole row (512 B per load); the running
//            accumulators are rescaled once per tile.
//   end      cross-wave sum, write (max, sum, acc[256]) per head.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_seq(const AttnParams &p, int chunk_id) {
  int s = 0;
  for (int i = 1; i < p.nseq; ++i)
    if (chunk_id >= p.seq[i].chunk_begin) s = i;
  return s;
}

// RPW: rows per wave per tile (tile = 4 * RPW rows).
template <int RPW>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(const AttnParams p) {
  constexpr int kTile = 4 * RPW;
  constexpr int kQuads = RPW / 4;
  __shared__ float s_cos[kHeadDim / 2];
  __shared__ float s_sin[kHeadDim / 2];
  __shared__ float s_q[kGroup][kHeadDim];
  __shared__ float s_kcur[kHeadDim];
  __shared__ float s_vcur[kHeadDim];
  __shared__ float4 s_p[2][kTile];             // [buffer][row] x 4 heads
  __shared__ float4 s_red[4][kGroup][kHeadDim / 4];
  __shared__ float s_m[kGroup];
  __shared__ float s_l[kGroup];
  __shared__ float s_alpha[kGroup];

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
  const int tile = kTile;
  const int rpw = RPW;
  const int wr0 = w * rpw;
  const int ntiles = (nrows + tile - 1) / tile;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(sd.k, sd.cache_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(sd.v, sd.cache_bytes);
  const unsigned head_off = (unsigned)g * kHeadDim * 2u;

  // byte offset of row `rel` (relative to t0) of this KV head, or out of range
  // (this token's own row is never read back: it is taken from LDS)
  auto row_off = [&](int rel) -> unsigned {
    if (rel >= nrows || (has_cur && rel == cur_rel)) return kOutOfRange;
    int ph = p0 + rel;
    if (ring && ph >= ring) ph -= ring;
    return (unsigned)ph * row_bytes + head_off;
  };
  const unsigned k_lane_off = (unsigned)(lane & 15) * 16u;   // lane's 16 bytes in each half row
  const unsigned v_lane_off = (unsigned)lane * 8u;           // lane's 8 bytes of a row

  const int sub = lane & 15;
  const int quad = lane >> 4;
  uint4 kr[kQuads][2];
  auto load_k = [&](int trow0) {
#pragma unroll
    for (int qi = 0; qi < kQuads; ++qi) {
      const unsigned off = row_off(trow0 + wr0 + qi * 4 + quad) + k_lane_off;
      kr[qi][0] = buf_load16(krs, off);
      kr[qi][1] = buf_load16(krs, off + kHeadDim);
    }
  };
  load_k(0);   // HBM traffic starts before the prologue

  // ---- phase 0: RoPE table, q, and this token's k/v ----
  const int rdim = p.rotary_dim;
  const int rhalf = rdim >> 1;
  if (tid < rhalf) {
    // angle = position * theta^(-2i/r), formed in fp64 so that positions in
    // the tens of thousands keep a small absolute angle error.
    const double inv = pow(p.theta, -2.0 * (double)tid / (double)rdim);
    const double ang = (double)sd.position * inv;
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[tid] = (float)cs;
    s_sin[tid] = (float)sn;
  }
  if (tid < kGroup) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
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

  // score of this token's own row for head w (kept in a register of wave w)
  float my_cur = 0.f;
  if (has_cur) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(s_q[w][lane * 4 + e], s_kcur[lane * 4 + e], s);
    my_cur = wave_sum(s);
  }

  float qreg[kGroup][16];
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qreg[i][e] = s_q[i][sub * 8 + e];
      qreg[i][8 + e] = s_q[i][kHeadDim / 2 + sub * 8 + e];
    }

  float acc[kGroup][4];
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int trow0 = it * tile;
    const int trows = min(tile, nrows - trow0);

    // scores of this tile
#pragma unroll
    for (int qi = 0; qi < kQuads; ++qi) {
      {
        const _Float16 *k0 = reinterpret_cast<const _Float16 *>(&kr[qi][0]);
        const _Float16 *k1 = reinterpret_cast<const _Float16 *>(&kr[qi][1]);
        float a[kGroup] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ka = (float)k0[e];
          const float kb = (float)k1[e];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            a[i] = fmaf(ka, qreg[i][e], a[i]);
            a[i] = fmaf(kb, qreg[i][8 + e], a[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) a[i] = row_sum16(a[i]);
        const int rt = wr0 + qi * 4 + quad;
        if (sub == 0 && rt < trows) s_p[buf][rt] = make_float4(a[0], a[1], a[2], a[3]);
      }
    }

    // V loads of this tile, K loads of the next one
    uint2 vr[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      vr[j] = buf_load8(vrs, row_off(trow0 + wr0 + j) + v_lane_off);
    }
    if (it + 1 < ntiles) load_k(trow0 + tile);
    __syncthreads();

    // running softmax statistics of head w
    {
      float *sp = reinterpret_cast<float *>(s_p[buf]);
      const int cur_t = has_cur ? cur_rel - trow0 : -1;   // this token's row in the tile, if any
      float tmax = -INFINITY;
      for (int r = lane; r < trows; r += 64) tmax = fmaxf(tmax, r == cur_t ? my_cur : sp[r * 4 + w]);
      tmax = wave_max(tmax);
      const float m_old = s_m[w];
      const float m_new = fmaxf(m_old, tmax);
      const float alpha = exp2f(m_old - m_new);
      float tsum = 0.f;
      for (int r = lane; r < trows; r += 64) {
        const float e = exp2f((r == cur_t ? my_cur : sp[r * 4 + w]) - m_new);
        sp[r * 4 + w] = e;
        tsum += e;
      }
      tsum = wave_sum(tsum);
      if (lane == 0) {
        s_m[w] = m_new;
        s_l[w] = fmaf(s_l[w], alpha, tsum);
        s_alpha[w] = alpha;
      }
    }
    __syncthreads();

    // P.V of this tile
    {
      const float al[kGroup] = {s_alpha[0], s_alpha[1], s_alpha[2], s_alpha[3]};
#pragma unroll
      for (int i = 0; i < kGroup; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] *= al[i];
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        if (wr0 + j < trows) {
          const float4 pp = s_p[buf][wr0 + j];
          const _Float16 *vh = reinterpret_cast<const _Float16 *>(&vr[j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float vv = (float)vh[e];
            acc[0][e] = fmaf(vv, pp.x, acc[0][e]);
            acc[1][e] = fmaf(vv, pp.y, acc[1][e]);
            acc[2][e] = fmaf(vv, pp.z, acc[2][e]);
            acc[3][e] = fmaf(vv, pp.w, acc[3][e]);
          }
        }
      }
      const int cur_t = has_cur ? cur_rel - trow0 : -1;
      if (cur_t >= wr0 && cur_t < wr0 + rpw && cur_t < trows) {
        const float4 pp = s_p[buf][cur_t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float vv = s_vcur[lane * 4 + e];
          acc[0][e] = fmaf(vv, pp.x, acc[0][e]);
          acc[1][e] = fmaf(vv, pp.y, acc[1][e]);
          acc[2][e] = fmaf(vv, pp.z, acc[2][e]);
          acc[3][e] = fmaf(vv, pp.w, acc[3][e]);
        }
      }
    }
  }

  // ---- sum the 4 waves, write this chunk's partials ----
#pragma unroll
  for (int i = 0; i < kGroup; ++i)
    s_red[w][i][lane] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  __syncthreads();
  {
    const float *red = reinterpret_cast<const float *>(s_red);
    const int d = tid;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      float o = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) o += red[(ww * kGroup + i) * kHeadDim + d];
      p.part_o[((size_t)cid * Hq + g * kGroup + i) * kHeadDim + d] = o;
    }
    if (tid < kGroup) {
      float *ml = p.part_ml + ((size_t)cid * Hq + g * kGroup + tid) * 2;
      ml[0] = s_m[tid];
      ml[1] = s_l[tid];
    }
  }
}

// Grid (Hq, nseq).  Thread (cg, dq): chunk group cg = tid/64 walks chunks
// cg, cg+4, ...; dq = tid%64 owns dims 4dq..4dq+3.
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const AttnParams p) {
  __shared__ float s_red[4];
  __shared__ float4 s_acc[4][kHeadDim / 4];
  __shared__ float s_lsum[4];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
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

  const int cg = tid >> 6;
  const int dq = tid & 63;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
#pragma unroll 8
  for (int c = cg; c < nchunks; c += 4) {
    const size_t base = (size_t)(f0 + c) * Hq + h;
    const float2 ml = *reinterpret_cast<const float2 *>(p.part_ml + base * 2);
    const float4 o = *reinterpret_cast<const float4 *>(p.part_o + base * kHeadDim + dq * 4);
    const float wgt = exp2f(ml.x - M);
    lsum = fmaf(wgt, ml.y, lsum);
    acc.x = fmaf(wgt, o.x, acc.x);
    acc.y = fmaf(wgt, o.y, acc.y);
    acc.z = fmaf(wgt, o.z, acc.z);
    acc.w = fmaf(wgt, o.w, acc.w);
  }
  s_acc[cg][dq] = acc;
  if (dq == 0) s_lsum[cg] = lsum;
  __syncthreads();
  if (tid < kHeadDim / 4) {
    float4 t = s_acc[0][tid];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      const float4 u = s_acc[k][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float L = (s_lsum[0] + s_lsum[1]) + (s_lsum[2] + s_lsum[3]);
    const float gl = p.gate[(size_t)b * p.ld_gate + h];
    const float gate = 1.0f / (1.0f + expf(-gl));
    const float sc = gate / L;
    float4 r;
    r.x = t.x * sc;
    r.y = t.y * sc;
    r.z = t.z * sc;
    r.w = t.w * sc;
    *reinterpret_cast<float4 *>(p.out + (size_t)b * p.ld_out + (size_t)h * kHeadDim + tid * 4) = r;
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
  if (p.batch == 1)
    hipLaunchKernelGGL((gemv_bf16_kernel<R, NIT, 1>), dim3(blocks), dim3(kThreads), 0, stream, p);
  else
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

}  // namespace

hipError_t launch_gemv(const GemvParams &p, hipStream_t stream) {
  const int rows = p.rows0 + p.rows1;
  // Enough waves to cover all CUs several times over, as few rows per wave
  // as that allows (more rows per wave = more bytes in flight per wave).
  if (rows >= 4 * 1024) return gemv_dispatch_nit<4>(p, (rows + 3) / 4, stream);
  if (rows >= 2 * 1024) return gemv_dispatch_nit<2>(p, (rows + 1) / 2, stream);
  return gemv_dispatch_nit<1>(p, rows, stream);
}

hipError_t launch_attention(const AttnParams &p, int num_heads, hipStream_t stream) {
  const dim3 grid(p.total_chunks, p.num_kv_heads);
  if (p.tile == 128)
    hipLaunchKernelGGL(attn_partial_kernel<32>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_partial_kernel<16>, grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(num_heads, p.nseq), dim3(kThreads), 0, stream, p);
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
