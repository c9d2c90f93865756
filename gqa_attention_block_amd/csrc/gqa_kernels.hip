// HIP kernels of the decode attention block for CDNA4 (gfx950), wave64.
//
// Steps and their source (docs.rs turbospark-runtime 0.3.0):
//   qkv_rope_kernel      -- the fused q_k_v_proj GEMV and the g_proj GEMV over
//                           the same input, with the split, the per-class
//                           NeoX RoPE of q and k, and the fp16 write of k and
//                           v into this token's cache slot done in the
//                           epilogue ([attn.rs] `encode_attention_block`:
//                           GEMV, split, RoPE steps; [kv_write.rs]
//                           `kv_write_target`)
//   attn_partial_kernel  -- split-K decode attention over the window/ring
//                           ([attn.rs] window and attention steps;
//                           [kv_write.rs] `encode_attention_any`)
//   attn_combine_kernel  -- merge of the split-K partials and the headwise
//                           sigmoid gate ([attn.rs] gate step, before o_proj)
//   block_fused_kernel   -- the whole block for one sequence in one
//                           persistent launch (every step above, then the
//                           merge with the gate and the o_proj GEMV: [attn.rs]
//                           gate step and last GEMV), or its attention and
//                           merge alone
//   gemv_bf16_kernel     -- the o_proj GEMV below the MFMA batch
//                           ([attn.rs] last GEMV)
//   proj_mfma_kernel     -- both projections on the matrix cores for batches
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

// MFMA operand and LDS pointer types
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

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

// v_permlane16_swap / v_permlane32_swap (VALU, no LDS traffic): every lane
// gets, in .x and .y, the values of its lane in the two rows of its row pair
// (16-lane rows 0/1 and 2/3), resp. of its lane in the two 32-lane halves.
__device__ __forceinline__ float2 pair16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 pair32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum / max over lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float sum_across_rows(float v) {
  float2 a = pair16(v);
  a = pair32(a.x + a.y);
  return a.x + a.y;
}
__device__ __forceinline__ float max_across_rows(float v) {
  float2 a = pair16(v);
  a = pair32(fmaxf(a.x, a.y));
  return fmaxf(a.x, a.y);
}

__device__ __forceinline__ float wave_sum(float v) { return sum_across_rows(row_sum16(v)); }

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return max_across_rows(v);
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

// Cache policy of the loads that stream bytes read once per call: the KV
// tiles of the attention and the projection weights.  2 = nt (non-temporal):
// the lines are not kept in the caches for reuse, which lets the memory
// system sustain a higher read rate on long streams.
constexpr int kKPolicy = 2;
constexpr int kVPolicy = 2;
constexpr int kWeightPolicy = 2;

template <int POLICY>
__device__ __forceinline__ uint4 buf_load16_p(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (to nearest even), packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 8 bf16 weights against x split into bf16 high and low parts (same columns),
// accumulated into a: per weight pair, the high product pair then the low one.
__device__ __forceinline__ float dot8_bf16_split(uint4 q, uint4 xh, uint4 xl, float a) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w}, h[4] = {xh.x, xh.y, xh.z, xh.w}, l[4] = {xl.x, xl.y, xl.z, xl.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]), __builtin_bit_cast(bf16x2_t, h[k]), a,
                                        false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]), __builtin_bit_cast(bf16x2_t, l[k]), a,
                                        false);
  }
  return a;
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
// Rows of x staged in LDS for the VALU projections.
//
// Lane l of a wave reads columns (it*64 + l)*8 .. +8 of its weight rows, so it
// needs x at the same columns in every wave of the workgroup; loaded per wave,
// x (fp32: twice the bytes of a bf16 row) would pass through the CU's L1 once
// per wave.  Here the workgroup loads each x row once: thread t holds float4s
// t, t + 256, ... (columns 4f .. 4f+3) and writes them to LDS as two arrays,
// s[0][j] = columns 8j .. 8j+3 and s[1][j] = 8j+4 .. 8j+7, so a wave's 16-byte
// reads of either are contiguous.  The first rows' loads are issued before
// the weight loads, so the wait for them does not include the weights.  NORM
// also multiplies by a bf16 weight and keeps the thread's sum of squares.
// ---------------------------------------------------------------------------
template <int NIT>
struct StagedX {
  static constexpr int kGroups = NIT * 64;                           // 8-column groups read
  static constexpr int kPer = (2 * kGroups + kThreads - 1) / kThreads;  // float4s per thread
  static constexpr int kSlots = kPer * kThreads / 2;                 // >= kGroups: every store in bounds
  float4 v[kPer];
  uint2 wn[kPer];

  // x row at byte `base` of rx.  No load or store is conditional (a
  // conditional store lets the compiler sink its load behind the weight
  // loads): float4s past the row read as zeros from the resource bound and
  // land in the slots past kGroups, which are never read.
  // (XPOL: the cache policy of the x loads)
  template <bool NORM, int XPOL = 0>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rx, unsigned base, __amdgpu_buffer_rsrc_t rn) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const unsigned f = threadIdx.x + k * kThreads;
      v[k] = __builtin_bit_cast(float4, buf_load16_p<XPOL>(rx, base + f * 16u));
      if constexpr (NORM) wn[k] = buf_load8(rn, f * 8u);
    }
  }
  // The projections' form: slot g of s[0] holds the bf16 high parts of
  // columns 8g .. 8g+7 and slot g of s[1] their bf16 low parts (x - high),
  // so that a dot product takes two v_dot2 per pair of bf16 weights, with
  // x to 16 significant bits.  Returns this thread's sum of squares of x
  // (NORM, in fp32 before the split) or 0.
  template <bool NORM>
  __device__ __forceinline__ float store_split(float4 (*s)[kSlots]) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const unsigned f = threadIdx.x + k * kThreads;
      float4 x = v[k];
      if constexpr (NORM) {
        ss = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, fmaf(x.w, x.w, ss))));
        x = make_float4(x.x * bf16_lo(wn[k].x), x.y * bf16_hi(wn[k].x), x.z * bf16_lo(wn[k].y),
                        x.w * bf16_hi(wn[k].y));
      }
      const uint2 hi = make_uint2(pack_bf16(x.x, x.y), pack_bf16(x.z, x.w));
      const uint2 lo = make_uint2(pack_bf16(x.x - bf16_lo(hi.x), x.y - bf16_hi(hi.x)),
                                  pack_bf16(x.z - bf16_lo(hi.y), x.w - bf16_hi(hi.y)));
      reinterpret_cast<uint2 *>(&s[0][f >> 1])[f & 1] = hi;
      reinterpret_cast<uint2 *>(&s[1][f >> 1])[f & 1] = lo;
    }
    return ss;
  }
  // writes LDS (fp32 x, as the batched GEMVs read it); returns this
  // thread's sum of squares of x (NORM) or 0
  template <bool NORM>
  __device__ __forceinline__ float store(float4 (*s)[kSlots]) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const unsigned f = threadIdx.x + k * kThreads;
      float4 x = v[k];
      if constexpr (NORM) {
        ss = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, fmaf(x.w, x.w, ss))));
        x = make_float4(x.x * bf16_lo(wn[k].x), x.y * bf16_hi(wn[k].x), x.z * bf16_lo(wn[k].y),
                        x.w * bf16_hi(wn[k].y));
      }
      s[f & 1][f >> 1] = x;
    }
    return ss;
  }
};

// ---------------------------------------------------------------------------
// GEMV: y[b][r] = sum_c W[r][c] x[b][c], bf16 W, fp32 x/y/accumulation, for
// the batches below the MFMA path (and the last rows of a batched o_proj).
//
// One wave owns R consecutive rows.  Lane l reads columns
// [(it*64 + l)*8, +8) for it < NIT (NIT = ceil(cols / 512)), so each 16-byte
// load instruction covers 1 KiB of one row; all R*NIT loads are issued before
// the first FMA and the weights stay in registers while the batch is walked
// RB rows at a time, x staged in LDS (StagedX), the next rows' x loads in
// flight during each pass.  ONE (batch 1) is the same without the loop, which
// keeps the x loads ahead of the weight loads in the compiled order.  Waves
// past the last row still take part in the barriers; their loads are out of
// range.  With accumulate the kernel adds into y (the layer's residual add).
// ---------------------------------------------------------------------------
template <int R, int NIT, int RB, bool ONE>
__global__ __launch_bounds__(kThreads) void gemv_bf16_kernel(const GemvParams p) {
  __shared__ float4 s_x[RB][2][StagedX<NIT>::kSlots];
  const int lane = threadIdx.x & 63;
  // wave index kept scalar: row-dependent choices (which weight buffer) stay uniform
  const int wave = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int total = p.rows0 + p.rows1;
  const int row0 = wave * R;
  const unsigned row_bytes = (unsigned)p.cols * 2u;
  const __amdgpu_buffer_rsrc_t r0 = make_rsrc(p.w0, (unsigned)p.rows0 * row_bytes);
  const __amdgpu_buffer_rsrc_t r1 = make_rsrc(p.w1, (unsigned)p.rows1 * row_bytes);
  // x row b, bounded at cols (a zero-size resource past the batch)
  auto xrow = [&](int b) { return make_rsrc(p.x + (size_t)b * p.ldx, b < p.batch ? (unsigned)p.cols * 4u : 0u); };

  StagedX<NIT> xs[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) xs[r].template issue<false>(xrow(r), 0u, xrow(r));
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
      w[r][it] = first ? buf_load16_p<kWeightPolicy>(r0, off) : buf_load16_p<kWeightPolicy>(r1, off);
    }
  }
  // the R rows' dot products with staged x row m (batch row b)
  auto emit = [&](int m, int b) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int it = 0; it < NIT; ++it)
        a = dot8_bf16_split(w[r][it], __builtin_bit_cast(uint4, s_x[m][0][it * 64 + lane]),
                            __builtin_bit_cast(uint4, s_x[m][1][it * 64 + lane]), a);
      const float s = wave_sum(a);
      const int row = row0 + r;
      if (lane == r && row < total && b < p.batch) {
        float *y = row < p.rows0 ? p.y0 + (size_t)b * p.ldy0 + row : p.y1 + (size_t)b * p.ldy1 + (row - p.rows0);
        *y = p.accumulate ? *y + s : s;
      }
    }
  };
  if constexpr (ONE) {
    xs[0].template store_split<false>(s_x[0]);
    __syncthreads();
    emit(0, 0);
  } else {
    for (int b0 = 0; b0 < p.batch; b0 += RB) {
#pragma unroll
      for (int m = 0; m < RB; ++m) {
        xs[m].template store_split<false>(s_x[m]);
        // next rows: unconditional (past the batch the resource is empty, no
        // traffic), so the compiler's waits stay exact
        xs[m].template issue<false>(xrow(b0 + RB + m), 0u, xrow(0));
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < RB; ++m) emit(m, b0 + m);
      if (b0 + RB < p.batch) __syncthreads();   // s_x is rewritten for the next rows
    }
  }
}

// ---------------------------------------------------------------------------
// Fused q_k_v_proj + g_proj GEMV with the split, RoPE and KV-slot write in the
// epilogue.
//
// Wave P computes TWO output rows that RoPE pairs: inside a q or k head with
// rotary width r, pair i < r/2 is rows (i, i + r/2), which turn together by
// the angle position * theta^(-2i/r); pairs i >= r/2, all v pairs and all
// gate pairs are rows (2i, 2i+1), left as they are.  Sections in pair order:
// q heads (128 pairs each), k heads, v heads, then Hq/2 gate pairs.  The dot
// products run like gemv_bf16_kernel (16-byte loads, all issued up front, x
// staged in LDS); then each batch row's angle is formed in fp64, the pair is
// rotated in fp32 and written: q -> q_out (fp32), k and v -> fp16, rounded
// once, straight into the cache slot of this position; gate logits ->
// gate_out.
// ---------------------------------------------------------------------------
// NeoX rotation of the pair (x_i, x_{i + r/2}) by angle position * theta^(-2i/r).
// The angle is formed and reduced mod 2*pi in fp64 (an fp32 angle at position
// 32767 would be off by ~4e-3 rad); the reduced angle is in [-pi, pi], where
// fp32 sin/cos are accurate.
__device__ __forceinline__ void rope_sincos(int position, int i, int rotary_dim, double log2_theta, float &sn,
                                            float &cs) {
  const double inv = exp2(-(2.0 * (double)i / (double)rotary_dim) * log2_theta);
  const double ang = (double)position * inv;
  const double k = rint(ang * 0.15915494309189535);          // 1 / (2 pi)
  double red = fma(-k, 6.283185307179586, ang);               // 2 pi, high part
  red = fma(-k, 2.4492935982947064e-16, red);                 // 2 pi, low part
  sincosf((float)red, &sn, &cs);
}

__device__ __forceinline__ void rope_apply(float sn, float cs, float &ya, float &yb) {
  const float ra = ya * cs - yb * sn;
  const float rb = yb * cs + ya * sn;
  ya = ra;
  yb = rb;
}

__device__ __forceinline__ void rope_rotate(int position, int i, int rotary_dim, double log2_theta, float &ya,
                                            float &yb) {
  float sn, cs;
  rope_sincos(position, i, rotary_dim, log2_theta, sn, cs);
  rope_apply(sn, cs, ya, yb);
}

// One RoPE pair of output rows: section sec (0 q, 1 k, 2 v, 3 gate logits),
// head, pair index pi; rows dA, dB inside the head (rotated pairs (i, i+r/2),
// the others (2i, 2i+1)) and the first weight row of the head.
struct PairRows {
  int sec, head, pi, dA, dB, base_row;
  bool rotate;
};

__device__ __forceinline__ PairRows pair_rows(int sec, int head, int pi, int Hq, int Hk, int rotary_dim) {
  PairRows r;
  r.sec = sec;
  r.head = head;
  r.pi = pi;
  const int rhalf = rotary_dim >> 1;
  r.rotate = sec <= 1 && pi < rhalf;
  r.dA = r.rotate ? pi : 2 * pi;
  r.dB = r.rotate ? pi + rhalf : 2 * pi + 1;
  r.base_row = sec == 0 ? head * kHeadDim
             : sec == 1 ? (Hq + head) * kHeadDim
             : sec == 2 ? (Hq + Hk + head) * kHeadDim : 0;
  return r;
}

// Stores whose values other workgroups of the same launch read: written
// through to the device's point of coherence (the sc1 scope bit), so a
// reader on another XCD that loads them coherently sees them once the store
// has completed.  COHERENT = false: plain stores (a later launch reads them).
template <bool COHERENT>
__device__ __forceinline__ void store_f32(float *p, float v) {
  if constexpr (COHERENT)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ void store_f16(_Float16 *p, float v) {
  const _Float16 h = (_Float16)v;
  if constexpr (COHERENT)
    __hip_atomic_store(reinterpret_cast<uint16_t *>(p), __builtin_bit_cast(uint16_t, h), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = h;
}
constexpr int kCoherent = 16;   // buffer-instruction cache policy: sc1, device-coherent

// Epilogue of one output pair for one sequence: RoPE, then q -> q_out
// (fp32, [Hq][D]), k and v -> fp16 into the cache slot of this position,
// gate logits -> gate_out ([Hq]).
template <bool COHERENT = false>
__device__ __forceinline__ void pair_store(float *q_out, float *gate_out, const SeqDesc &sd, int Hk, const PairRows &r,
                                           float sn, float cs, float ya, float yb) {
  if (r.rotate) rope_apply(sn, cs, ya, yb);
  if (r.sec == 0) {
    float *q = q_out + (size_t)r.head * kHeadDim;
    store_f32<COHERENT>(q + r.dA, ya);
    store_f32<COHERENT>(q + r.dB, yb);
  } else if (r.sec == 3) {
    store_f32<COHERENT>(gate_out + r.dA, ya);
    store_f32<COHERENT>(gate_out + r.dB, yb);
  } else {
    _Float16 *dst = (r.sec == 1 ? sd.k : sd.v) + (size_t)sd.slot * Hk * kHeadDim + (size_t)r.head * kHeadDim;
    store_f16<COHERENT>(dst + r.dA, ya);
    store_f16<COHERENT>(dst + r.dB, yb);
  }
}

// The pair's two dot products with the staged x (s0: columns 8j .. 8j+3, s1:
// 8j+4 .. 8j+7), summed over the wave; NORM scales them by inv_rms(h), the
// workgroup's four wave sums of squares added in a fixed order.
template <int NIT, bool NORM>
__device__ __forceinline__ void pair_dots(const uint4 (&wa)[NIT], const uint4 (&wb)[NIT], const float4 *s0,
                                          const float4 *s1, const float *ss, int hidden, float eps, int lane,
                                          float &ya, float &yb) {
  float a = 0.f, c = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const uint4 xh = __builtin_bit_cast(uint4, s0[it * 64 + lane]);
    const uint4 xl = __builtin_bit_cast(uint4, s1[it * 64 + lane]);
    a = dot8_bf16_split(wa[it], xh, xl, a);
    c = dot8_bf16_split(wb[it], xh, xl, c);
  }
  ya = wave_sum(a);
  yb = wave_sum(c);
  if constexpr (NORM) {
    const float inv = rsqrtf((ss[0] + ss[1] + ss[2] + ss[3]) / (float)hidden + eps);
    ya *= inv;
    yb *= inv;
  }
}

// pair_dots with x already in registers (x0[it], x1[it]: the staged slots
// it * 64 + lane of s0 and s1): the same arithmetic in the same order.
template <int NIT, bool NORM>
__device__ __forceinline__ void pair_dots_x(const uint4 (&wa)[NIT], const uint4 (&wb)[NIT], const float4 (&x0)[NIT],
                                            const float4 (&x1)[NIT], const float *ss, int hidden, float eps,
                                            float &ya, float &yb) {
  float a = 0.f, c = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const uint4 xh = __builtin_bit_cast(uint4, x0[it]);
    const uint4 xl = __builtin_bit_cast(uint4, x1[it]);
    a = dot8_bf16_split(wa[it], xh, xl, a);
    c = dot8_bf16_split(wb[it], xh, xl, c);
  }
  ya = wave_sum(a);
  yb = wave_sum(c);
  if constexpr (NORM) {
    const float inv = rsqrtf((ss[0] + ss[1] + ss[2] + ss[3]) / (float)hidden + eps);
    ya *= inv;
    yb *= inv;
  }
}

// NORM: x is the raw residual stream h and each projection is
// inv_rms(h) * W (h * w_norm), the sum of squares taken over the same loads
// and summed over the workgroup in LDS.  The batch is walked RB rows at a
// time with x staged in LDS, as in gemv_bf16_kernel; waves past the last pair
// take part in the barriers with out-of-range loads and no writes.
template <int NIT, int RB, bool NORM, bool ONE>
__global__ __launch_bounds__(kThreads) void qkv_rope_kernel(const QkvParams p) {
  __shared__ float4 s_x[RB][2][StagedX<NIT>::kSlots];
  __shared__ float s_ss[RB][kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int P = blockIdx.x * (kThreads / 64) + wv;   // scalar
  const int Hq = p.num_heads, Hk = p.num_kv_heads;
  constexpr int kPairs = kHeadDim / 2;
  const int nq = Hq * kPairs, nk = Hk * kPairs, nv = Hk * kPairs;
  const bool active = P < nq + nk + nv + Hq / 2;
  int sec, head, pi;
  if (P < nq) {
    sec = 0; head = P / kPairs; pi = P % kPairs;
  } else if (P < nq + nk) {
    sec = 1; head = (P - nq) / kPairs; pi = (P - nq) % kPairs;
  } else if (P < nq + nk + nv) {
    sec = 2; head = (P - nq - nk) / kPairs; pi = (P - nq - nk) % kPairs;
  } else {
    sec = 3; head = 0; pi = P - nq - nk - nv;
  }
  const PairRows pr = pair_rows(sec, head, pi, Hq, Hk, p.rotary_dim);
  const bool rotate = pr.rotate;
  const int dA = pr.dA, dB = pr.dB, base_row = pr.base_row;
  const unsigned row_bytes = (unsigned)p.hidden * 2u;
  const int qkv_rows = (Hq + 2 * Hk) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rw = sec < 3 ? make_rsrc(p.w_qkv, (unsigned)qkv_rows * row_bytes)
                                            : make_rsrc(p.w_g, (unsigned)Hq * row_bytes);
  // x row b, bounded at hidden (ldx may be larger; a zero-size resource past the batch)
  auto xrow = [&](int b) {
    return make_rsrc(p.x + (size_t)b * p.ldx, b < p.batch ? (unsigned)p.hidden * 4u : 0u);
  };
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(NORM ? p.w_norm : nullptr, NORM ? (unsigned)p.hidden * 2u : 0u);

  StagedX<NIT> xs[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) xs[r].template issue<NORM>(xrow(r), 0u, rn);
  uint4 wa[NIT], wb[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int col = (it * 64 + lane) * 8;
    const bool ok = active && col < p.hidden;
    wa[it] = buf_load16_p<kWeightPolicy>(rw, ok ? (unsigned)(base_row + dA) * row_bytes + (unsigned)col * 2u : kOutOfRange);
    wb[it] = buf_load16_p<kWeightPolicy>(rw, ok ? (unsigned)(base_row + dB) * row_bytes + (unsigned)col * 2u : kOutOfRange);
  }

  // the rotation of batch row b does not depend on the loads: formed while
  // they are in flight
  auto angle = [&](int b, float &sn, float &cs) {
    sn = 0.f;
    cs = 1.f;
    if (rotate && b < p.batch) rope_sincos(p.seq[b].position, pi, p.rotary_dim, p.log2_theta, sn, cs);
  };
  auto stage = [&](int m) {
    const float ss = wave_sum(xs[m].template store_split<NORM>(s_x[m]));
    if (NORM && lane == 0) s_ss[m][wv] = ss;
  };
  // the pair's dot products with staged x row m, then the epilogue for batch row b
  auto emit = [&](int m, int b, float sn, float cs) {
    float ya, yb;
    pair_dots<NIT, NORM>(wa, wb, s_x[m][0], s_x[m][1], s_ss[m], p.hidden, p.rms_eps, lane, ya, yb);
    if (lane == 0 && active && b < p.batch)
      pair_store(p.q_out + (size_t)b * p.ld_q, p.gate_out + (size_t)b * p.ld_gate, p.seq[b], Hk, pr, sn, cs, ya, yb);
  };
  if constexpr (ONE) {
    float sn, cs;
    angle(0, sn, cs);
    stage(0);
    __syncthreads();
    emit(0, 0, sn, cs);
  } else {
    for (int b0 = 0; b0 < p.batch; b0 += RB) {
      float sn[RB], cs[RB];
#pragma unroll
      for (int m = 0; m < RB; ++m) angle(b0 + m, sn[m], cs[m]);
#pragma unroll
      for (int m = 0; m < RB; ++m) {
        stage(m);
        xs[m].template issue<NORM>(xrow(b0 + RB + m), 0u, rn);   // next rows: unconditional, as in the GEMV
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < RB; ++m) emit(m, b0 + m, sn[m], cs[m]);
      if (b0 + RB < p.batch) __syncthreads();   // s_x and s_ss are rewritten for the next rows
    }
  }
}

// ---------------------------------------------------------------------------
// Batched projections on the matrix cores.
//
// At batch B >= kMfmaMinBatch a projection y[b][r] = sum_c W[r][c] x[b][c] is
// a [rows x C] x [C x B] product with enough columns for MFMA: the fp32 VALU
// GEMV needs one FMA per weight and batch row, and at B = 32 that is the bound,
// not HBM.  v_mfma_f32_16x16x32_bf16 takes W (bf16) as the A operand straight
// from HBM (lane (G, n): row n, 8 columns = 16 B) and x (fp32) split into bf16
// high and low parts, x = hi + lo up to 2^-16 |x|, as two B operands, so the
// product keeps fp32 accuracy.
//
// A workgroup owns a unit of two 16-row tiles for up to MB 16-row batch tiles; its
// kProjSplit waves split the columns and add their partial sums in LDS in a
// fixed order (the result does not depend on timing).  Every workgroup reads
// x for all columns of its batch rows; o_proj takes one 16-row batch tile per
// workgroup, which spreads that traffic over twice the workgroups (2 x 80 at
// H = 2560 and batch 32).  For q_k_v_proj the two
// tiles of a unit are RoPE partners inside a head (rows i and i + r/2), so the
// epilogue rotates, splits and writes q, k, v and the gate logits as the fused
// batch-1 kernel does.
// ---------------------------------------------------------------------------
constexpr int kProjSplit = 8;                 // waves (column splits) per workgroup
constexpr int kProjThreads = 64 * kProjSplit;

// Which two 16-row tiles a unit covers.  Plain: tiles 2u, 2u+1 of the
// concatenated rows.  q_k_v_proj + g_proj: per head (q, k, v sections) 8
// units; with rt = rotary_dim / 16 rotated tiles, unit j < rt/2 pairs tiles
// (j, j + rt/2), the others pair the remaining tiles in order; the last unit
// is the gate rows (W_g).
struct ProjUnit {
  int sec;        // 0 q, 1 k, 2 v, 3 gate (qkv mode); 0 plain
  int head;
  int ta, tb;     // tile index inside the head (qkv) or global tile (plain)
  bool rotate;
};

__device__ __forceinline__ ProjUnit qkv_unit(const QkvParams &p, int u) {
  ProjUnit U{};
  const int nheads = p.num_heads + 2 * p.num_kv_heads;
  if (u >= 8 * nheads) {
    U.sec = 3; U.head = 0; U.ta = 0; U.tb = 1; U.rotate = false;
    return U;
  }
  const int h = u >> 3, uh = u & 7;
  U.sec = h < p.num_heads ? 0 : (h < p.num_heads + p.num_kv_heads ? 1 : 2);
  U.head = U.sec == 0 ? h : (U.sec == 1 ? h - p.num_heads : h - p.num_heads - p.num_kv_heads);
  const int rt = U.sec == 2 ? 0 : p.rotary_dim / 16;
  if (uh < rt / 2) {
    U.ta = uh; U.tb = uh + rt / 2; U.rotate = true;
  } else {
    U.ta = rt + 2 * (uh - rt / 2); U.tb = U.ta + 1; U.rotate = false;
  }
  return U;
}

__device__ __forceinline__ void proj_to_bf16(const float4 x0, const float4 x1, bf16x8_t &hi, bf16x8_t &lo) {
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = (__bf16)v[i];
    lo[i] = (__bf16)(v[i] - (float)hi[i]);
  }
}

// 32-row units of a launch: per head 8 (q, k, v sections) plus the gate rows;
// plain: w0's rows, then w1's
__host__ __device__ __forceinline__ int proj_units(const QkvParams &p) {
  return 8 * (p.num_heads + 2 * p.num_kv_heads) + 1;
}
__host__ __device__ __forceinline__ int proj_units(const GemvParams &p) {
  return (p.rows0 + 31) / 32 + (p.rows1 + 31) / 32;
}

__device__ __forceinline__ const uint16_t *norm_weights(const QkvParams &p) { return p.w_norm; }
__device__ __forceinline__ const uint16_t *norm_weights(const GemvParams &) { return nullptr; }

// MODE 0: plain product into y0 / y1 (GemvParams); MODE 1: q_k_v_proj +
// g_proj with the RoPE / KV-slot epilogue (QkvParams).  MB batch tiles of 16.
// NORM (MODE 1): x is the raw residual stream h; the product takes h * w_norm
// and the epilogue scales by inv_rms(h), whose sum of squares the waves
// gather over their columns and add in LDS.
template <int MODE, int MB, bool NORM, typename Params>
__global__ __launch_bounds__(kProjThreads) void proj_mfma_kernel(const Params p) {
  __shared__ float4 s_red[kProjSplit][2][16 * MB][4];   // [wave][tile][batch][rows 4k..4k+3] per 16-row tile
  __shared__ float s_ss[kProjSplit][16 * MB];           // NORM: [wave][batch] partial sums of squares
  __shared__ uint4 s_stage[kProjSplit * (32 * 8 + MB * 16 * 16)];   // per wave: one staged k-step pair

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, n = lane & 15;
  // workgroup -> (unit u, batch tile bt): the batch tiles of a unit sit 8
  // workgroups apart, i.e. on the same XCD, whose L2 then serves the second
  // read of the unit's weights
  const int nbt = (p.batch + 16 * MB - 1) / (16 * MB);
  const int grp = blockIdx.x / (8 * nbt), off = blockIdx.x - grp * (8 * nbt);
  const int u = grp * 8 + (off & 7);
  const int b0 = (off >> 3) * 16 * MB;   // first batch row of this workgroup
  if (u >= proj_units(p)) return;

  // rows of the two tiles, their matrix and its row count
  const uint16_t *wmat;
  int wrows, rowA, rowB, cols, batch;
  ProjUnit U{};
  const float *x;
  long ldx;
  bool first = true;   // plain mode: the unit's rows are in w0 (else w1)
  if constexpr (MODE == 0) {
    // plain: units over w0's rows, then units over w1's rows
    const int u0 = (p.rows0 + 31) / 32;
    first = u < u0;
    if (first) {
      wmat = p.w0; wrows = p.rows0; rowA = u * 32;
    } else {
      wmat = p.w1; wrows = p.rows1; rowA = (u - u0) * 32;
    }
    rowB = rowA + 16;
    cols = p.cols; batch = min(16 * MB, p.batch - b0); x = p.x + (size_t)b0 * p.ldx; ldx = p.ldx;
  } else {
    U = qkv_unit(p, u);
    if (U.sec == 3) {
      wmat = p.w_g; wrows = p.num_heads; rowA = 0; rowB = 16;
    } else {
      const int hrow = (U.sec == 0 ? U.head : U.sec == 1 ? p.num_heads + U.head
                                                         : p.num_heads + p.num_kv_heads + U.head) * kHeadDim;
      wmat = p.w_qkv; wrows = (p.num_heads + 2 * p.num_kv_heads) * kHeadDim;
      rowA = hrow + U.ta * 16; rowB = hrow + U.tb * 16;
    }
    cols = p.hidden; batch = min(16 * MB, p.batch - b0); x = p.x + (size_t)b0 * p.ldx; ldx = p.ldx;
  }
  const unsigned row_bytes = (unsigned)cols * 2u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wmat, (unsigned)wrows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (unsigned)((size_t)batch * ldx * 4u));
  // this wave's k-steps: [s0, s0 + spw), in pairs (64 columns); spw a
  // multiple of 4 so the pairs come in twos
  const int nsteps = (cols + 31) / 32;
  int spw = (nsteps + kProjSplit - 1) / kProjSplit;
  spw = (spw + 3) / 4 * 4;
  const int s0 = w * spw;
  const int npairs = spw / 2;

  // Coalesced loads of one pair of k-steps.  W: 4 loads of 8 rows x 128 B
  // (whole cache lines) of the unit's 32 rows, lane l taking row 8i + l/8,
  // 16-byte chunk l%8.  x: per batch tile 4 loads of 4 rows x 256 B, lane l
  // taking row 4i + l/16, chunk l%16.  The MFMA operand layout (16 rows x
  // 64 B per fragment) read straight from memory touches twice the lines per
  // byte; here the fragments come from LDS instead.
  const int lwr = lane >> 3, lwc = lane & 7;
  const int lxr = lane >> 4, lxc = lane & 15;
  unsigned woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + lwr;                       // row of the unit: tile A, then tile B
    const int grow = r < 16 ? rowA + r : rowB + (r - 16);
    woff[i] = grow < wrows ? (unsigned)grow * row_bytes + (unsigned)lwc * 16u : kOutOfRange;
  }
  unsigned xoff[MB][4];
#pragma unroll
  for (int bt = 0; bt < MB; ++bt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = bt * 16 + 4 * i + lxr;
      xoff[bt][i] = r < batch ? (unsigned)((size_t)r * ldx * 4u) + (unsigned)lxc * 16u : kOutOfRange;
    }
  // NORM: the w_norm resource (a zero-size resource otherwise, never read)
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(NORM ? (const void *)norm_weights(p) : nullptr,
                                              NORM ? (unsigned)cols * 2u : 0u);
  struct Pair {
    uint4 w[4];
    float4 x[MB][4];
    uint4 wn[NORM ? 2 : 1];   // w_norm at lane (G, n)'s 8 columns of each k-step
  };
  auto load_pair = [&](Pair &P, int pr) {
    const int c0 = (s0 + 2 * pr) * 32;             // first column of the pair
#pragma unroll
    for (int i = 0; i < 4; ++i)
      P.w[i] = buf_load16_p<kWeightPolicy>(rw, woff[i] != kOutOfRange && c0 + lwc * 8 < cols ? woff[i] + (unsigned)c0 * 2u
                                                                             : kOutOfRange);
#pragma unroll
    for (int bt = 0; bt < MB; ++bt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        P.x[bt][i] = __builtin_bit_cast(
            float4, buf_load16(rx, xoff[bt][i] != kOutOfRange && c0 + lxc * 4 < cols
                                       ? xoff[bt][i] + (unsigned)c0 * 4u : kOutOfRange));
    if constexpr (NORM)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int col = c0 + k * 32 + G * 8;
        P.wn[k] = buf_load16(rn, col < cols ? (unsigned)col * 2u : kOutOfRange);
      }
  };
  // This wave's LDS: W as 32 rows x 8 chunks, x as MB x 16 rows x 16 chunks
  // (16 B each), chunk j of row r stored at slot j ^ (r & 7) of its row, so
  // that the 8 lanes of a fragment read phase (8 rows, one chunk) and of a
  // store phase (one row, 8 chunks) fall on distinct banks.
  uint4 *const sw = s_stage + w * (32 * 8 + MB * 16 * 16);
  float4 *const sx = reinterpret_cast<float4 *>(sw + 32 * 8);
  auto stage_pair = [&](const Pair &P) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + lwr;
      sw[r * 8 + (lwc ^ (r & 7))] = P.w[i];
    }
#pragma unroll
    for (int bt = 0; bt < MB; ++bt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + lxr;
        sx[(bt * 16 + r) * 16 + (lxc ^ (r & 7))] = P.x[bt][i];
      }
  };

  float ssp[MB];   // NORM: this lane's sum of squares per batch tile
#pragma unroll
  for (int bt = 0; bt < MB; ++bt) ssp[bt] = 0.f;
  floatx4_t accA[MB], accB[MB];
#pragma unroll
  for (int bt = 0; bt < MB; ++bt) {
    accA[bt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
    accB[bt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  }
  // k-step s of the staged pair: lane (G, n) takes row n (tile A) and row
  // 16 + n (tile B), columns 8G .. 8G+7 of the step, and batch row n's x at
  // the same columns (chunks 8s + 2G and 8s + 2G + 1 of its 64)
  auto compute_pair = [&](const Pair &P) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int jw = (4 * s + G) ^ (n & 7);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, sw[n * 8 + jw]);
      const bf16x8_t b2 = __builtin_bit_cast(bf16x8_t, sw[(16 + n) * 8 + jw]);
#pragma unroll
      for (int bt = 0; bt < MB; ++bt) {
        float4 x0 = sx[(bt * 16 + n) * 16 + ((8 * s + 2 * G) ^ (n & 7))];
        float4 x1 = sx[(bt * 16 + n) * 16 + ((8 * s + 2 * G + 1) ^ (n & 7))];
        if constexpr (NORM) {
          float q = ssp[bt];
          q = fmaf(x0.x, x0.x, fmaf(x0.y, x0.y, fmaf(x0.z, x0.z, fmaf(x0.w, x0.w, q))));
          q = fmaf(x1.x, x1.x, fmaf(x1.y, x1.y, fmaf(x1.z, x1.z, fmaf(x1.w, x1.w, q))));
          ssp[bt] = q;
          const uint4 wv = P.wn[s];
          x0 = make_float4(x0.x * bf16_lo(wv.x), x0.y * bf16_hi(wv.x), x0.z * bf16_lo(wv.y), x0.w * bf16_hi(wv.y));
          x1 = make_float4(x1.x * bf16_lo(wv.z), x1.y * bf16_hi(wv.z), x1.z * bf16_lo(wv.w), x1.w * bf16_hi(wv.w));
        }
        bf16x8_t hi, lo;
        proj_to_bf16(x0, x1, hi, lo);
        accA[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, accA[bt], 0, 0, 0);
        accA[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, accA[bt], 0, 0, 0);
        accB[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b2, hi, accB[bt], 0, 0, 0);
        accB[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b2, lo, accB[bt], 0, 0, 0);
      }
    }
  };
  // two pairs in flight; no load is conditional (columns past the end are
  // out of range: zeros without HBM traffic), so the waits stay exact.  A
  // wave's LDS stores and reads are issued in order, so staging a pair over
  // the previous one needs no barrier.
  Pair PA, PB;
  load_pair(PA, 0);
  load_pair(PB, 1);
  for (int pr = 0; pr + 2 < npairs; pr += 2) {
    stage_pair(PA);
    compute_pair(PA);
    load_pair(PA, pr + 2);
    stage_pair(PB);
    compute_pair(PB);
    load_pair(PB, pr + 3);
  }
  stage_pair(PA);
  compute_pair(PA);
  stage_pair(PB);
  compute_pair(PB);

  // partial sums: lane (G, n) holds rows 4G..4G+3 of batch column n
#pragma unroll
  for (int bt = 0; bt < MB; ++bt) {
    s_red[w][0][bt * 16 + n][G] = make_float4(accA[bt][0], accA[bt][1], accA[bt][2], accA[bt][3]);
    s_red[w][1][bt * 16 + n][G] = make_float4(accB[bt][0], accB[bt][1], accB[bt][2], accB[bt][3]);
  }
  if constexpr (NORM) {
#pragma unroll
    for (int bt = 0; bt < MB; ++bt) {
      const float q = sum_across_rows(ssp[bt]);   // the 4 lane groups of batch column n
      if (G == 0) s_ss[w][bt * 16 + n] = q;
    }
  }
  __syncthreads();
  // thread t: batch row b = t / 16 of this workgroup (b0 + b overall), row
  // xr = t % 16 of both tiles
  const int t = threadIdx.x;
  const int b = t >> 4, xr = t & 15;
  if (b >= MB * 16 || b >= batch) return;
  const int bg = b0 + b;
  float ya = 0.f, yb = 0.f;
#pragma unroll
  for (int ww = 0; ww < kProjSplit; ++ww) {
    ya += reinterpret_cast<const float *>(&s_red[ww][0][b][0])[xr];
    yb += reinterpret_cast<const float *>(&s_red[ww][1][b][0])[xr];
  }
  if constexpr (MODE == 0) {
    float *y = first ? p.y0 : p.y1;
    const long ldy = first ? p.ldy0 : p.ldy1;
    if (rowA + xr < wrows) {
      float *d = y + (size_t)bg * ldy + rowA + xr;
      *d = p.accumulate ? *d + ya : ya;
    }
    if (rowB + xr < wrows) {
      float *d = y + (size_t)bg * ldy + rowB + xr;
      *d = p.accumulate ? *d + yb : yb;
    }
  } else {
    if constexpr (NORM) {
      float q = 0.f;
#pragma unroll
      for (int ww = 0; ww < kProjSplit; ++ww) q += s_ss[ww][b];
      const float inv = rsqrtf(q / (float)cols + p.rms_eps);
      ya *= inv;
      yb *= inv;
    }
    if (U.sec == 3) {
      float *gl = p.gate_out + (size_t)bg * p.ld_gate;
      if (xr < p.num_heads) gl[xr] = ya;
      if (16 + xr < p.num_heads) gl[16 + xr] = yb;
      return;
    }
    const SeqDesc &sd = p.seq[bg];
    const int dA = U.ta * 16 + xr, dB = U.tb * 16 + xr;
    if (U.rotate) rope_rotate(sd.position, dA, p.rotary_dim, p.log2_theta, ya, yb);
    if (U.sec == 0) {
      float *q = p.q_out + (size_t)bg * p.ld_q + (size_t)U.head * kHeadDim;
      q[dA] = ya;
      q[dB] = yb;
    } else {
      _Float16 *dst = (U.sec == 1 ? sd.k : sd.v) + (size_t)sd.slot * p.num_kv_heads * kHeadDim +
                      (size_t)U.head * kHeadDim;
      dst[dA] = (_Float16)ya;
      dst[dB] = (_Float16)yb;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention, split-K over the window, on the matrix cores.
//
// A workgroup owns chunk cid (logical positions [t0, t0 + chunk) of one
// sequence) for KV head g (partial_unit gives the map) and serves that head's
// 4 query heads, so each KV byte is read from HBM once.  Its W waves (4, or 2
// for batches) take interleaved 16-row tiles of the chunk: wave w tiles w,
// w + W, w + 2W, ...  This token's k and v are already in the cache (the qkv
// kernel wrote them), so every row of the window is read the same way.
//
// Both products are small dense contractions per 16-row tile -- S = K q for
// 4 query heads and O += P V -- and on VALU they cost ~65 instructions per
// row, more than the HBM stream leaves room for; on MFMA they cost ~2.
// Per 16-row tile:
//   S^T[16 rows x 16] = K[16 x 256] * Qf[256 x 16] with
//           v_mfma_f32_16x16x32_f16: the K tile is staged in LDS and read
//           as A fragments (lane l: row l%16, 8 dims), Qf's columns 0-3 hold
//           the fp16 high part of the 4 query heads (pre-scaled by
//           scale*log2(e)) and 4-7 the fp16 low part (q - hi), so
//           S = hi + lo keeps fp32 accuracy.
//   online softmax with a lazily moved reference max (see kRescaleSlack).
//   O[16 x 256] += P[16 x 16 rows] * V[16 rows x 256] with
//           v_mfma_f32_16x16x16_f16: P's rows 0-3 are the fp16 high part of
//           exp2(s - m) for the 4 heads, rows 4-7 the low part; V goes from
//           HBM straight into LDS (buffer_load ... lds) and is read back
//           transposed (ds_read_b64_tr_b16) into the B-operand layout.
// K and V of the next tile are in flight while a tile is computed (two LDS
// buffers each per wave).  Buffer loads whose offsets are out of range return
// zeros without an HBM access, which pads the last tile.  The W waves then
// merge their (m, l, O) in LDS and the workgroup writes one partial per query
// head; a combine kernel, or the merge tasks of the one-launch kernels,
// merge the chunks.
// ---------------------------------------------------------------------------

// Workgroup -> (chunk cid, KV head g).  The hardware deals workgroups to the
// 8 XCDs round-robin (workgroup b runs on XCD b % 8).  When the chunk count
// is a multiple of 8, XCD x takes chunks x, x + 8, x + 16, ... with all of
// their KV heads, so each XCD's L2 sees whole cache rows; otherwise
// consecutive workgroups are the KV heads of one chunk.  Either way the map
// is a bijection onto [0, total_chunks) x [0, Hk).
constexpr bool kXcdChunkMap = true;
__device__ __forceinline__ void partial_unit(const AttnParams &p, int &cid, int &g) {
  const int b = blockIdx.x;
  const int Hk = p.num_kv_heads;
  if (kXcdChunkMap && (p.total_chunks & 7) == 0) {
    const int k = b >> 3;
    const int j = k / Hk;
    g = k - j * Hk;
    cid = (b & 7) + 8 * j;
  } else {
    cid = b / Hk;
    g = b - cid * Hk;
  }
}

__device__ __forceinline__ int find_seq(const AttnParams &p, int chunk_id) {
  int s = 0;
  for (int i = 1; i < p.nseq; ++i)
    if (chunk_id >= p.seq[i].chunk_begin) s = i;
  return s;
}

constexpr int kTileHalves = kTileRows * kHeadDim;   // one staged V tile: 8 KB

// Wait until at most N of this wave's vector-memory operations are in flight
// (s_waitcnt vmcnt(N) in the gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt and lgkmcnt left at their no-wait maxima).  The attention's tile
// pipeline states its own waits: the compiler's tracking of loads into LDS
// cannot always tell which staged buffer a read depends on, and where it
// cannot it has been seen to leave the wait out.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// One column block J of a staged V tile: 64 lanes x 16 B from HBM into LDS
// at sv + J KB + 16 B * lane.  The block's 64 B of each row is selected with
// the scalar offset J * 64, which moves only the global address (the
// instruction's immediate offset would move the LDS address as well).
template <int J, int POLICY = 0>
__device__ __forceinline__ void vload_block(__amdgpu_buffer_rsrc_t rs, _Float16 *sv, unsigned off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(sv + J * 512), 16, off, J * 64, 0, POLICY);
}

// Staged V tile in LDS: eight 1 KB column blocks j (dims 32j .. 32j+31), each
// with the 16 rows at 64 B per row; rows r with bit 2 set keep their two 32 B
// halves swapped.  A transposed read of a 16-dim slice then lands 8 rows x
// 32 B on distinct banks in each half wave, with the slice's offset an
// immediate.  One buffer_load ... lds writes 1 KB (64 lanes x 16 B) = one
// column block: lane l brings row l/4, quarter l%4 of that row's 64 B.
// One wave's work.  sv0 / sv1 are this wave's two staged V buffers; passing
// them as restrict parameters gives their accesses alias scopes, so the
// compiler waits for a buffer's LDS-bound loads only before reading that
// buffer (not for the other buffer's loads, which are still in flight).
// sq is this wave's 4 KB staging area for its query fragments.
// The chunk: rows [t0, t0 + chunk) of sequence sd (chunk index ci inside
// the sequence), KV head g, whose 4 query heads start at q_seq + g * 4 * D.
// before_q() runs after the first tiles' loads are issued and before q is
// read (the fused block kernel waits there for q).
struct NoWait {
  __device__ __forceinline__ void operator()() const {}
};

// QC: q is read coherently (other workgroups of the same launch wrote it),
// and so are the tiles.  tc (with QC): the chunk holds this token's cache
// row, written in the same launch; its first tiles are still issued before
// before_q() waits, and the one row the wait makes visible is loaded again
// after it (every chunk takes the same path, so that the fused kernel
// carries one copy of this code).
template <int W, bool QC = false, typename BeforeQ = NoWait>
__device__ __forceinline__ void attn_partial_wave(const float *q_seq, const SeqDesc &sd, int ci, int chunk, int Hk,
                                                  float qscale, int g, int w, _Float16 *__restrict__ sk0,
                                                  _Float16 *__restrict__ sk1, _Float16 *__restrict__ sv0,
                                                  _Float16 *__restrict__ sv1, _Float16 *__restrict__ sq,
                                                  float &m_out, float &l_out, BeforeQ before_q = BeforeQ(),
                                                  bool tc = false) {
  const int lane = threadIdx.x & 63;
  const int t0 = sd.kv_start + ci * chunk;
  const int nrows = min(chunk, sd.kv_start + sd.n - t0);
  // wave w of the W takes tiles w, w + W, w + 2W, ... of the chunk
  const int ntiles = nrows > kTileRows * w ? (nrows - kTileRows * w + W * kTileRows - 1) / (W * kTileRows) : 0;
  const unsigned row_bytes = (unsigned)Hk * kHeadDim * 2u;
  const int ring = sd.ring;
  const int p0 = ring ? (t0 % ring) : t0;        // physical row of t0; a chunk wraps at most once
  const int ring_end = ring ? ring : 0x7FFFFFFF;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(sd.k, sd.cache_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(sd.v, sd.cache_bytes);
  const unsigned head_off = (unsigned)g * kHeadDim * 2u;
  const int G = lane >> 4;                       // lane group (MFMA k-slot group / D row group)
  const int n = lane & 15;                       // lane within the group (MFMA row / column)

  // byte offset of row `rel` (relative to t0) of this KV head, or out of range
  auto row_off = [&](int rel) -> unsigned {
    int ph = p0 + rel;
    ph -= ph >= ring_end ? ring : 0;
    const unsigned off = __umul24((unsigned)ph, row_bytes) + head_off;   // ph, row_bytes < 2^24
    return rel < nrows ? off : kOutOfRange;
  };
  // Tile t of this wave into a staged buffer: instruction j brings rows 2j
  // and 2j + 1 of the tile (lane l: row 2j + l/32, LDS position l % 32 of
  // that row's 32 pieces of 16 B), so every instruction reads whole 128 B
  // lines, which the non-temporal policy needs.  Row r's piece p sits at
  // position p ^ swz(r) (K: swz = r % 16; V: swz = 2 (r % 8)), chosen so
  // that the fragment reads below hit distinct LDS banks.
  auto load_piece = [&](_Float16 *sbuf, int t, int jj, auto k_tag) {
    constexpr bool is_k = decltype(k_tag)::value;
    const __amdgpu_buffer_rsrc_t rs = is_k ? krs : vrs;
    const int pos = lane & 31;
    const int r = 2 * jj + (lane >> 5);
    const int pc = is_k ? (pos & 16) | ((pos ^ r) & 15) : pos ^ (2 * (r & 7));
    const unsigned off = row_off((W * t + w) * kTileRows + r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(sbuf + jj * 512), 16,
                                             off == kOutOfRange ? off : off + 16u * (unsigned)pc, 0, 0,
                                             (is_k ? kKPolicy : kVPolicy) | (QC ? kCoherent : 0));
  };
  auto load_tile = [&](_Float16 *sbuf, int t, auto k_tag) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) load_piece(sbuf, t, jj, k_tag);
  };
  auto load_k = [&](_Float16 *sk, int t) { load_tile(sk, t, std::true_type{}); };
  auto load_v = [&](_Float16 *sv, int t) { load_tile(sv, t, std::false_type{}); };

  // An even number of tiles (a padding tile is fully masked and its loads
  // are out of range: no HBM traffic), so that no load below is conditional
  // and the compiler's waits stay exact.
  // A wave without rows (a short chunk) runs two fully masked tiles: its
  // loads are out of range and it contributes m = -inf, l = 0, O = 0.
  const int ne = ntiles > 2 ? (ntiles + 1) & ~1 : 2;
  // With QC the q loads follow the first tiles and are waited for before the
  // first scores, so every first tile has landed by then and the waits below
  // do not count on them: a wave with fewer than two tiles of rows issues no
  // padding tile (each costs the wave about 0.2 us of issue time, in range or
  // not).
  auto first_tiles = [&]() {
    if (!QC || ntiles >= 1) {
      load_k(sk0, 0);
      load_v(sv0, 0);
    }
    if (!QC || ntiles >= 2) {
      load_k(sk1, 1);
      load_v(sv1, 1);
    }
  };
  // Without a wait, q is loaded first (its wait then does not include the
  // tile loads); lane l takes dims 4l .. 4l+3 of the KV head's 4 query heads.
  float4 qv[kGroup];
  auto load_q = [&]() {
    const float *qh = q_seq + (size_t)g * kGroup * kHeadDim + lane * 4;
    if constexpr (QC) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(q_seq + (size_t)g * kGroup * kHeadDim, (unsigned)(kGroup * kHeadDim * 4));
#pragma unroll
      for (int i = 0; i < kGroup; ++i)
        qv[i] = __builtin_bit_cast(float4, buf_load16_p<kCoherent>(rq, (unsigned)((i * kHeadDim + lane * 4) * 4)));
    } else {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) qv[i] = *reinterpret_cast<const float4 *>(qh + i * kHeadDim);
    }
  };
  if constexpr (QC) {
    first_tiles();
    before_q();
    if (tc) {
      // This chunk holds this token's cache row (its last row), written in
      // this launch: the wave whose first tiles hold it loads that row's
      // piece of K and V again now that the wait has made it visible, once
      // its earlier loads into the same LDS have landed.  (A row in a later
      // tile is loaded after the wait anyway.)
      const int rel = nrows - 1;
      const int T = rel / kTileRows;
      if (T % W == w && T / W < 2) {
        vm_wait<0>();
        const int jj = (rel % kTileRows) / 2;
        load_piece(T / W == 0 ? sk0 : sk1, T / W, jj, std::true_type{});
        load_piece(T / W == 0 ? sv0 : sv1, T / W, jj, std::false_type{});
      }
    }
    load_q();
  } else {
    before_q();
    load_q();
    first_tiles();
  }

  // Query fragments, built while the first tiles are in flight: each lane
  // splits its dims (pre-scaled by scale * log2(e)) into fp16 high and low
  // parts in the wave's staging area sq = [hi, lo][query head][dim]; then the
  // Qf B-fragments: lane (G, n) holds column n, dims 32s + 8G .. +8 of
  // hi(q_{n % 4}) for n % 8 < 4, else lo(q_{n % 4}).  Columns 8-15 repeat
  // columns 0-7; only columns 0-7 of the scores are used.
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float x[4] = {qv[i].x * qscale, qv[i].y * qscale, qv[i].z * qscale, qv[i].w * qscale};
    half4_t hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi[j] = (_Float16)x[j];
      lo[j] = (_Float16)(x[j] - (float)hi[j]);
    }
    *reinterpret_cast<half4_t *>(sq + i * kHeadDim + lane * 4) = hi;
    *reinterpret_cast<half4_t *>(sq + (kGroup + i) * kHeadDim + lane * 4) = lo;
  }
  half8_t qf[8];
  {
    const _Float16 *src = sq + (((n >> 2) & 1) * kGroup + (n & 3)) * kHeadDim + G * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = *reinterpret_cast<const half8_t *>(src + s * 32);
    }
  }

  // acc[c][i] at lane (G, n): row 4G + i, dim 16c + n of O, i.e. head i
  // (G = 0 high part, G = 1 low part; rows 8-15 stay zero)
  floatx4_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // lanes (G, n < 4): reference max of head n (log2 units)
  float l_run = 0.f;         // lanes (G, n < 4): this lane group's share of head n's sum
  // K A-fragment of k-step s: lane (G, n) reads row n, piece 4s + G, i.e.
  // byte 512 n + 256 (s / 4) + 16 ((4 (s % 4) + G) ^ n); a quarter wave
  // (fixed G) covers 16 distinct bank groups.
  int kaddr[4];
#pragma unroll
  for (int s3 = 0; s3 < 4; ++s3) kaddr[s3] = n * 512 + 16 * ((4 * s3 + G) ^ n);
  // V transposed read of dim slice c (dims 16c .. 16c+15): lane (G, n) points
  // at row 4G + n/4, dims 16c + 4 (n % 4) .. +3 = piece 2c + (n % 4) / 2, half
  // n % 2; with the swizzle that is byte 512 row + 256 (c / 8)
  // + 32 ((c % 8) ^ (row % 8)) + 16 ((n / 2) % 2) + 8 (n % 2).  A half wave
  // reads 8 rows x 32 B on distinct banks.
  const int vrow = 4 * G + (n >> 2);
  int vaddr[8];
#pragma unroll
  for (int c7 = 0; c7 < 8; ++c7) vaddr[c7] = vrow * 512 + 32 * (c7 ^ (vrow & 7)) + 16 * ((n >> 1) & 1) + 8 * (n & 1);

  // Every tile is 8 load instructions per wave, issued in the order K_t, V_t,
  // K_{t+1}, V_{t+1}, K_{t+2}, ...: before a tile is read, the loads issued
  // after its own are the ones allowed in flight (24 inside the loop, then
  // 24, 16, 8, 0 for the last two tiles).
  //
  // S^T = K Qf for the staged K tile: d[i] = S[row 4G+i][column n]; column
  // n+4 holds the low part
  auto scores = [&](const _Float16 *sk, auto wait) {
    vm_wait<decltype(wait)::value>();
    const char *kbase = reinterpret_cast<const char *>(sk);
    half8_t kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = *reinterpret_cast<const half8_t *>(kbase + kaddr[s & 3] + (s >> 2) * 256);
    __builtin_amdgcn_sched_barrier(0);   // all 8 reads in flight before the first product
    floatx4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], qf[s], d, 0, 0, 0);
    return d;
  };
  // online softmax of tile t's scores and O += P V from the staged V tile.
  // The 16 B fragments of V are read first, into registers of their own, so
  // that their LDS latency overlaps the softmax (read into one register pair
  // each, the reads and products would run one LDS round trip at a time).
  auto process = [&](floatx4_t d, const _Float16 *sv, int t, auto wait) {
    vm_wait<decltype(wait)::value>();
    const char *base = reinterpret_cast<const char *>(sv);
    short4_t vt[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
      vt[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)(base + vaddr[c & 7] + (c >> 3) * 256));
    __builtin_amdgcn_sched_barrier(0);
    float sc[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = d[i] + dpp<0x104>(d[i]);             // row_shl:4 -> value of lane n+4
      if (n >= kGroup || (W * t + w) * kTileRows + 4 * G + i >= nrows) sc[i] = -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = max_across_rows(tmax);
    // Lazy rescaling: the reference max m_run moves only when a score exceeds
    // it by more than kRescaleSlack (log2 units), so P = exp2(s - m_run) stays
    // <= 2^kRescaleSlack (exact in fp16 hi + lo) and the 64 accumulators are
    // rescaled only on the rare tiles where the max jumps.
    // While no head has a finite reference max, no score has been taken
    // in: O and l are still zero and there is nothing to rescale.
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleSlack) != 0) {
      const bool seen = __builtin_amdgcn_ballot_w64(m_run != -INFINITY) != 0;
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      if (seen) {
        float al[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) al[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
#pragma unroll
        for (int c = 0; c < 16; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[c][i] *= al[i];
      }
    }
    float pr[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m_run);
      psum += pr[i];
    }
    l_run += psum;
    // P A-fragment: lane (G, m) holds P[row m][k = rows 4G..4G+3]; rows 0-3 the
    // high fp16 part of head m, rows 4-7 the low part of head m-4 (from lane m-4)
    half4_t pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = n < 4 ? pr[i] : dpp<0x114>(pr[i]);   // row_shr:4 -> value of lane n-4
      const _Float16 hi = (_Float16)pv;
      pf[i] = n < 4 ? hi : (n < 8 ? (_Float16)(pv - (float)hi) : (_Float16)0.f);
    }
    // O += P V
#pragma unroll
    for (int c = 0; c < 16; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(pf, __builtin_bit_cast(half4_t, vt[c]), acc[c], 0, 0, 0);
  };
  // A K buffer is refilled as soon as its scores are formed (the MFMAs have
  // consumed every read of it), a V buffer after O += P V; sched_barrier keeps
  // each refill behind the reads of its buffer.
  using in_flight_24 = std::integral_constant<int, 24>;
  for (int t = 0; t + 2 < ne; t += 2) {
    floatx4_t d = scores(sk0, in_flight_24{});
    __builtin_amdgcn_sched_barrier(0);
    load_k(sk0, t + 2);
    process(d, sv0, t, in_flight_24{});
    __builtin_amdgcn_sched_barrier(0);
    load_v(sv0, t + 2);
    d = scores(sk1, in_flight_24{});
    __builtin_amdgcn_sched_barrier(0);
    load_k(sk1, t + 3);
    process(d, sv1, t + 1, in_flight_24{});
    __builtin_amdgcn_sched_barrier(0);
    load_v(sv1, t + 3);
  }
  // The last two tiles; a wave with fewer than two tiles of rows skips the
  // padding tiles' arithmetic (a fully masked tile adds exactly nothing; its
  // out-of-range loads still complete before the buffers are reused).
  if (ntiles >= ne - 1) {
    const floatx4_t d = scores(sk0, in_flight_24{});
    process(d, sv0, ne - 2, std::integral_constant<int, 16>{});
  }
  if (ntiles >= ne) {
    const floatx4_t d = scores(sk1, std::integral_constant<int, 8>{});
    process(d, sv1, ne - 1, std::integral_constant<int, 0>{});
  }
  vm_wait<0>();   // (a skipped tile's loads land in sv0 / sv1 before they are reused below)

  // ---- this wave's partial: add the high and low rows, stage (m, l, O) ----
  // One row swap serves two accumulators: swapping rows 1 / 3 of acc[c][i]
  // with rows 0 / 2 of acc[c + 8][i] and adding leaves, in lane group 0,
  // high + low of acc[c][i] and, in lane group 1, high + low of acc[c + 8][i].
  l_run = sum_across_rows(l_run);
  float o8[8][4];   // lane group 0: dims 16c + n; lane group 1: dims 16 (c + 8) + n
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[c][i]), __float_as_uint(acc[c + 8][i]),
                                                      false, false);
      o8[c][i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  // staged per query head i in the first 4 KB of sv0 (idle now): element
  // n * 16 + c holds dim 16c + n, the layout of the partials
  if (G < 2) {
    float *st = reinterpret_cast<float *>(sv0) + n * 16 + G * 8;
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
#pragma unroll
      for (int c4 = 0; c4 < 2; ++c4)
        *reinterpret_cast<float4 *>(st + i * kHeadDim + c4 * 4) =
            make_float4(o8[c4 * 4][i], o8[c4 * 4 + 1][i], o8[c4 * 4 + 2][i], o8[c4 * 4 + 3][i]);
  }
  m_out = m_run;
  l_out = l_run;
}

// The attention-sink term of query head h's softmax denominator, relative to
// the reference point M of the merged sum (log2 units): 2^(sigma_h log2(e) - M),
// 0 without sinks.  Sink logits are in the units of the scaled scores and
// carry no value row, so only the denominator grows.  A term past the fp32
// range gives 0 output, which is the limit.
__device__ __forceinline__ float sink_term(const float *sinks, int h, float M) {
  return sinks ? __builtin_amdgcn_exp2f(fmaf(sinks[h], 1.4426950408889634f, -M)) : 0.f;
}

// The W waves' (m, l, O) of query head i (staged by attn_partial_wave: (m, l)
// at the start of each wave's sq, O in the first 4 KB of its sv0) merged into
// one partial: M the largest m, L and lane l's elements 4l .. 4l+3 of O
// weighed by 2^(m - M), waves in order.
template <int W>
__device__ __forceinline__ void merge_waves(const _Float16 (*sq)[2 * kGroup * kHeadDim],
                                            const _Float16 (*sv0)[kTileHalves], int i, int lane, float &M, float &L,
                                            float4 &o) {
  auto m_of = [&](int ww) { return reinterpret_cast<const float *>(sq[ww])[i]; };
  auto l_of = [&](int ww) { return reinterpret_cast<const float *>(sq[ww])[kGroup + i]; };
  M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) M = fmaxf(M, m_of(ww));
  L = 0.f;
  o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int ww = 0; ww < W; ++ww) {
    const float mw = m_of(ww);
    const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);   // a wave without rows
    L = fmaf(wt, l_of(ww), L);
    const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(sv0[ww]) +
                                                       i * kHeadDim + lane * 4);
    o.x = fmaf(wt, v.x, o.x);
    o.y = fmaf(wt, v.y, o.y);
    o.z = fmaf(wt, v.z, o.z);
    o.w = fmaf(wt, v.w, o.w);
  }
}

// Workgroup = (chunk cid, KV head g); its W waves split the chunk's rows and
// then merge in LDS, so one partial per (chunk, query head) is written.
// 36 KB of LDS per wave: W = 4 (144 KB) runs one workgroup per CU, W = 2
// (72 KB) two; either way one wave per SIMD.  Measured on 32 sequences of up
// to 16K rows: W = 2 with 512 workgroups 202.4 us against 209.6 us for W = 4
// with 256; on one 32K sequence W = 2 was slower (26.5 against 26.1 us).
template <int W>
__global__ __launch_bounds__(64 * W, 1) void attn_partial_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) _Float16 s_k0[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_k1[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_v0[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_v1[W][kTileHalves];
  // per wave: its query fragments during the loop, then its (m, l) per query head
  __shared__ __attribute__((aligned(16))) _Float16 s_q[W][2 * kGroup * kHeadDim];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, kept scalar
  const int Hk = p.num_kv_heads;
  const int Hq = Hk * kGroup;
  int cid, g;
  partial_unit(p, cid, g);
  const int b = find_seq(p, cid);
  float m_run, l_run;
  attn_partial_wave<W>(p.q + (size_t)b * p.ld_q, p.seq[b], cid - p.seq[b].chunk_begin, p.chunk, Hk, p.qscale, g, w,
                       s_k0[w], s_k1[w], s_v0[w], s_v1[w], s_q[w], m_run, l_run);
  if (lane < kGroup) {
    float *ml = reinterpret_cast<float *>(s_q[w]);
    ml[lane] = m_run;
    ml[kGroup + lane] = l_run;
  }
  __syncthreads();
  // wave w merges query heads i = w, w + W, ... of this KV head: lane l owns
  // elements 4l .. 4l+3
  for (int i = w; i < kGroup; i += W) {
    float M, L;
    float4 o;
    merge_waves<W>(s_q, s_v0, i, lane, M, L, o);
    if (p.direct) {
      // the chunk is the whole window of sequence cid: normalise, gate, write
      const int qh = g * kGroup + i;
      const float gl = p.gate[(size_t)cid * p.ld_gate + qh];
      const float sc = (1.0f / (1.0f + expf(-gl))) / (L + sink_term(p.sinks, qh, M));
      float *dst = p.out + (size_t)cid * p.ld_out + (size_t)qh * kHeadDim;
      const float v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;                  // element e holds dim 16 (e % 16) + e / 16
        dst[16 * (e & 15) + (e >> 4)] = v[j] * sc;
      }
      continue;
    }
    const size_t row = (size_t)cid * Hq + g * kGroup + i;
    *reinterpret_cast<float4 *>(p.part_o + row * kHeadDim + lane * 4) = o;
    if (lane == 0) *reinterpret_cast<float2 *>(p.part_ml + row * 2) = make_float2(M, L);
  }
}

// ---------------------------------------------------------------------------
// Attention for several tokens of one sequence (a chunk of prefill, a
// verify step): every K/V tile is read once for 16 query vectors at a time.
//
// Wave w of workgroup (row chunk c, KV head g, token group tg) serves tokens
// 4 (4 tg + w) .. +3, i.e. 16 query vectors n = 4 * token + head (the KV
// head's 4 query heads), over all rows of chunk c; the 4 waves of a
// workgroup read the same rows (from L1/L2 after the first), the token
// groups of a (c, g) sit 8 workgroups apart, i.e. on one XCD.  Per 16-row
// tile, as in attn_partial_wave but with 16 query columns:
//   S^T = K Qf on v_mfma_f32_16x16x32_f16, q split into fp16 high and low
//         parts as two B operands (two chains of 8);
//   causal mask per column: row r counts for token t iff ks_t <= r <= pos_t;
//   online softmax per column with the lazy reference max;
//   O += P V on v_mfma_f32_16x16x16_f16 with P's high and low parts as two
//         A operands (S^T's output layout is already P's A layout: lane
//         (G, n) holds column n, rows 4G .. 4G+3).
// O's rows are the 16 queries; each wave writes its own partials (no merge
// inside the workgroup).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void attn_chunk_wave(const ChunkAttnParams &p, int c, int g, int tb,
                                                _Float16 *__restrict__ sv0, _Float16 *__restrict__ sv1) {
  const int lane = threadIdx.x & 63;
  const int Hk = p.num_kv_heads;
  const int Hq = Hk * kGroup;
  const int G = lane >> 4, n = lane & 15;
  const SeqDesc &sd = p.seq;
  const int rbase = p.r0 + c * p.chunk;               // first row (logical position) of the chunk
  const int rend = p.first_pos + p.m_tokens;           // rows end (exclusive)
  const int nrows = min(p.chunk, rend - rbase);
  const int ne = p.chunk / kTileRows;                  // even: chunk is a multiple of 32
  const unsigned row_bytes = (unsigned)Hk * kHeadDim * 2u;
  const int ring = sd.ring;
  const int pb = ring ? rbase % ring : rbase;          // physical row of rbase; a chunk wraps at most once
  const int ring_end = ring ? ring : 0x7FFFFFFF;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(sd.k, sd.cache_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(sd.v, sd.cache_bytes);
  const unsigned head_off = (unsigned)g * kHeadDim * 2u;

  auto row_off = [&](int rel) -> unsigned {
    int ph = pb + rel;
    ph -= ph >= ring_end ? ring : 0;
    const unsigned off = __umul24((unsigned)ph, row_bytes) + head_off;
    return rel < nrows ? off : kOutOfRange;
  };
  auto load_k = [&](half8_t (&kf)[8], int t) {
    const unsigned off = row_off(t * kTileRows + n) + (unsigned)G * 16u;
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = __builtin_bit_cast(half8_t, buf_load16(krs, off + (unsigned)s * 64u));
  };
  auto load_v = [&](_Float16 *sv, int t) {
    const int r = lane >> 2;
    const int q = lane & 3;
    const unsigned off = row_off(t * kTileRows + r) + 32u * (unsigned)(((q >> 1) ^ (r >> 2)) & 1) +
                         16u * (unsigned)(q & 1);
    vload_block<0>(vrs, sv, off);
    vload_block<1>(vrs, sv, off);
    vload_block<2>(vrs, sv, off);
    vload_block<3>(vrs, sv, off);
    vload_block<4>(vrs, sv, off);
    vload_block<5>(vrs, sv, off);
    vload_block<6>(vrs, sv, off);
    vload_block<7>(vrs, sv, off);
  };

  // this lane's column: query n = token tq, query head g*4 + (n & 3)
  const int tq = 4 * tb + (n >> 2);
  const int qpos = p.first_pos + tq;
  const int qlo = max(0, qpos + 1 - p.window);         // first row token tq reads
  const bool qvalid = tq < p.m_tokens;
  // its q, dims 32s + 8G .. +8 (out of range past the last token: zeros)
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q, (unsigned)((size_t)p.m_tokens * p.ld_q * 4u));
  const unsigned qoff = (unsigned)(((size_t)tq * p.ld_q + (size_t)(g * kGroup + (n & 3)) * kHeadDim) * 4u) +
                        (unsigned)G * 32u;
  float4 qa[8], qb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const unsigned o = qvalid ? qoff + (unsigned)s * 128u : kOutOfRange;
    qa[s] = __builtin_bit_cast(float4, buf_load16(rq, o));
    qb[s] = __builtin_bit_cast(float4, buf_load16(rq, o == kOutOfRange ? o : o + 16u));
  }
  half8_t kA[8], kB[8];
  load_k(kA, 0);
  load_v(sv0, 0);
  load_k(kB, 1);
  load_v(sv1, 1);
  // Qf B-fragments: q * scale * log2(e) as fp16 high + low parts
  half8_t qh[8], ql[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float x[8] = {qa[s].x, qa[s].y, qa[s].z, qa[s].w, qb[s].x, qb[s].y, qb[s].z, qb[s].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = x[j] * p.qscale;
      const _Float16 h = (_Float16)v;
      qh[s][j] = h;
      ql[s][j] = (_Float16)(v - (float)h);
    }
  }

  // acc[c][i] at lane (G, n): query 4G + i, dim 16c + n
  floatx4_t acc[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) acc[cc] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // column n's reference max (log2 units), in every lane group
  float l_run = 0.f;         // this lane group's share of column n's sum
  const int vrow = 4 * G + (n >> 2);
  const int rd_even = vrow * 64 + (G & 1) * 32 + (n & 3) * 8;
  const int rd_odd = vrow * 64 + ((G & 1) ^ 1) * 32 + (n & 3) * 8;

  auto process = [&](const half8_t (&kf)[8], const _Float16 *sv, int t) {
    floatx4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], qh[s], d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], ql[s], d1, 0, 0, 0);
    }
    float sc[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + t * kTileRows + 4 * G + i;   // row of d[i]
      sc[i] = d0[i] + d1[i];
      if (!qvalid || r < qlo || r > qpos) sc[i] = -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = max_across_rows(tmax);
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      // acc row 4G + i is query 4G + i: its factor sits in lane 4G + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float al = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * G + i) * 4, __float_as_int(alpha)));
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) acc[cc][i] *= al;
      }
    }
    half4_t ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m_run);
      l_run += pv;
      const _Float16 h = (_Float16)pv;
      ph[i] = h;
      pl[i] = (_Float16)(pv - (float)h);
    }
    const char *base = reinterpret_cast<const char *>(sv);
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) {
      const half4_t vt = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t *)(base + (cc & 1 ? rd_odd : rd_even) + (cc >> 1) * 1024)));
      acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vt, acc[cc], 0, 0, 0);
      acc[cc] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vt, acc[cc], 0, 0, 0);
    }
  };
  for (int t = 0; t + 2 < ne; t += 2) {
    process(kA, sv0, t);
    __builtin_amdgcn_sched_barrier(0);
    load_k(kA, t + 2);
    load_v(sv0, t + 2);
    process(kB, sv1, t + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_k(kB, t + 3);
    load_v(sv1, t + 3);
  }
  process(kA, sv0, ne - 2);
  process(kB, sv1, ne - 1);

  // ---- partials of the 16 queries: O staged through this wave's V buffers
  // (query q' < 8 in sv0, else sv1; element n * 16 + c holds dim 16c + n) ----
  l_run = sum_across_rows(l_run);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = 4 * G + i;
    float *st = reinterpret_cast<float *>(qq < 8 ? sv0 : sv1) + (qq & 7) * kHeadDim + n * 16;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      *reinterpret_cast<float4 *>(st + c4 * 4) =
          make_float4(acc[c4 * 4][i], acc[c4 * 4 + 1][i], acc[c4 * 4 + 2][i], acc[c4 * 4 + 3][i]);
  }
  // (LDS writes and reads of one wave are in order: no barrier)
#pragma unroll
  for (int qq = 0; qq < 16; ++qq) {
    const int t2 = 4 * tb + (qq >> 2);
    if (t2 >= p.m_tokens) break;
    const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(qq < 8 ? sv0 : sv1) +
                                                       (qq & 7) * kHeadDim + lane * 4);
    const size_t row = ((size_t)t2 * p.nchunks + c) * Hq + g * kGroup + (qq & 3);
    *reinterpret_cast<float4 *>(p.part_o + row * kHeadDim + lane * 4) = v;
  }
  if (G == 0 && qvalid) {
    const size_t row = ((size_t)tq * p.nchunks + c) * Hq + g * kGroup + (n & 3);
    *reinterpret_cast<float2 *>(p.part_ml + row * 2) = make_float2(m_run, l_run);
  }
}

// Grid: units (chunk, KV head) rounded up to 8, times token groups; the token
// groups of a unit are 8 workgroups apart (one XCD).
__global__ __launch_bounds__(kThreads, 2) void attn_chunk_kernel(const ChunkAttnParams p) {
  __shared__ __attribute__((aligned(1024))) _Float16 s_v0[4][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_v1[4][kTileHalves];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntg = (p.m_tokens + 15) / 16;
  const int grp = blockIdx.x / (8 * ntg), off = blockIdx.x - grp * (8 * ntg);
  const int u = grp * 8 + (off & 7);
  const int tg = off >> 3;
  if (u >= p.nchunks * p.num_kv_heads) return;
  const int c = u / p.num_kv_heads;
  const int g = u - c * p.num_kv_heads;
  const int tb = 4 * tg + w;                            // token block: tokens 4 tb .. 4 tb + 3
  if (4 * tb >= p.m_tokens) return;                     // no token of this wave (no barrier follows)
  attn_chunk_wave(p, c, g, tb, s_v0[w], s_v1[w]);
}

// Merge of the split-K partials and the headwise gate.
// Grid (Hq * kCombineSplit, nseq).  Workgroup (h, part) owns query head h and
// the 16 stored elements [part*16, part*16 + 16) of its partials (stored
// element n * 16 + c holds dim 16c + n).  Thread (cg, dq): dq = tid % 4 owns
// 4 elements, chunk group cg = tid / 4 takes chunks cg, cg + 64, ... and
// merges them online (running max, sum, acc), four chunks' loads at a time;
// then wave dq merges the 64 groups of its 4 elements across its lanes.
constexpr int kCombineSplit = 16;
constexpr int kCombineElems = kHeadDim / kCombineSplit;   // 16
constexpr int kCombineQuads = kCombineElems / 4;          // 4 threads per chunk row
constexpr int kCombineGroups = kThreads / kCombineQuads;  // 64 chunk groups
constexpr int kCombineBatch = 4;

__global__ __launch_bounds__(kThreads) void attn_combine_kernel(const AttnParams p) {
  __shared__ float4 s_o[kCombineGroups][kCombineQuads];
  __shared__ float2 s_ml[kCombineGroups];

  const int tid = threadIdx.x;
  const int h = blockIdx.x / kCombineSplit;
  const int part = blockIdx.x % kCombineSplit;
  const int b = blockIdx.y;
  const SeqDesc sd = p.seq[b];
  const int Hq = p.num_kv_heads * kGroup;
  const int nchunks = (sd.n + p.chunk - 1) / p.chunk;
  const int f0 = sd.chunk_begin;
  const int cg = tid / kCombineQuads;
  const int dq = tid % kCombineQuads;
  const int e0 = part * kCombineElems + dq * 4;

  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = cg; c0 < nchunks; c0 += kCombineGroups * kCombineBatch) {
    float4 o[kCombineBatch];
    float2 ml[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int c = c0 + u * kCombineGroups;
      if (c < nchunks) {
        const size_t row = (size_t)(f0 + c) * Hq + h;
        ml[u] = *reinterpret_cast<const float2 *>(p.part_ml + row * 2);
        o[u] = *reinterpret_cast<const float4 *>(p.part_o + row * kHeadDim + e0);
      } else {
        ml[u] = make_float2(-INFINITY, 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (ml[u].x == -INFINITY) continue;   // padding entry (a chunk always has rows)
      const float mn = fmaxf(m, ml[u].x);
      const float a = __builtin_amdgcn_exp2f(m - mn);       // 0 while m is -inf
      const float c = __builtin_amdgcn_exp2f(ml[u].x - mn);
      l = fmaf(l, a, ml[u].y * c);
      acc.x = fmaf(acc.x, a, o[u].x * c);
      acc.y = fmaf(acc.y, a, o[u].y * c);
      acc.z = fmaf(acc.z, a, o[u].z * c);
      acc.w = fmaf(acc.w, a, o[u].w * c);
      m = mn;
    }
  }
  s_o[cg][dq] = acc;
  if (dq == 0) s_ml[cg] = make_float2(m, l);
  __syncthreads();
  // wave q merges element quad q: lane k holds chunk group k
  const int lane = tid & 63;
  const int q = tid >> 6;
  const float2 mlk = s_ml[lane];
  const float M = wave_max(mlk.x);
  const float wt = mlk.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mlk.x - M);
  const float L = wave_sum(wt * mlk.y);
  const float4 ok = s_o[lane][q];
  const float ox = wave_sum(wt * ok.x);
  const float oy = wave_sum(wt * ok.y);
  const float oz = wave_sum(wt * ok.z);
  const float ow = wave_sum(wt * ok.w);
  if (lane == 0) {
    const float gl = p.gate[(size_t)b * p.ld_gate + h];
    const float gate = 1.0f / (1.0f + expf(-gl));
    const float sc = gate / (L + sink_term(p.sinks, h, M));
    // element e = n * 16 + c holds dim 16c + n
    const int e = part * kCombineElems + q * 4;
    float *dst = p.out + (size_t)b * p.ld_out + (size_t)h * kHeadDim + (e >> 4);
    const int c0 = e & 15;
    dst[16 * c0] = ox * sc;
    dst[16 * (c0 + 1)] = oy * sc;
    dst[16 * (c0 + 2)] = oz * sc;
    dst[16 * (c0 + 3)] = ow * sc;
  }
}

// The merge for plans with at most kCombineSmallChunks chunks per sequence
// (short windows, many sequences): one wave per (query head, sequence), lane
// l owns elements 4l .. 4l+3 and loads every chunk's partial at once.
constexpr int kCombineSmallChunks = 8;

__global__ __launch_bounds__(64) void attn_combine_small_kernel(const AttnParams p) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const SeqDesc sd = p.seq[b];
  const int Hq = p.num_kv_heads * kGroup;
  const int nchunks = (sd.n + p.chunk - 1) / p.chunk;
  float2 ml[kCombineSmallChunks];
  float4 o[kCombineSmallChunks];
#pragma unroll
  for (int u = 0; u < kCombineSmallChunks; ++u) {
    if (u < nchunks) {
      const size_t row = (size_t)(sd.chunk_begin + u) * Hq + h;
      ml[u] = *reinterpret_cast<const float2 *>(p.part_ml + row * 2);
      o[u] = *reinterpret_cast<const float4 *>(p.part_o + row * kHeadDim + lane * 4);
    } else {
      ml[u] = make_float2(-INFINITY, 0.f);
      o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < kCombineSmallChunks; ++u) M = fmaxf(M, ml[u].x);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kCombineSmallChunks; ++u) {
    const float wt = ml[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - M);
    L = fmaf(wt, ml[u].y, L);
    acc.x = fmaf(wt, o[u].x, acc.x);
    acc.y = fmaf(wt, o[u].y, acc.y);
    acc.z = fmaf(wt, o[u].z, acc.z);
    acc.w = fmaf(wt, o[u].w, acc.w);
  }
  const float gl = p.gate[(size_t)b * p.ld_gate + h];
  const float sc = (1.0f / (1.0f + expf(-gl))) / (L + sink_term(p.sinks, h, M));
  float *dst = p.out + (size_t)b * p.ld_out + (size_t)h * kHeadDim;
  const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane * 4 + j;                    // element e holds dim 16 (e % 16) + e / 16
    dst[16 * (e & 15) + (e >> 4)] = v[j] * sc;
  }
}

// The merge for plans with at most kCombineMidChunks chunks per sequence and
// enough (sequence, query head) pairs to fill the chip (several tokens of one
// sequence, batches of long windows): one workgroup per pair.  Lane c holds
// chunk c's (m, l), so every wave has the common reference max and the
// weights; wave w sums chunks w, w + 4, ... (all its loads issued at once),
// lane l owning elements 4l .. 4l+3, and the four sums are added in LDS.
constexpr int kCombineMidChunks = 64;

__global__ __launch_bounds__(kThreads) void attn_combine_mid_kernel(const AttnParams p) {
  __shared__ float4 s_acc[kThreads / 64][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const SeqDesc sd = p.seq[b];
  const int Hq = p.num_kv_heads * kGroup;
  const int nchunks = (sd.n + p.chunk - 1) / p.chunk;
  constexpr int kPer = kCombineMidChunks / (kThreads / 64);
  float4 o[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = w + (kThreads / 64) * u;
    o[u] = c < nchunks ? *reinterpret_cast<const float4 *>(
                             p.part_o + ((size_t)(sd.chunk_begin + c) * Hq + h) * kHeadDim + lane * 4)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float2 mlc = lane < nchunks
                         ? *reinterpret_cast<const float2 *>(p.part_ml + ((size_t)(sd.chunk_begin + lane) * Hq + h) * 2)
                         : make_float2(-INFINITY, 0.f);
  const float M = wave_max(mlc.x);
  const float wtc = mlc.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mlc.x - M);
  const float L = wave_sum(wtc * mlc.y);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = w + (kThreads / 64) * u;     // uniform: the weight comes from lane c
    const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wtc), c));
    acc.x = fmaf(wt, o[u].x, acc.x);
    acc.y = fmaf(wt, o[u].y, acc.y);
    acc.z = fmaf(wt, o[u].z, acc.z);
    acc.w = fmaf(wt, o[u].w, acc.w);
  }
  s_acc[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int k = 1; k < kThreads / 64; ++k) {
    const float4 t = s_acc[k][lane];
    acc.x += t.x;
    acc.y += t.y;
    acc.z += t.z;
    acc.w += t.w;
  }
  const float gl = p.gate[(size_t)b * p.ld_gate + h];
  const float sc = (1.0f / (1.0f + expf(-gl))) / (L + sink_term(p.sinks, h, M));
  float *dst = p.out + (size_t)b * p.ld_out + (size_t)h * kHeadDim;
  const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane * 4 + j;                    // element e holds dim 16 (e % 16) + e / 16
    dst[16 * (e & 15) + (e >> 4)] = v[j] * sc;
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

template <int R, int NIT, int RB, bool ONE>
hipError_t gemv_launch(const GemvParams &p, hipStream_t stream) {
  const int waves = (p.rows0 + p.rows1 + R - 1) / R;
  hipLaunchKernelGGL((gemv_bf16_kernel<R, NIT, RB, ONE>), dim3((waves + 3) / 4), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Two weight rows per wave while that still gives >= 2048 waves, else one;
// two batch rows per pass from batch 2 on while their x fits (NIT <= 8).
template <int NIT>
hipError_t gemv_rows(const GemvParams &p, hipStream_t stream) {
  const bool two = p.rows0 + p.rows1 >= 4096;
  if (p.batch == 1) return two ? gemv_launch<2, NIT, 1, true>(p, stream) : gemv_launch<1, NIT, 1, true>(p, stream);
  if constexpr (NIT <= 8) return two ? gemv_launch<2, NIT, 2, false>(p, stream) : gemv_launch<1, NIT, 2, false>(p, stream);
  return two ? gemv_launch<2, NIT, 1, false>(p, stream) : gemv_launch<1, NIT, 1, false>(p, stream);
}

template <int NIT, int RB, bool ONE>
hipError_t qkv_launch_rb(const QkvParams &p, hipStream_t stream) {
  const int pairs = (p.num_heads + 2 * p.num_kv_heads) * (kHeadDim / 2) + p.num_heads / 2;
  const dim3 grid((pairs + 3) / 4);
  if (p.w_norm != nullptr)
    hipLaunchKernelGGL((qkv_rope_kernel<NIT, RB, true, ONE>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((qkv_rope_kernel<NIT, RB, false, ONE>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// batch 1: no loop; then two batch rows per pass while their x fits (NIT <= 8)
template <int NIT>
hipError_t qkv_launch(const QkvParams &p, hipStream_t stream) {
  if (p.batch == 1) return qkv_launch_rb<NIT, 1, true>(p, stream);
  if constexpr (NIT <= 8) return qkv_launch_rb<NIT, 2, false>(p, stream);
  return qkv_launch_rb<NIT, 1, false>(p, stream);
}

// ---------------------------------------------------------------------------
// The whole block for one sequence in one launch.
//
// Run as separate launches, each step of the block pays a dispatch ramp
// (workgroups start over several microseconds, XCD by XCD) and a tail in
// which finished CUs idle, and a 31 MB projection launch on its own cannot
// fill the memory pipeline.  block_fused_kernel runs the steps as one task
// list in one persistent launch of one workgroup per CU:
//   projection tasks  4 * P RoPE pairs each (P per wave), grouped by KV head
//                     (its 4 query heads, then its k and v heads), then the
//                     gate rows; each pair computed as qkv_rope_kernel does
//   attention tasks   (chunk, KV head), chunk-major: attn_partial_wave and
//                     the 4-wave merge of attn_partial_kernel, one partial
//                     per query head
//   merge tasks       (query head, quarter of its elements): the chunks'
//                     partials merged in a fixed order, the sigmoid gate and
//                     any sink applied, written to a
//   o_proj tasks      4 * RW rows of W_o, each row computed as
//                     gemv_bf16_kernel does (y = W_o a, or y += for the layer)
// Workgroup b takes the tasks b, b + G, b + 2G, ... of each phase in phase
// order (the merge tasks on the last workgroups, which have no o_proj task).
// A task waits only for tasks of earlier phases: an attention task for the
// projections of its KV head group, a merge task for the attention of its
// group and the gate rows, an o_proj task for every merge.  The workgroup
// holding the lowest unfinished task never waits on an unfinished one, so
// the launch always progresses while its workgroups are resident (one per
// CU, at most the CU count).  Before it waits, an attention task issues its
// first K/V tiles (except the chunk holding this token's row) and an o_proj
// task its rows of W_o, so one phase's end overlaps the next one's start.
//
// Values that cross workgroups (q, gate logits, this token's cache row,
// partials, a) are stored and loaded device-coherently (the sc1 scope bit),
// per access, instead of writing back and invalidating whole caches.  A task
// marks itself done by storing the call's flag value in its own flag word
// once its waves' stores have completed; waiting is polling those words.
// The flag value is derived from an epoch word that every workgroup reads at
// its start and that the last task of the list (which follows, through its
// waits, the first task of every workgroup) advances, so flags need no
// clearing and arbitrary initial workspace contents match a flag only with
// probability 2^-64 per word.  Every value is computed by the code, and in
// the order, of the step kernels: the block's output is bit-identical to its
// steps' and the same on every run.
//
// Workspace words (64-bit): [0] epoch, then one flag per projection task,
// per attention task, per merge task, per o_proj task, and per KV head group
// a merged flag and a counter, each flag in a 128-byte line of its own: flags
// that shared lines (several writers, and every poller reading the line)
// measured 4% slower over a 36-layer stack.
// ---------------------------------------------------------------------------
constexpr int kFlagStride = 16;   // 64-bit words per flag (128 bytes)
// flags: projection tasks (at most 800), attention tasks (256 chunks x 8 KV
// heads), merge tasks (32 query heads x 4), o_proj tasks (4096 rows / 16),
// group flags and counters (8 KV heads each), attention tasks' first tiles
// issued (at most 256: only when they run beside the o_proj workgroups),
// after the epoch's line
static_assert((1 + 800 + kFusedMaxChunks * 8 + 32 * 4 + kFusedMaxHidden / 16 + 2 * 8 + 256) * kFlagStride * 8 <=
                  kSyncBytes,
              "flag words fit their bytes");
// A wait gives up after this many polls (about a second): reached only if
// calls overlap on one workspace, or if other work holds CUs the launch
// needs; the kernel then still ends.
constexpr int kSpinLimit = 1 << 20;
constexpr int kPairsPerGroup = (kGroup + 2) * (kHeadDim / 2);   // 4 q heads, k, v: 768 pairs
constexpr int kFusedRowsPerWave = 32 / (kFusedMaxQDim / 512);   // o_proj rows per wave (4)

__device__ __forceinline__ unsigned long long flag_value(unsigned long long epoch) {
  return epoch * 0x9E3779B97F4A7C15ull ^ 0xD1B54A32D192ED03ull;
}

// Flag i of the array starting at f.
__device__ __forceinline__ unsigned long long *flag_at(unsigned long long *f, int i) { return f + i * kFlagStride; }

// Wave 0 polls flags first + k * stride (flag indices), k < count, until
// every one holds fv; then the workgroup continues.  Every wave must call it.
// A poll reads up to 4 flags per lane with one round trip.
__device__ __forceinline__ void await_flags(const unsigned long long *flags, int first, int count, int stride,
                                            unsigned long long fv) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int i = 0; i < kSpinLimit; ++i) {
      bool done = true;
      for (int k0 = 0; k0 < count; k0 += 256) {
        // only the 64-flag slots that hold flags are read (a uniform
        // branch), all before the first wait; lanes past the end read a flag
        // of their own slot again
        const int nj = min(4, (count - k0 + 63) >> 6);
        unsigned long long v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = fv;
          if (j < nj) {
            const int base = k0 + 64 * j;
            const int k = base + lane % min(64, count - base);
            v[j] = __hip_atomic_load(flags + (first + k * stride) * kFlagStride, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) done &= v[j] == fv;
      }
      if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// The task's stores have completed in every wave; then its flag is set.
__device__ __forceinline__ void set_flag(unsigned long long *flag, unsigned long long fv) {
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, fv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave's four 8 KB tile buffers, addressed as 1 KB blocks 0 .. 31.
struct WaveBufs {
  _Float16 *b[4];
  __device__ __forceinline__ _Float16 *block(int m) const { return b[m >> 3] + (m & 7) * 512; }
};

// Output pair j of wave w in projection task i: pairs in group-major order
// (per KV head group: its 4 query heads, then its k and v heads).
template <int P>
__device__ __forceinline__ PairRows task_pair(const FusedParams &p, int i, int w, int j) {
  const int u = (i * 4 + w) * P + j;   // wave-uniform, < Hk * kPairsPerGroup
  const int g = u / kPairsPerGroup, r = u - g * kPairsPerGroup;
  int sec, head, pi;
  if (r < kGroup * 128) {
    sec = 0; head = g * kGroup + (r >> 7); pi = r & 127;
  } else if (r < (kGroup + 1) * 128) {
    sec = 1; head = g; pi = r - kGroup * 128;
  } else {
    sec = 2; head = g; pi = r - (kGroup + 1) * 128;
  }
  return pair_rows(sec, head, pi, p.num_heads, p.num_kv_heads, p.rotary_dim);
}

// A copy of an LDS value that every lane holds alike, in scalar registers
// (read word by word with readfirstlane, so that pointers and sizes built
// from it stay wave-uniform).
template <typename T>
__device__ __forceinline__ T lds_uniform(const T &src) {
  static_assert(sizeof(T) % 4 == 0, "whole words");
  uint32_t wd[sizeof(T) / 4];
  __builtin_memcpy(wd, &src, sizeof(T));
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) wd[i] = __builtin_amdgcn_readfirstlane(wd[i]);
  T r;
  __builtin_memcpy(&r, wd, sizeof(T));
  return r;
}

// The weight rows of wave w's pairs in projection task i, from HBM straight
// into LDS (buffer_load ... lds) in sw: row 2j (A) and 2j + 1 (B) of pair j
// in blocks (2j + ab) NIT + it, block it of a row holding columns
// (it * 64 + lane) * 8 .. +7 at 16 B * lane, the layout the task's register
// loads have.  Columns past the row read as zeros (out-of-range offsets).
// The loads complete in the wave's vector-memory count; the task waits for
// them before reading sw.
template <int NIT, int P>
__device__ __forceinline__ void fused_qkv_prefetch(const FusedParams &p, int i, const WaveBufs &sw, int lane, int w) {
  const unsigned row_bytes = (unsigned)p.hidden * 2u;
  const int qkv_rows = (p.num_heads + 2 * p.num_kv_heads) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.w_qkv, (unsigned)qkv_rows * row_bytes);
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const PairRows pr = task_pair<P>(p, i, w, j);
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) {
      const unsigned row = (unsigned)(pr.base_row + (ab ? pr.dB : pr.dA));
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int col = (it * 64 + lane) * 8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (lds_void_t *)sw.block((2 * j + ab) * NIT + it), 16,
            col < p.hidden ? row * row_bytes + (unsigned)col * 2u : kOutOfRange, 0, 0, kWeightPolicy);
      }
    }
  }
}

// Projection task i: pairs [4 P i, 4 P (i + 1)) of q_k_v_proj in group-major
// order, P per wave (the gate rows are computed by the merge tasks).  x is
// staged in LDS by the workgroup's first projection task (of the layer).  In
// a stack (STACK) x is h as the previous layer left it: the weight loads go
// out first, then wait_h() waits for that layer's o_proj, then x is read
// coherently.  LDSW: the weights were put in LDS at sw by fused_qkv_prefetch
// (this wave's rows) and are read from there.
template <int NIT, bool NORM, int P, bool STACK = false, bool LDSW = false, typename WaitH = NoWait>
__device__ __forceinline__ void fused_qkv_task(const FusedParams &p, int i, bool staged,
                                               float4 (*s_x)[StagedX<NIT>::kSlots], float *s_ss, int lane, int w,
                                               WaitH wait_h = WaitH(), const WaveBufs *sw = nullptr,
                                               const float2 *rot = nullptr) {
  const int Hk = p.num_kv_heads;
  const unsigned row_bytes = (unsigned)p.hidden * 2u;
  const int qkv_rows = (p.num_heads + 2 * Hk) * kHeadDim;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.w_qkv, (unsigned)qkv_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (unsigned)p.hidden * 4u);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(NORM ? p.w_norm : nullptr, NORM ? (unsigned)p.hidden * 2u : 0u);
  StagedX<NIT> xs;
  if (!STACK && !staged) xs.template issue<NORM>(rx, 0u, rn);
  PairRows pr[P];
  uint4 wa[P][NIT], wb[P][NIT];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    pr[j] = task_pair<P>(p, i, w, j);
    if constexpr (!LDSW) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int col = (it * 64 + lane) * 8;
        const bool ok = col < p.hidden;
        wa[j][it] = buf_load16_p<kWeightPolicy>(
            rq, ok ? (unsigned)(pr[j].base_row + pr[j].dA) * row_bytes + (unsigned)col * 2u : kOutOfRange);
        wb[j][it] = buf_load16_p<kWeightPolicy>(
            rq, ok ? (unsigned)(pr[j].base_row + pr[j].dB) * row_bytes + (unsigned)col * 2u : kOutOfRange);
      }
    }
  }
  // the rotations, while the loads are in flight (rot: this wave's, formed
  // at the start of the launch)
  float sn[P], cs[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    sn[j] = 0.f;
    cs[j] = 1.f;
    if (rot) {
      sn[j] = rot[j].x;
      cs[j] = rot[j].y;
    } else if (pr[j].rotate) {
      rope_sincos(p.seq.position, pr[j].pi, p.rotary_dim, p.log2_theta, sn[j], cs[j]);
    }
  }
  if constexpr (STACK) {
    // (the empty asm keeps the rotations here, ahead of the wait, instead of
    // being moved to their use after it)
#pragma unroll
    for (int j = 0; j < P; ++j) asm volatile("" : "+v"(sn[j]), "+v"(cs[j]));
    wait_h();
    if (!staged) xs.template issue<NORM, kCoherent>(rx, 0u, rn);
  }
  if (!staged) {
    const float ss = wave_sum(xs.template store_split<NORM>(s_x));
    if (NORM && lane == 0) s_ss[w] = ss;
    __syncthreads();
  }
  // x into registers once for all P pairs (each LDS read's latency is
  // exposed: one wave per SIMD)
  float4 x0[NIT], x1[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    x0[it] = s_x[0][it * 64 + lane];
    x1[it] = s_x[1][it * 64 + lane];
  }
  if constexpr (LDSW) {
    vm_wait<0>();   // this wave's prefetched rows are in LDS
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        wa[j][it] = *reinterpret_cast<const uint4 *>(sw->block((2 * j) * NIT + it) + lane * 8);
        wb[j][it] = *reinterpret_cast<const uint4 *>(sw->block((2 * j + 1) * NIT + it) + lane * 8);
      }
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    float ya, yb;
    pair_dots_x<NIT, NORM>(wa[j], wb[j], x0, x1, s_ss, p.hidden, p.rms_eps, ya, yb);
    if (lane == 0) pair_store<true>(p.q, p.gate, p.seq, Hk, pr[j], sn[j], cs[j], ya, yb);
  }
}

// The gated attention a as the one-launch blocks with o_proj keep it: per
// 8-dim group g of a head, the 8 bf16 high parts and then the 8 bf16 low
// parts (value - high) of dims 8g .. 8g+7, i.e. the split that
// StagedX::store_split makes of an fp32 a, so that o_proj reads its x as its
// step kernel stages it.  Written coherently (o_proj runs in the same launch).
__device__ __forceinline__ void store_a_split(float *head, int d, float v) {
  asm volatile("" : "+v"(v));  // v is final: keep the product that formed it out of v - hi
  const uint32_t hi = pack_bf16(v, 0.f) & 0xFFFFu;
  const uint32_t lo = pack_bf16(v - bf16_lo(hi), 0.f) & 0xFFFFu;
  uint16_t *g = reinterpret_cast<uint16_t *>(head) + (d >> 3) * 16 + (d & 7);
  __hip_atomic_store(g, (uint16_t)hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(g + 8, (uint16_t)lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (the empty asm makes v opaque: without it the product that formed v can be
// contracted with v - hi into one fma, whose low part then differs from the
// split of the rounded fp32 value)
template <bool SPLIT>
__device__ __forceinline__ void store_a(float *head, int d, float v) {
  if constexpr (SPLIT)
    store_a_split(head, d, v);
  else
    store_f32<true>(head + d, v);
}

// Merge task (query head h, elements 64 qd .. 64 qd + 63 of its partials):
// the chunks merged in a fixed order, gated, written to a.  Lane c of every
// wave takes chunks c, c + 64, ... for the reference max and the sum; thread
// (cg, eq) sums elements 4 eq .. +3 of chunks cg, cg + 16, ..., and the 16
// chunk groups are added in order.  The partials were written in this
// launch: they are read coherently, and a is written so.  gl is the head's
// gate logit.
template <bool SPLIT>
__device__ __forceinline__ void fused_merge_task(const FusedParams &p, int h, int qd, float gl, float2 *s_ml,
                                                 float4 *s_acc, int tid, int lane) {
  const int Hq = p.num_heads;
  const int nch = p.nchunks;
  const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.part_ml, (unsigned)nch * Hq * 8u);
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(p.part_o, (unsigned)nch * Hq * kHeadDim * 4u);
  const int eq = tid & 15, cg = tid >> 4;
  const unsigned po = ((unsigned)h * kHeadDim + 64u * qd + 4u * eq) * 4u;
  // partials of chunks c0 + 16 k, k < 4 (out of range past the last chunk)
  auto load_group = [&](int c0, float4 (&v)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 16 * k;
      v[k] = __builtin_bit_cast(float4, buf_load16_p<kCoherent>(rpo, c < nch ? po + (unsigned)c * Hq * kHeadDim * 4u
                                                                              : kOutOfRange));
    }
  };
  // the first chunk group's partials go out with the (m, l) loads: one round trip
  float4 v0[4];
  load_group(cg, v0);
  for (int c = tid; c < nch; c += kThreads)
    s_ml[c] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rml, ((unsigned)c * Hq + h) * 8u, 0,
                                                                              kCoherent));
  __syncthreads();
  float m = -INFINITY;
  for (int c = lane; c < nch; c += 64) m = fmaxf(m, s_ml[c].x);
  const float M = wave_max(m);
  float l = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const float2 ml = s_ml[c];
    l = fmaf(ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M), ml.y, l);
  }
  const float L = wave_sum(l);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = cg; c0 < nch; c0 += 4 * 16) {
    float4 v[4];
    float wc[4];
    if (c0 == cg) {
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = v0[k];
    } else {
      load_group(c0, v);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 16 * k;
      const float mc = c < nch ? s_ml[c].x : -INFINITY;
      wc[k] = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc.x = fmaf(wc[k], v[k].x, acc.x);
      acc.y = fmaf(wc[k], v[k].y, acc.y);
      acc.z = fmaf(wc[k], v[k].z, acc.z);
      acc.w = fmaf(wc[k], v[k].w, acc.w);
    }
  }
  s_acc[cg * 16 + eq] = acc;
  __syncthreads();
  if (tid < 16) {
    float4 tot = s_acc[tid];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      const float4 t = s_acc[k * 16 + tid];
      tot.x += t.x;
      tot.y += t.y;
      tot.z += t.z;
      tot.w += t.w;
    }
    const float sc = (1.0f / (1.0f + expf(-gl))) / (L + sink_term(p.sinks, h, M));
    const float v[4] = {tot.x, tot.y, tot.z, tot.w};
    float *dst = p.a + (size_t)h * kHeadDim;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 64 * qd + 4 * tid + j;             // element e holds dim 16 (e % 16) + e / 16
      store_a<SPLIT>(dst, 16 * (e & 15) + (e >> 4), v[j] * sc);
    }
  }
}

// A layer whose chunks are few (at most kGroupMergeMaxChunks) has no merge
// tasks: the attention task of a KV head group that finishes last (a counter
// per group, cleared by the group's first projection task, tells it) merges
// the group's 4 query heads itself and sets one flag per group for o_proj.
// Each of its waves takes one query head (lane l: elements 4l .. 4l+3 of the
// partial layout) with the arithmetic of fused_merge_task, operation for
// operation (chunk group cg adds chunks cg, cg + 16, ... in an fmaf chain, a
// chunk past the end counting as weight 0 times 0; the 16 groups are added
// in order), so the result is the same to the bit.
constexpr int kGroupMergeMaxChunks = 16;

// The g_proj row pair of query head h in every lane of the calling wave
// (issued ahead of the attention task's tiles, finished on x staged in LDS).
template <int NIT, bool NORM>
struct GateWave {
  uint4 wa[NIT], wb[NIT];
  __device__ __forceinline__ void issue(const FusedParams &p, int h, int lane) {
    const unsigned row_bytes = (unsigned)p.hidden * 2u;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.w_g, (unsigned)p.num_heads * row_bytes);
    const int r = h & ~1;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int col = (it * 64 + lane) * 8;
      const bool ok = col < p.hidden;
      wa[it] = buf_load16_p<kWeightPolicy>(rg, ok ? (unsigned)r * row_bytes + (unsigned)col * 2u : kOutOfRange);
      wb[it] = buf_load16_p<kWeightPolicy>(rg, ok ? (unsigned)(r + 1) * row_bytes + (unsigned)col * 2u : kOutOfRange);
    }
  }
  __device__ __forceinline__ float finish(const FusedParams &p, int h, float4 (*s_x)[StagedX<NIT>::kSlots],
                                          const float *s_ss, int lane) {
    float ya, yb;
    pair_dots<NIT, NORM>(wa, wb, s_x[0], s_x[1], s_ss, p.hidden, p.rms_eps, lane, ya, yb);
    return (h & 1) ? yb : ya;
  }
};

// The last attention task of KV head group g merges its query heads (wave w:
// head g * 4 + w, gate logit gl); a is written coherently, in the split form.
__device__ __forceinline__ void fused_group_merge(const FusedParams &p, int g, int w, int lane, float gl) {
  const int Hq = p.num_heads;
  const int nch = p.nchunks;   // <= kGroupMergeMaxChunks
  const int h = g * kGroup + w;
  const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.part_ml, (unsigned)nch * Hq * 8u);
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(p.part_o, (unsigned)nch * Hq * kHeadDim * 4u);
  // (m, l) of chunk c in lane c; the partials of every chunk, one round trip
  const float2 ml = __builtin_bit_cast(
      float2, __builtin_amdgcn_raw_buffer_load_b64(rml, lane < nch ? ((unsigned)lane * Hq + h) * 8u : kOutOfRange, 0,
                                                   kCoherent));
  float4 v[kGroupMergeMaxChunks];
  const unsigned po = ((unsigned)h * kHeadDim + 4u * lane) * 4u;
#pragma unroll
  for (int c = 0; c < kGroupMergeMaxChunks; ++c)
    v[c] = __builtin_bit_cast(
        float4, buf_load16_p<kCoherent>(rpo, c < nch ? po + (unsigned)c * Hq * kHeadDim * 4u : kOutOfRange));
  const float M = wave_max(lane < nch ? ml.x : -INFINITY);
  const float mc = lane < nch ? ml.x : -INFINITY;
  const float wl = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);   // chunk lane's weight
  const float L = wave_sum(lane < nch ? fmaf(wl, ml.y, 0.f) : 0.f);
  float4 tot = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int cg = 0; cg < 16; ++cg) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (cg < nch) {
      const float wc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), cg));
      acc.x = fmaf(wc, v[cg].x, acc.x);
      acc.y = fmaf(wc, v[cg].y, acc.y);
      acc.z = fmaf(wc, v[cg].z, acc.z);
      acc.w = fmaf(wc, v[cg].w, acc.w);
#pragma unroll
      for (int k = 1; k < 4; ++k) {   // chunks cg + 16 k are past the end: weight 0 times 0
        acc.x = fmaf(0.f, 0.f, acc.x);
        acc.y = fmaf(0.f, 0.f, acc.y);
        acc.z = fmaf(0.f, 0.f, acc.z);
        acc.w = fmaf(0.f, 0.f, acc.w);
      }
    }
    if (cg == 0) {
      tot = acc;
    } else {
      tot.x += acc.x;
      tot.y += acc.y;
      tot.z += acc.z;
      tot.w += acc.w;
    }
  }
  const float sc = (1.0f / (1.0f + expf(-gl))) / (L + sink_term(p.sinks, h, M));
  const float vv[4] = {tot.x, tot.y, tot.z, tot.w};
  float *dst = p.a + (size_t)h * kHeadDim;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * lane + j;   // element e holds dim 16 (e % 16) + e / 16
    store_a<true>(dst, 16 * (e & 15) + (e >> 4), vv[j] * sc);
  }
}

// The gate logit of query head h, computed by wave 0 as qkv_rope_kernel
// computes g_proj's row pair (h / 2): x staged in LDS by the whole workgroup
// (sum of squares for NORM as well), the two dot products over the wave.
// The weight and x loads are issued by gate_issue before the merge task
// waits; gate_finish stages x and returns the logit in every lane of wave 0.
template <int NIT, bool NORM>
struct GateRows {
  StagedX<NIT> xs;
  uint4 wa[NIT], wb[NIT];
  template <int XPOL = 0>
  __device__ __forceinline__ void issue(const FusedParams &p, int h, int lane) {
    const unsigned row_bytes = (unsigned)p.hidden * 2u;
    xs.template issue<NORM, XPOL>(make_rsrc(p.x, (unsigned)p.hidden * 4u), 0u,
                                  make_rsrc(NORM ? p.w_norm : nullptr, NORM ? (unsigned)p.hidden * 2u : 0u));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.w_g, (unsigned)p.num_heads * row_bytes);
    const int r = h & ~1;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int col = (it * 64 + lane) * 8;
      const bool ok = threadIdx.x < 64 && col < p.hidden;
      wa[it] = buf_load16_p<kWeightPolicy>(rg, ok ? (unsigned)r * row_bytes + (unsigned)col * 2u : kOutOfRange);
      wb[it] = buf_load16_p<kWeightPolicy>(rg, ok ? (unsigned)(r + 1) * row_bytes + (unsigned)col * 2u : kOutOfRange);
    }
  }
  __device__ __forceinline__ float finish(const FusedParams &p, int h, float4 (*s_x)[StagedX<NIT>::kSlots],
                                          float *s_ss, int lane, int w) {
    const float ss = wave_sum(xs.template store_split<NORM>(s_x));
    if (NORM && lane == 0) s_ss[w] = ss;
    __syncthreads();
    float ya = 0.f, yb = 0.f;
    if (w == 0) pair_dots<NIT, NORM>(wa, wb, s_x[0], s_x[1], s_ss, p.hidden, p.rms_eps, lane, ya, yb);
    return (h & 1) ? yb : ya;
  }
};

// The tasks of one launch: one layer (block_fused_kernel) or, with STACK,
// the layers of a stack in order (stack_fused_kernel; sp its StackParams).
// Layer l's flags hold the value derived from (epoch, l), so a word still
// holding an earlier layer's value never satisfies a wait.  In a stack, x and
// y are both h: a projection task and a merge task (its gate row reads h)
// wait for every o_proj task of the previous layer before they read h, and
// an o_proj task reads and writes its rows of h coherently and then sets its
// flag.  Every task of a layer is awaited, directly or through later tasks of
// the layer, by the layer's o_proj tasks, and those by the next layer's
// projections, so a word is rewritten only after every wait on it has ended.
template <int NIT, bool NORM, bool STACK, bool HAS_QKV, bool GM, typename SP>
__device__ __forceinline__ void fused_run(const FusedParams &p0, const SP &sp) {
  constexpr int W = kThreads / 64;
  constexpr int P = fused_pairs_per_wave(NIT);
  constexpr int NITO = kFusedMaxQDim / 512;
  constexpr int RW = kFusedRowsPerWave;
  static_assert(kPairsPerGroup % (W * P) == 0, "a projection task stays inside one KV head group");
  // the attention's staged tiles: K (two buffers) and V (two buffers), per
  // wave (four arrays, so that the compiler can tell a buffer's loads from
  // another's)
  __shared__ __attribute__((aligned(1024))) _Float16 s_k0[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_k1[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_v0[W][kTileHalves];
  __shared__ __attribute__((aligned(1024))) _Float16 s_v1[W][kTileHalves];
  __shared__ __attribute__((aligned(16))) _Float16 s_q[W][2 * kGroup * kHeadDim];
  __shared__ float s_ss[W];
  __shared__ float s_gate;
  __shared__ float s_gate4[4];
  __shared__ int s_last;
  __shared__ unsigned long long s_epoch;
  // a stack's per-layer pointers and shapes, and per shape the rotations of
  // each wave's pairs in the workgroup's first projection task
  __shared__ StackTables s_tab;
  __shared__ float2 s_rot[kStackMaxDescs][W][P];
  using XS = StagedX<NIT>;
  static_assert(2 * XS::kSlots * sizeof(float4) <= sizeof(s_k0) && 2 * XS::kSlots * sizeof(float4) <= sizeof(s_q),
                "staged x fits the first K buffers and the q staging");
  static_assert(kFusedMaxChunks * sizeof(float2) <= sizeof(s_v0) && 256 * sizeof(float4) <= sizeof(s_v1),
                "merge scratch fits the V buffers");
  // x (projection tasks) is staged in the q staging area (in a stack the
  // tile buffers hold the next projection task's weights meanwhile; x stays
  // there until the attention task builds its q fragments), the merge
  // scratch is in the V buffers: a workgroup's tasks come in phase order
  float4 (*s_x)[XS::kSlots] = reinterpret_cast<float4 (*)[XS::kSlots]>(&s_q[0][0]);
  float2 *s_ml = reinterpret_cast<float2 *>(&s_v0[0][0]);
  float4 *s_acc = reinterpret_cast<float4 *>(&s_v1[0][0]);
  // In a stack the weight rows of the workgroup's first projection task of
  // the next layer are loaded into the tile buffers as soon as the workgroup
  // is done with LDS for this layer (before its o_proj task), so that they
  // stream while this layer finishes: 2 P rows of H bf16 per wave, in 1 KB
  // blocks over the wave's four 8 KB tile buffers.
  constexpr bool PF = STACK && 2 * P * NIT <= 4 * (int)(sizeof(s_k0[0]) / 1024);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WaveBufs s_w{s_k0[w], s_k1[w], s_v0[w], s_v1[w]};   // this wave's prefetched rows
  const int Hq = p0.num_heads, Hk = p0.num_kv_heads;
  const int G = gridDim.x, b = blockIdx.x;
  int t_attn_slots = p0.t_attn;
  int num_layers = 1;
  if constexpr (STACK) {
    t_attn_slots = sp.t_attn_max;
    num_layers = sp.num_layers;
  }
  unsigned long long *const words = p0.sync;
  unsigned long long *const f_qkv = words + kFlagStride;   // flag i at f_qkv + i * kFlagStride (flag_at)
  unsigned long long *const f_attn = flag_at(f_qkv, p0.t_qkv);
  unsigned long long *const f_merge = flag_at(f_attn, t_attn_slots);
  unsigned long long *const f_oproj = flag_at(f_merge, p0.t_merge);
  unsigned long long *const f_group = flag_at(f_oproj, p0.t_oproj);   // per KV head group: merged (no merge tasks)
  unsigned long long *const g_count = flag_at(f_group, 8);             // per KV head group: attention tasks done
  unsigned long long *const f_tiles = flag_at(g_count, 8);             // per attention task: first tiles issued
  constexpr bool has_qkv = HAS_QKV;   // the projections run in this launch (t_qkv > 0)

  if (tid == 0) s_epoch = __hip_atomic_load(words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (STACK) {
    const uint32_t *src = reinterpret_cast<const uint32_t *>(&sp.tab);
    uint32_t *dst = reinterpret_cast<uint32_t *>(&s_tab);
    for (int i = tid; i < (int)(sizeof(StackTables) / 4); i += kThreads) dst[i] = src[i];
  }
  __syncthreads();
  const unsigned long long epoch = s_epoch;
  // the last task of the list advances the epoch for the next call
  const bool last_is_oproj = p0.t_oproj > 0;
  auto advance_epoch = [&]() {
    if (tid == 0) __hip_atomic_store(words, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // layer l's parameters (a stack's layers differ in weights, cache and shape)
  auto layer_params = [&](int l) {
    FusedParams p = p0;
    if constexpr (STACK) {
      const StackDesc d = lds_uniform(s_tab.desc[__builtin_amdgcn_readfirstlane((int)s_tab.desc_of[l])]);
      p.w_norm = lds_uniform(s_tab.w_norm[l]);
      p.w_qkv = lds_uniform(s_tab.w_qkv[l]);
      p.w_g = lds_uniform(s_tab.w_g[l]);
      p.w_o = lds_uniform(s_tab.w_o[l]);
      p.sinks = lds_uniform(s_tab.sinks[l]);
      p.seq = d.seq;
      p.seq.k = lds_uniform(s_tab.k[l]);
      p.seq.v = lds_uniform(s_tab.v[l]);
      p.chunk = d.chunk;
      p.nchunks = d.nchunks;
      p.t_attn = d.t_attn;
      p.rotary_dim = d.rotary_dim;
      p.log2_theta = d.log2_theta;
    }
    return p;
  };
  bool pf_ready = false;   // this workgroup's next projection task has its weights in LDS
  if constexpr (PF) {
    if (b < p0.t_qkv) {
      fused_qkv_prefetch<NIT, P>(layer_params(0), b, s_w, lane, w);
      pf_ready = true;
    }
  }
  if constexpr (STACK) {
    // the rotations of the workgroup's first projection task, per shape (the
    // same in every layer of that shape), while the first weights stream in
    if (b < p0.t_qkv) {
      for (int d = 0; d < sp.num_descs; ++d) {
        const StackDesc dd = lds_uniform(s_tab.desc[d]);
        FusedParams pd = p0;
        pd.rotary_dim = dd.rotary_dim;
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const PairRows pr = task_pair<P>(pd, b, w, j);
          float sn = 0.f, cs = 1.f;
          if (pr.rotate) rope_sincos(dd.seq.position, pr.pi, dd.rotary_dim, dd.log2_theta, sn, cs);
          if (lane == 0) s_rot[d][w][j] = make_float2(sn, cs);
        }
      }
    }
  }

  for (int l = 0; l < num_layers; ++l) {
    const FusedParams p = layer_params(l);
    const float2 *rot_l = nullptr;   // this layer's shape's rotations (first projection task)
    if constexpr (STACK) rot_l = &s_rot[__builtin_amdgcn_readfirstlane((int)s_tab.desc_of[l])][w][0];
    const unsigned long long fv = flag_value((epoch << 8) | (unsigned)l);
    // h as the previous layer of the stack leaves it
    auto wait_h = [&]() {
      if (STACK && l > 0) await_flags(f_oproj, 0, p.t_oproj, 1, flag_value((epoch << 8) | (unsigned)(l - 1)));
    };

    // A layer with few chunks merges in its last attention task per group.
    // Every workgroup then runs a projection task first (there are at least
    // as many as workgroups) and at most one attention task, so x is still
    // staged when its attention task starts.
    const bool group_merge =
        GM && has_qkv && p.t_oproj > 0 && p.nchunks <= kGroupMergeMaxChunks && p.t_qkv >= G && p.t_attn <= G;
    const int t_merge = group_merge ? 0 : p.t_merge;

    // this workgroup's attention task (see below) and merge task, if any
    const int a_off = p.t_oproj + p.t_attn + t_merge <= G ? p.t_oproj : 0;
    // in a stack, attention tasks beside the o_proj workgroups announce their
    // first tiles (those workgroups' prefetch waits for them)
    const bool pf_after_tiles = PF && a_off > 0 && p.t_attn <= 256;
    const int t_a0 = (b - a_off + G) % G;
    const int t_m0 = (b + t_merge) % G;
    // in a stack, a workgroup with a projection task and a merge task forms
    // the merge's gate logit right after the projection (its attention task
    // would otherwise delay it)
    const bool mgate = STACK && t_m0 < t_merge && b < p.t_qkv;

    // ---- projections ----
    bool staged = false;
    for (int t = b; t < p.t_qkv; t += G) {
      // with group_merge each wave forms the gate logit of one query head of
      // its attention task's group right after the projection task (x is
      // staged; its g_proj rows load with the task's weights)
      const bool gate_here = group_merge && t == b && t_a0 < p.t_attn;
      const bool mgate_here = mgate && t == b;
      GateWave<NIT, NORM> gate_w;
      if (gate_here) gate_w.issue(p, (t_a0 % Hk) * kGroup + w, lane);
      if (mgate_here) gate_w.issue(p, t_m0 >> 2, lane);
      if (PF && t == b && pf_ready)
        fused_qkv_task<NIT, NORM, P, STACK, PF>(p, t, staged, s_x, s_ss, lane, w, wait_h, &s_w, rot_l);
      else
        fused_qkv_task<NIT, NORM, P, STACK>(p, t, staged, s_x, s_ss, lane, w, wait_h, nullptr,
                                            t == b ? rot_l : nullptr);
      staged = true;
      // the group's first task clears its counter (every attention task of
      // the group waits for this task's flag before it counts itself)
      if (group_merge && tid == 0 && t % p.qkv_per_group == 0)
        __hip_atomic_store(flag_at(g_count, t / p.qkv_per_group), 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      set_flag(flag_at(f_qkv, t), fv);
      if (gate_here) {
        const float gv = gate_w.finish(p, (t_a0 % Hk) * kGroup + w, s_x, s_ss, lane);
        if (lane == 0) s_gate4[w] = gv;   // read after the attention task's barriers
      }
      if (mgate_here) {
        const float gv = gate_w.finish(p, t_m0 >> 2, s_x, s_ss, lane);
        if (tid == 0) s_gate = gv;   // read by the merge task (barriers in between)
      }
    }

    // ---- attention ----
    // When the attention tasks fit on the workgroups that have neither an
    // o_proj nor a merge task, they run there (task t on workgroup
    // t + t_oproj, a_off above): an o_proj workgroup then issues its W_o
    // loads right after its projection task instead of after an attention
    // task.  (A merge workgroup with an attention task would form its gate
    // logit only after it, so otherwise the tasks stay on the first
    // workgroups.)
    for (int t = t_a0; t < p.t_attn; t += G) {
      const int c = t / Hk, g = t - c * Hk;
      auto wait_q = [&]() {
        if (pf_after_tiles && tid == 0)
          __hip_atomic_store(flag_at(f_tiles, t), fv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (has_qkv) await_flags(f_qkv, g * p.qkv_per_group, p.qkv_per_group, 1, fv);
      };
      float m_run, l_run;
      if constexpr (!has_qkv)
        attn_partial_wave<W, false>(p.q, p.seq, c, p.chunk, Hk, p.qscale, g, w, s_k0[w], s_k1[w], s_v0[w], s_v1[w],
                                    s_q[w], m_run, l_run, wait_q);
      else   // the last chunk holds this token's cache row
        attn_partial_wave<W, true>(p.q, p.seq, c, p.chunk, Hk, p.qscale, g, w, s_k0[w], s_k1[w], s_v0[w], s_v1[w],
                                   s_q[w], m_run, l_run, wait_q, c == p.nchunks - 1);
      if (lane < kGroup) {
        float *ml = reinterpret_cast<float *>(s_q[w]);
        ml[lane] = m_run;
        ml[kGroup + lane] = l_run;
      }
      __syncthreads();
      float M, L;
      float4 o;
      merge_waves<W>(s_q, s_v0, w, lane, M, L, o);   // wave w: query head g * 4 + w
      const unsigned row = (unsigned)c * Hq + g * kGroup + w;
      const __amdgpu_buffer_rsrc_t rpo = make_rsrc(p.part_o, (unsigned)p.nchunks * Hq * kHeadDim * 4u);
      const __amdgpu_buffer_rsrc_t rml = make_rsrc(p.part_ml, (unsigned)p.nchunks * Hq * 8u);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), rpo, (row * kHeadDim + lane * 4) * 4u, 0,
                                             kCoherent);
      if (lane == 0)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, make_float2(M, L)), rml, row * 8u, 0,
                                              kCoherent);
      if (group_merge) {
        // the partial has landed; the task that counts last merges the group
        vm_wait<0>();
        __syncthreads();
        if (tid == 0)
          s_last = __hip_atomic_fetch_add(flag_at(g_count, g), 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (unsigned long long)(p.nchunks - 1);
        __syncthreads();
        if (s_last) {
          fused_group_merge(p, g, w, lane, s_gate4[w]);
          set_flag(flag_at(f_group, g), fv);
        }
      } else {
        set_flag(flag_at(f_attn, t), fv);
      }
      __syncthreads();   // s_q and s_v0 are rewritten by the next task
    }

    // ---- merge: on the last workgroups (they have no o_proj task) ----
    for (int t = (b + t_merge) % G; t < t_merge; t += G) {
      const int h = t >> 2, qd = t & 3;
      // in the one-launch block the head's gate logit is computed here,
      // before the wait for the attention (it needs only x)
      float gl;
      if (mgate && t == t_m0) {   // formed after the projection task
        gl = s_gate;
      } else if constexpr (has_qkv) {
        GateRows<NIT, NORM> gate;
        if constexpr (STACK) {
          wait_h();
          gate.template issue<kCoherent>(p, h, lane);
        } else {
          gate.issue(p, h, lane);
        }
        const float v = gate.finish(p, h, s_x, s_ss, lane, w);
        if (tid == 0) s_gate = v;   // to every wave
        __syncthreads();
        gl = s_gate;
      } else {
        gl = p.gate[h];
      }
      // the attention of this head's group: chunk c is attention task c * Hk + g.
      // Without o_proj tasks the last merge task is the list's last task and
      // waits for every attention task (so that it follows every workgroup's
      // first task) before it advances the epoch.
      const bool final_task = !last_is_oproj && t == p.t_merge - 1;
      if (final_task)
        await_flags(f_attn, 0, p.t_attn, 1, fv);
      else
        await_flags(f_attn, h / kGroup, p.nchunks, Hk, fv);
      fused_merge_task<HAS_QKV>(p, h, qd, gl, s_ml, s_acc, tid, lane);
      set_flag(flag_at(f_merge, t), fv);
      if (final_task) advance_epoch();
      __syncthreads();   // LDS is rewritten by the next task
    }
    if constexpr (PF) {
      // every LDS task of the layer has ended (each ends in a barrier).  A
      // workgroup that ran an attention task and has an o_proj task does not
      // prefetch: its W_o loads would queue behind the prefetch, and its
      // next projection task loads its weights itself.
      const bool oproj_after_attn = b < p.t_oproj && t_a0 < p.t_attn;
      pf_ready = l + 1 < num_layers && b < p.t_qkv && !oproj_after_attn;
      // an o_proj workgroup without an attention task holds its prefetch
      // until every attention task has issued its first tiles: started at
      // once, its loads slowed the issue of those tiles (the layer's
      // critical path) several times over
      if (pf_ready && pf_after_tiles && b < p.t_oproj) await_flags(f_tiles, 0, p.t_attn, 1, fv);
      if (pf_ready) fused_qkv_prefetch<NIT, P>(layer_params(l + 1), b, s_w, lane, w);
    }

    // ---- o_proj ---- (only with the projections in the launch: it reads a
    // in the split form, which only those launches' merges write)
    for (int t = b; HAS_QKV && t < p.t_oproj; t += G) {
      // rows r0 .. r0 + RW - 1 of this wave: the W_o loads go out before the wait for a
      const int r0 = (t * W + w) * RW;
      const int qdim = Hq * kHeadDim;
      const unsigned row_bytes = (unsigned)qdim * 2u;
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w_o, (unsigned)p.hidden * row_bytes);
      uint4 wv[RW][NITO];
#pragma unroll
      for (int k = 0; k < RW; ++k)
#pragma unroll
        for (int it = 0; it < NITO; ++it) {
          const int col = (it * 64 + lane) * 8;
          const int r = r0 + k;
          wv[k][it] = buf_load16_p<kWeightPolicy>(
              rw, (r < p.hidden && col < qdim) ? (unsigned)r * row_bytes + (unsigned)col * 2u : kOutOfRange);
        }
      // in a stack: this wave's RW rows of h (a multiple of 4 rows: one 16 B
      // load), which this wave itself wrote in the previous layer
      static_assert(RW == 4, "one float4 of h per wave");
      const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y, (unsigned)p.hidden * 4u);
      float4 yold = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (STACK)
        yold = __builtin_bit_cast(float4, buf_load16_p<kCoherent>(ry, r0 < p.hidden ? (unsigned)r0 * 4u : kOutOfRange));
      if (group_merge)
        await_flags(f_group, 0, Hk, 1, fv);
      else if (p.t_merge > 0)
        await_flags(f_merge, 0, p.t_merge, 1, fv);
      // a in the split form (8-dim group g: 16 B of bf16 high parts, then 16 B
      // of low parts), read as the GEMV's staged x: once per workgroup (16 B
      // per lane, coalesced) into LDS, where all four waves read it; read by
      // every wave from memory it put four times the coherent reads on the
      // same few lines.  Slots past q_dim hold zeros (out-of-range loads).
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, (unsigned)qdim * 4u);
      uint4 *s_a = reinterpret_cast<uint4 *>(&s_q[0][0]);
      static_assert(sizeof(s_q) == kFusedMaxQDim * 4, "a in the split form fills s_q");
      constexpr int kA16 = kFusedMaxQDim * 4 / 16 / kThreads;
      uint4 av[kA16];
#pragma unroll
      for (int k = 0; k < kA16; ++k) av[k] = buf_load16_p<kCoherent>(ra, (unsigned)(k * kThreads + tid) * 16u);
#pragma unroll
      for (int k = 0; k < kA16; ++k) s_a[k * kThreads + tid] = av[k];
      __syncthreads();
      float4 xa[NITO], xb[NITO];
#pragma unroll
      for (int it = 0; it < NITO; ++it) {
        xa[it] = __builtin_bit_cast(float4, s_a[(it * 64 + lane) * 2]);
        xb[it] = __builtin_bit_cast(float4, s_a[(it * 64 + lane) * 2 + 1]);
      }
      float ynew[RW];
#pragma unroll
      for (int k = 0; k < RW; ++k) {
        float acc = 0.f;
#pragma unroll
        for (int it = 0; it < NITO; ++it)
          acc = dot8_bf16_split(wv[k][it], __builtin_bit_cast(uint4, xa[it]), __builtin_bit_cast(uint4, xb[it]), acc);
        const float s = wave_sum(acc);
        const int r = r0 + k;
        if constexpr (STACK) {
          ynew[k] = (k == 0 ? yold.x : k == 1 ? yold.y : k == 2 ? yold.z : yold.w) + s;
        } else {
          if (lane == 0 && r < p.hidden) p.y[r] = p.accumulate ? p.y[r] + s : s;
        }
      }
      if constexpr (STACK) {
        if (lane == 0)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4_t, make_float4(ynew[0], ynew[1], ynew[2], ynew[3])), ry,
              r0 < p.hidden ? (unsigned)r0 * 4u : kOutOfRange, 0, kCoherent);
        set_flag(flag_at(f_oproj, t), fv);
      }
      if (l == num_layers - 1 && t == p.t_oproj - 1) advance_epoch();
    }
  }
}

// HAS_QKV: the whole block (projections in the launch); else its attention
// and merge alone, on a q and gate logits already in memory.
// GM: the launch may merge in the attention tasks (layers with few chunks);
// its code is left out of the launches that never do.
template <int NIT, bool NORM, bool HAS_QKV, bool GM>
__global__ __launch_bounds__(kThreads, 1) void block_fused_kernel(const FusedParams p) {
  fused_run<NIT, NORM, false, HAS_QKV, GM>(p, p);
}

template <int NIT>
__global__ __launch_bounds__(kThreads, 1) void stack_fused_kernel(const StackParams sp) {
  fused_run<NIT, true, true, true, true>(sp.base, sp);
}

template <int NIT>
hipError_t fused_launch(const FusedParams &p, dim3 grid, hipStream_t stream) {
  const int G = (int)grid.x;
  const bool gm = p.t_oproj > 0 && p.nchunks <= kGroupMergeMaxChunks && p.t_qkv >= G && p.t_attn <= G;
  if (p.t_qkv == 0)   // attention + merge only (no norm: x is not read)
    hipLaunchKernelGGL((block_fused_kernel<NIT, false, false, false>), grid, dim3(kThreads), 0, stream, p);
  else if (p.w_norm != nullptr && gm)
    hipLaunchKernelGGL((block_fused_kernel<NIT, true, true, true>), grid, dim3(kThreads), 0, stream, p);
  else if (p.w_norm != nullptr)
    hipLaunchKernelGGL((block_fused_kernel<NIT, true, true, false>), grid, dim3(kThreads), 0, stream, p);
  else if (gm)
    hipLaunchKernelGGL((block_fused_kernel<NIT, false, true, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((block_fused_kernel<NIT, false, true, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int NIT>
hipError_t stack_launch(const StackParams &sp, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((stack_fused_kernel<NIT>), grid, dim3(kThreads), 0, stream, sp);
  return hipGetLastError();
}

}  // namespace

// Grid of the batched projections: units rounded up to 8 (the unit -> XCD
// mapping), times the batch tiles of 16 * MB rows.
template <int MB, typename Params>
dim3 proj_grid(const Params &p) {
  const int nbt = (p.batch + 16 * MB - 1) / (16 * MB);
  return dim3((unsigned)((proj_units(p) + 7) / 8 * 8 * nbt));
}

// o_proj: one 16-row batch tile per workgroup (its 80 units at H = 2560 would
// leave most CUs idle).  q_k_v_proj: all <= 32 rows per workgroup (its 193
// units fill the chip; measured 19.9 vs 24.7 us split at batch 32).
hipError_t launch_proj_mfma(const GemvParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((proj_mfma_kernel<0, 1, false, GemvParams>), proj_grid<1>(p), dim3(kProjThreads), 0, stream,
                     p);
  return hipGetLastError();
}

hipError_t launch_qkv_mfma(const QkvParams &p, hipStream_t stream) {
  const bool norm = p.w_norm != nullptr;
  if (p.batch > 16) {
    if (norm)
      hipLaunchKernelGGL((proj_mfma_kernel<1, 2, true, QkvParams>), proj_grid<2>(p), dim3(kProjThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((proj_mfma_kernel<1, 2, false, QkvParams>), proj_grid<2>(p), dim3(kProjThreads), 0, stream,
                         p);
  } else {
    if (norm)
      hipLaunchKernelGGL((proj_mfma_kernel<1, 1, true, QkvParams>), proj_grid<1>(p), dim3(kProjThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((proj_mfma_kernel<1, 1, false, QkvParams>), proj_grid<1>(p), dim3(kProjThreads), 0, stream,
                         p);
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvParams &p, hipStream_t stream) {
  switch ((p.cols + 511) / 512) {
    case 1: return gemv_rows<1>(p, stream);
    case 2: return gemv_rows<2>(p, stream);
    case 3: return gemv_rows<3>(p, stream);
    case 4: return gemv_rows<4>(p, stream);
    case 5: return gemv_rows<5>(p, stream);
    case 6: return gemv_rows<6>(p, stream);
    case 7: return gemv_rows<7>(p, stream);
    case 8: return gemv_rows<8>(p, stream);
    case 9: case 10: return gemv_rows<10>(p, stream);
    case 11: case 12: return gemv_rows<12>(p, stream);
    default: return gemv_rows<16>(p, stream);
  }
}

hipError_t launch_qkv_rope(const QkvParams &p, hipStream_t stream) {
  switch ((p.hidden + 511) / 512) {
    case 1: return qkv_launch<1>(p, stream);
    case 2: return qkv_launch<2>(p, stream);
    case 3: return qkv_launch<3>(p, stream);
    case 4: return qkv_launch<4>(p, stream);
    case 5: return qkv_launch<5>(p, stream);
    case 6: return qkv_launch<6>(p, stream);
    case 7: return qkv_launch<7>(p, stream);
    case 8: return qkv_launch<8>(p, stream);
    case 9: case 10: return qkv_launch<10>(p, stream);
    case 11: case 12: return qkv_launch<12>(p, stream);
    default: return qkv_launch<16>(p, stream);
  }
}

void fused_tasks(FusedParams &p) {
  const int Hq = p.num_heads, Hk = p.num_kv_heads;
  const int per_task = (kThreads / 64) * fused_pairs_per_wave((p.hidden + 511) / 512);
  p.qkv_per_group = kPairsPerGroup / per_task;
  p.t_qkv = (p.phases & kPhaseQkv) ? Hk * p.qkv_per_group : 0;
  p.t_attn = (p.phases & kPhaseAttn) ? p.nchunks * Hk : 0;
  p.t_merge = (p.phases & kPhaseAttn) ? Hq * 4 : 0;
  const int rows = (kThreads / 64) * kFusedRowsPerWave;
  p.t_oproj = (p.phases & kPhaseOproj) ? (p.hidden + rows - 1) / rows : 0;
}

namespace {

// The CU count of the current device, asked once per device.
hipError_t device_cus(int *cus) {
  static int cu_count[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int n = dev >= 0 && dev < 64 ? __atomic_load_n(&cu_count[dev], __ATOMIC_RELAXED) : 0;
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) __atomic_store_n(&cu_count[dev], n, __ATOMIC_RELAXED);
  }
  *cus = n;
  return hipSuccess;
}

}  // namespace

// One workgroup per CU, and no more workgroups than the largest of the
// projection, attention and merge phases has tasks, so that every workgroup
// runs one of them (the list's last task then follows every workgroup's
// start); without o_proj tasks, no more than the attention tasks.
hipError_t launch_block_fused(const FusedParams &p, hipStream_t stream) {
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int cover = p.t_oproj > 0 ? std::max(p.t_qkv, std::max(p.t_attn, p.t_merge)) : p.t_attn;
  const dim3 grid((unsigned)std::max(1, std::min(cus, cover)));
  switch ((p.hidden + 511) / 512) {
    case 1: return fused_launch<1>(p, grid, stream);
    case 2: return fused_launch<2>(p, grid, stream);
    case 3: return fused_launch<3>(p, grid, stream);
    case 4: return fused_launch<4>(p, grid, stream);
    case 5: return fused_launch<5>(p, grid, stream);
    case 6: return fused_launch<6>(p, grid, stream);
    case 7: return fused_launch<7>(p, grid, stream);
    default: return fused_launch<8>(p, grid, stream);
  }
}

// As the block: one workgroup per CU, at most the largest phase of any layer.
hipError_t launch_stack_fused(const StackParams &sp, hipStream_t stream) {
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const FusedParams &p = sp.base;
  const int cover = std::max(p.t_qkv, std::max(sp.t_attn_max, p.t_merge));
  const dim3 grid((unsigned)std::max(1, std::min(cus, cover)));
  switch ((p.hidden + 511) / 512) {
    case 1: return stack_launch<1>(sp, grid, stream);
    case 2: return stack_launch<2>(sp, grid, stream);
    case 3: return stack_launch<3>(sp, grid, stream);
    case 4: return stack_launch<4>(sp, grid, stream);
    case 5: return stack_launch<5>(sp, grid, stream);
    case 6: return stack_launch<6>(sp, grid, stream);
    case 7: return stack_launch<7>(sp, grid, stream);
    default: return stack_launch<8>(sp, grid, stream);
  }
}

// gate[i] <- gelu_erf(gate[i]) * up[i] for i < n ([mod] transcribed layer:
// the erf GELU of the gate projection times the up projection).
__global__ __launch_bounds__(kThreads) void gelu_mul_kernel(float *gate, const float *up, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float g = gate[i];
    gate[i] = 0.5f * g * (1.0f + erff(g * 0.70710678118654752f)) * up[i];
  }
}

// The MLP's first half for batch 1-3 ([mod] transcribed layer): x = rms(h) *
// w_post is staged in LDS (the sum of squares comes from the staging loads,
// summed over the workgroup), and wave i computes gate_i . x and up_i . x for
// every batch row, so it can write act[b][i] = gelu_erf(g) * u itself: the
// norm, both projections and the activation in one launch.  Weight loads are
// issued before the first FMA, as in gemv_bf16_kernel.
template <int NIT, int RB, bool ONE>
__global__ __launch_bounds__(kThreads) void mlp_gate_up_kernel(const MlpParams p) {
  __shared__ float4 s_x[RB][2][StagedX<NIT>::kSlots];
  __shared__ float s_ss[RB][kThreads / 64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * (kThreads / 64) + wv;   // intermediate index of this wave
  const unsigned row_bytes = (unsigned)p.hidden * 2u;
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.w_gate, (unsigned)p.inter * row_bytes);
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.w_up, (unsigned)p.inter * row_bytes);
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(p.w_post, row_bytes);
  auto hrow = [&](int b) {
    return make_rsrc(p.h + (size_t)b * p.hidden, b < p.batch ? (unsigned)p.hidden * 4u : 0u);
  };
  StagedX<NIT> xs[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) xs[r].template issue<true>(hrow(r), 0u, rn);
  uint4 wg[NIT], wu[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int col = (it * 64 + lane) * 8;
    const unsigned off = (i < p.inter && col < p.hidden) ? (unsigned)i * row_bytes + (unsigned)col * 2u : kOutOfRange;
    wg[it] = buf_load16_p<kWeightPolicy>(rg, off);
    wu[it] = buf_load16_p<kWeightPolicy>(ru, off);
  }
  auto emit = [&](int m, int b) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      g = dot8_bf16(wg[it], s_x[m][0][it * 64 + lane], s_x[m][1][it * 64 + lane], g);
      u = dot8_bf16(wu[it], s_x[m][0][it * 64 + lane], s_x[m][1][it * 64 + lane], u);
    }
    const float inv = rsqrtf((s_ss[m][0] + s_ss[m][1] + s_ss[m][2] + s_ss[m][3]) / (float)p.hidden + p.eps);
    g = wave_sum(g) * inv;
    u = wave_sum(u) * inv;
    if (lane == 0 && i < p.inter && b < p.batch)
      p.act[(size_t)b * p.inter + i] = 0.5f * g * (1.0f + erff(g * 0.70710678118654752f)) * u;
  };
  if constexpr (ONE) {
    const float ss = wave_sum(xs[0].template store<true>(s_x[0]));
    if (lane == 0) s_ss[0][wv] = ss;
    __syncthreads();
    emit(0, 0);
  } else {
    for (int b0 = 0; b0 < p.batch; b0 += RB) {
#pragma unroll
      for (int m = 0; m < RB; ++m) {
        const float ss = wave_sum(xs[m].template store<true>(s_x[m]));
        if (lane == 0) s_ss[m][wv] = ss;
        xs[m].template issue<true>(hrow(b0 + RB + m), 0u, rn);   // next rows, unconditional
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < RB; ++m) emit(m, b0 + m);
      if (b0 + RB < p.batch) __syncthreads();   // s_x and s_ss are rewritten for the next rows
    }
  }
}

template <int NIT>
hipError_t mlp_gate_up_nit(const MlpParams &p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.inter + 3) / 4));
  if (p.batch == 1)
    hipLaunchKernelGGL((mlp_gate_up_kernel<NIT, 1, true>), grid, dim3(kThreads), 0, stream, p);
  else if constexpr (NIT <= 8)
    hipLaunchKernelGGL((mlp_gate_up_kernel<NIT, 2, false>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((mlp_gate_up_kernel<NIT, 1, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_mlp_gate_up(const MlpParams &p, hipStream_t stream) {
  switch ((p.hidden + 511) / 512) {
    case 1: return mlp_gate_up_nit<1>(p, stream);
    case 2: return mlp_gate_up_nit<2>(p, stream);
    case 3: return mlp_gate_up_nit<3>(p, stream);
    case 4: return mlp_gate_up_nit<4>(p, stream);
    case 5: return mlp_gate_up_nit<5>(p, stream);
    case 6: return mlp_gate_up_nit<6>(p, stream);
    case 7: return mlp_gate_up_nit<7>(p, stream);
    case 8: return mlp_gate_up_nit<8>(p, stream);
    case 9: case 10: return mlp_gate_up_nit<10>(p, stream);
    case 11: case 12: return mlp_gate_up_nit<12>(p, stream);
    default: return mlp_gate_up_nit<16>(p, stream);
  }
}

hipError_t launch_gelu_mul(float *gate, const float *up, int64_t n, hipStream_t stream) {
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + kThreads - 1) / kThreads, 2048));
  hipLaunchKernelGGL(gelu_mul_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, gate, up, n);
  return hipGetLastError();
}

hipError_t launch_attention_partials(const AttnParams &p, hipStream_t stream) {
  const dim3 grid(p.total_chunks * p.num_kv_heads);
  if (p.waves == 2)
    hipLaunchKernelGGL(attn_partial_kernel<2>, grid, dim3(128), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_partial_kernel<4>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention_chunk(const ChunkAttnParams &p, hipStream_t stream) {
  const int ntg = (p.m_tokens + 15) / 16;
  const int units = p.nchunks * p.num_kv_heads;
  hipLaunchKernelGGL(attn_chunk_kernel, dim3((unsigned)((units + 7) / 8 * 8 * ntg)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams &p, int num_heads, hipStream_t stream) {
  hipError_t e = launch_attention_partials(p, stream);
  if (e != hipSuccess || p.direct) return e;
  return launch_combine(p, num_heads, stream);
}

hipError_t launch_combine(const AttnParams &p, int num_heads, hipStream_t stream) {
  int most = 0;
  for (int i = 0; i < p.nseq; ++i) most = std::max(most, (p.seq[i].n + p.chunk - 1) / p.chunk);
  if (most <= kCombineSmallChunks)
    hipLaunchKernelGGL(attn_combine_small_kernel, dim3(num_heads, p.nseq), dim3(64), 0, stream, p);
  else if (most <= kCombineMidChunks && p.nseq * num_heads >= kAttnTargetWgs)
    hipLaunchKernelGGL(attn_combine_mid_kernel, dim3(num_heads, p.nseq), dim3(kThreads), 0, stream, p);
  else
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
