// Internal definitions shared by the host side and the kernels of libgqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gqa.h"

namespace gqa {

constexpr int kHeadDim = 256;        // kernels specialise D = 256
constexpr int kGroup = 4;            // query heads per KV head
constexpr int kThreads = 256;        // 4 wave64 per workgroup
constexpr int kMaxSeqPerLaunch = 32; // sequence descriptors carried in kernel arguments
constexpr int kTileRows = 16;        // attention rows per MFMA tile
constexpr int kChunkQuantum = 4 * kTileRows;  // attention chunks: a multiple of 4 tiles (whole tiles per wave)
// Attention workgroups a launch aims for: one wave per SIMD of MI355X
// (256 CUs x 4 SIMDs, 4 waves per workgroup).  Measured on a 32K-row window:
// 1024 waves of 8 tiles finish together, while 2048 waves of 4 tiles (the two
// that fit per SIMD) spread their end times over ~10 us as HBM serves their
// first tiles in arbitrary order.  A constant (not the device's CU count) so
// the split plan, and the workspace bound derived from it, are the same
// everywhere.
constexpr int kAttnTargetWgs = 256;
// attn_partial_kernel runs workgroups of 4 waves (144 KB of LDS: one per CU)
// or, for launches of at least kNarrowMinSeqs sequences with more rows than
// a short plan, of 2 waves (72 KB: two per CU) aiming for twice the
// workgroups.  Measured (attention step, full layers, 16K rows per
// sequence): 2, 4 and 8 sequences the same either way; 12 sequences 185 us
// with 4 waves (288 workgroups on 256 CUs: a second round) against 137 us;
// 32 ragged sequences (up to 16K) 209.6 against 201.7 us for the pass.
constexpr int kNarrowMinSeqs = 2;
constexpr long kShortPlanRows = 4096;  // launches of at most this many window rows aim for half
// Workgroups the several-token path aims for: (chunk, KV head, 16 tokens)
// each, every wave walking all tiles of its chunk in sequence.  Measured on
// 32 tokens at 4K rows (whole chunk step): 128 -> 57.6 us, 256 -> 60.2 us,
// 64 -> 76.5 us, 512 -> 69.8 us: fewer, longer chains write fewer partials
// until too few workgroups are left to stream the cache.
constexpr int kChunkTargetWgs = 128;
// Windows of at most this many rows run as one chunk per sequence and KV
// head, finished inside the partial kernel (no combine launch).  Measured:
// at 64 rows this saves the combine (~3.4 us); at 512 rows the 16 waves of
// a one-chunk plan walk 8 tiles each in sequence (~14 us), slower than 8
// chunks plus the combine (~10 us).
constexpr int kDirectMaxRows = 128;
constexpr int kMfmaMinBatch = 4;     // projections run on MFMA from this batch on
constexpr float kRescaleSlack = 8.f; // log2 headroom before the softmax reference moves
constexpr unsigned kMaxBufferBytes = 0x7FFFFFFFu;  // buffer loads use 31-bit offsets
constexpr int kMaxHidden = 8192;     // GEMV keeps up to 16 x 512 columns in registers

// One sequence of one attention launch.  Window and slot are resolved on the
// host so the kernels only do integer arithmetic that is the same for every row.
struct SeqDesc {
  _Float16 *k;        // cache base, [capacity][Hk][D]
  _Float16 *v;
  int kv_start;       // first attended logical position
  int n;              // attended rows: seq_len - kv_start (>= 1)
  int ring;           // active ring size, 0 = identity addressing
  int slot;           // physical row that receives this token's k and v
  int position;       // this token's position (RoPE angle)
  int chunk_begin;    // first flat chunk index of this sequence in the launch
  unsigned cache_bytes;  // bytes of each of k and v
};

struct AttnParams {
  const float *q;     // [nseq][ld_q] RoPE'd query heads, head-major
  long ld_q;
  const float *gate;  // [nseq][ld_gate] gate logits
  long ld_gate;
  float *out;         // [nseq][ld_out] gated attention, head-major
  long ld_out;
  float *part_o;      // [total_chunks][Hq][D]   unnormalised partial outputs, element
                      // n * 16 + c of a head holding dim 16c + n
  float *part_ml;     // [total_chunks][Hq][2]   (reference max in log2 units, sum)
  const float *sinks; // [Hq] attention-sink logits (one more softmax term per query
                      // head, no value row), or null: none
  int num_kv_heads;
  float qscale;       // attention_scale * log2(e): scores come out in log2 units
  int chunk;          // rows per chunk (one workgroup per chunk and KV head, interleaved
                      // 16-row tiles per wave): a multiple of kChunkQuantum
  int direct;         // 1: every sequence is one chunk and the partial kernel writes
                      // the gated output itself (no partials, no combine)
  int waves;          // waves per workgroup of attn_partial_kernel: 4 or 2
  int nseq;
  int total_chunks;
  SeqDesc seq[kMaxSeqPerLaunch];
};

// Several tokens of one sequence (attn_chunk_kernel): token t at position
// first_pos + t attends rows [ks_t, first_pos + t], ks_t = 0 (full) or
// max(0, first_pos + t + 1 - window) (sliding).  The rows [r0, first_pos + M)
// are cut into nchunks chunks of `chunk` rows; the partial of token t, chunk
// c, query head h is row (t * nchunks + c) * Hq + h of part_o / part_ml (the
// layout attn_combine_kernel reads with one "sequence" per token).
struct ChunkAttnParams {
  const float *q;       // [M][ld_q] RoPE'd queries of the M tokens
  long ld_q;
  float *part_o;
  float *part_ml;
  int num_kv_heads;
  float qscale;         // attention_scale * log2(e)
  int m_tokens;
  int first_pos;
  int window;           // sliding window; full layers: first_pos + M (every row from 0)
  int r0;               // first attended row of token 0
  int chunk;            // rows per chunk, a multiple of 32
  int nchunks;
  SeqDesc seq;          // the cache (k, v, cache_bytes; ring = ring_capacity or 0)
};

// The fused projection step: q_k_v_proj and g_proj over the same x, then the
// split, RoPE and the fp16 KV-slot write (uses seq[].k, .v, .slot, .position).
struct QkvParams {
  const uint16_t *w_qkv;  // bf16 [(Hq + 2 Hk) * D][hidden]
  const uint16_t *w_g;    // bf16 [Hq][hidden]
  int hidden;
  int batch;              // <= kMaxSeqPerLaunch
  const float *x;         // [batch][ldx]
  long ldx;
  float *q_out;           // [batch][ld_q] RoPE'd q
  long ld_q;
  float *gate_out;        // [batch][ld_gate] gate logits
  long ld_gate;
  int num_heads;
  int num_kv_heads;
  int rotary_dim;
  double log2_theta;
  const uint16_t *w_norm; // bf16 [hidden] or null: x is then the raw residual stream h and
                          // the projections see RMSNorm(h) * w_norm (eps rms_eps)
  float rms_eps;
  SeqDesc seq[kMaxSeqPerLaunch];
};

// The block for ONE sequence as one persistent launch (block_fused_kernel):
// tasks of up to four phases run in dependency order, each marking itself
// done in a flag word of the workspace's synchronisation area.
constexpr int kPhaseQkv = 1;      // projections, split, RoPE, KV-slot write
constexpr int kPhaseAttn = 2;     // split-K attention and the merge with the gate
constexpr int kPhaseOproj = 4;    // o_proj
constexpr int kSyncBytes = 524288;  // synchronisation words at the start of the workspace (one flag per 128 B)
constexpr int kFusedMaxChunks = 256;   // chunks per sequence the merge tasks take
constexpr int kFusedMaxHidden = 4096;  // x staged in LDS beside the attention buffers
constexpr int kFusedMaxQDim = 4096;    // o_proj rows held in registers
// RoPE pairs per wave of a projection task: 3, so that the 4 x 768 pairs of
// the family's 4 KV head groups make 256 tasks, one per CU
__host__ __device__ constexpr int fused_pairs_per_wave(int) { return 3; }
struct FusedParams {
  int phases;             // kPhaseQkv | kPhaseAttn | kPhaseOproj, or kPhaseAttn alone
  // projections
  const uint16_t *w_qkv;  // bf16 [(Hq + 2 Hk) * D][hidden]
  const uint16_t *w_g;    // bf16 [Hq][hidden]
  int hidden;
  const float *x;         // [hidden]: the normed input, or (w_norm set) the residual stream h
  const uint16_t *w_norm; // bf16 [hidden] or null
  float rms_eps;
  int rotary_dim;
  double log2_theta;
  float *q;               // [Hq * D] RoPE'd q (written by the projections, read by the attention)
  float *gate;            // [Hq] gate logits
  // attention
  SeqDesc seq;            // chunk_begin 0
  int chunk;              // rows per chunk (the split-K plan's)
  int nchunks;
  float qscale;           // attention_scale * log2(e)
  const float *sinks;     // [Hq] or null
  float *part_o;          // [nchunks][Hq][D]
  float *part_ml;         // [nchunks][Hq][2]
  float *a;               // [Hq * D] gated attention (written by the merge, read by o_proj)
  // o_proj
  const uint16_t *w_o;    // bf16 [hidden][Hq * D]
  float *y;               // [hidden]
  int accumulate;         // 1: y += W_o a (the layer's residual add)
  // scheduling
  unsigned long long *sync;  // kSyncBytes of workspace
  int num_heads, num_kv_heads;
  int t_qkv, t_attn, t_merge, t_oproj;  // tasks of each phase (0 if it does not run)
  int qkv_per_group;      // projection tasks per KV head group
};

// A stack of layers for ONE sequence as one persistent launch
// (stack_fused_kernel): layer l's tasks follow layer l - 1's, the projections
// of layer l waiting for every o_proj task of layer l - 1 (h complete).  The
// layers' attention shapes (window, chunking, RoPE class) come from a small
// table of distinct descriptors, the weights and caches per layer.
constexpr int kStackMaxLayers = 40;  // layers per launch (more run as further launches)
constexpr int kStackMaxDescs = 4;    // distinct attention shapes per launch
struct StackDesc {
  SeqDesc seq;            // window and slot of the token (k and v are per layer)
  int chunk;              // rows per chunk
  int nchunks;
  int t_attn;             // attention tasks: nchunks * Hk
  int rotary_dim;
  double log2_theta;
};
// The per-layer part of a stack's arguments.  The kernel copies it into LDS
// at its start and reads each layer's pointers and shape from there: read
// from the kernel arguments at each layer's start, they cost a chain of
// dependent memory round trips on the layer's critical path.
struct StackTables {
  unsigned char desc_of[kStackMaxLayers];
  StackDesc desc[kStackMaxDescs];
  const uint16_t *w_norm[kStackMaxLayers];
  const uint16_t *w_qkv[kStackMaxLayers];
  const uint16_t *w_g[kStackMaxLayers];
  const uint16_t *w_o[kStackMaxLayers];
  _Float16 *k[kStackMaxLayers];
  _Float16 *v[kStackMaxLayers];
  const float *sinks[kStackMaxLayers];
};
static_assert(sizeof(StackTables) % 4 == 0, "the tables are copied as 32-bit words");
struct StackParams {
  FusedParams base;       // shared fields: shapes, workspace buffers, x = y = h, task counts
  int num_layers;
  int t_attn_max;         // attention flag words reserved per layer
  int num_descs;          // distinct shapes in desc (1 .. kStackMaxDescs)
  StackTables tab;
};
static_assert(sizeof(StackParams) <= 3072, "the stack's kernel arguments stay under 3 KB");

// The embedding gather: h[b] = table[ids[b]] (bf16 row -> fp32), up to
// kMaxEmbedIds tokens per launch; ids are checked on the host.
constexpr int kMaxEmbedIds = 64;
struct EmbedParams {
  const uint16_t *table;  // bf16 [vocab][hidden]
  float *h;               // [count][hidden]
  int hidden;             // a multiple of 8
  int count;
  int ids[kMaxEmbedIds];
};

// The MLP's first half for small batches: act[b][i] = gelu_erf(g) * u with
// g = gate_i . x_b, u = up_i . x_b, x_b = rms(h_b) * w_post.
struct MlpParams {
  const uint16_t *w_post;  // bf16 [hidden]
  const uint16_t *w_gate;  // bf16 [inter][hidden]
  const uint16_t *w_up;    // bf16 [inter][hidden]
  const float *h;          // [batch][hidden] residual stream
  float *act;              // [batch][inter]
  int hidden;
  int inter;
  int batch;
  float eps;
};

struct GemvParams {
  const uint16_t *w0; // bf16 [rows0][cols]
  const uint16_t *w1; // bf16 [rows1][cols], rows appended after w0's
  int rows0;
  int rows1;
  int cols;
  int batch;
  const float *x;     // [batch][ldx]
  long ldx;
  float *y0;          // [batch][ldy0] receives rows of w0
  long ldy0;
  float *y1;          // [batch][ldy1] receives rows of w1
  long ldy1;
  int accumulate;     // 1: y += W x (the residual add of the layer loop), else y = W x
};

// Launchers (gqa_kernels.hip).  They return the hipError_t of the launch.
// fused_tasks fills the task counts of p for its phases (hidden, heads, nchunks set).
void fused_tasks(FusedParams &p);
hipError_t launch_block_fused(const FusedParams &p, hipStream_t stream);
// sp.base's task counts as fused_tasks gives them (t_attn unused: per descriptor)
hipError_t launch_stack_fused(const StackParams &sp, hipStream_t stream);
hipError_t launch_gemv(const GemvParams &p, hipStream_t stream);
hipError_t launch_qkv_rope(const QkvParams &p, hipStream_t stream);
hipError_t launch_attention(const AttnParams &p, int num_heads, hipStream_t stream);
hipError_t launch_attention_partials(const AttnParams &p, hipStream_t stream);
hipError_t launch_gelu_mul(float *gate, const float *up, int64_t n, hipStream_t stream);
hipError_t launch_mlp_gate_up(const MlpParams &p, hipStream_t stream);
hipError_t launch_embed_gather(const EmbedParams &p, hipStream_t stream);
// The merge + gate launch of launch_attention alone (partials already written).
hipError_t launch_combine(const AttnParams &p, int num_heads, hipStream_t stream);
// Token groups of 16 (4 waves x 4 tokens) per chunk and KV head.
hipError_t launch_attention_chunk(const ChunkAttnParams &p, hipStream_t stream);
// Batched projections on MFMA (batch <= 32 per launch; see kMfmaMinBatch).
hipError_t launch_proj_mfma(const GemvParams &p, hipStream_t stream);
hipError_t launch_qkv_mfma(const QkvParams &p, hipStream_t stream);
hipError_t launch_rms_norm(const float *h, const uint16_t *w, float *out, int rows,
                           int hidden, float eps, hipStream_t stream);
hipError_t launch_residual_add(float *h, const float *o, int64_t n, hipStream_t stream);

// Host side (gqa_host.cpp): checks every argument of gqa_attention_block_decode
// except x_normed, out and the workspace, and gives the workspace bytes the
// block needs for these sequences (0 for batch 0).  Sets the error string.
gqa_status block_workspace_need(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                                const gqa_kv_seq *seqs, int32_t batch, size_t *need);
// Records a failure in the thread-local error string and returns st.
gqa_status report(gqa_status st, const char *fmt, ...);

}  // namespace gqa
