/*
 * gqa.h -- C ABI of the MI355X (gfx950) hybrid-window GQA decode attention block.
 *
 * The operation is the single-token decode attention block of the spark2_5
 * family as stated on the docs.rs pages of turbospark-runtime 0.3.0:
 *   [attn] src/families/spark/attn.rs  -- `encode_attention_block` (its steps,
 *          in order), `rope_params_for` and its unit test, the module doc;
 *   [mod]  src/families/spark/mod.rs   -- the module doc's transcription of one
 *          decoder layer; `produce_real_spark_inner`'s layer loop;
 *   [kvw]  src/kv_write.rs             -- `kv_write_target`, `encode_attention_any`.
 *
 * One call computes, for each of `batch` independent sequences b:
 *   qkv   = W_qkv x_b              rows q (Hq*D) | k (Hk*D) | v (Hk*D)
 *   g     = W_g x_b                one logit per query head, same x
 *   q,k,v = split(qkv); k and v go straight into this token's cache slot
 *   NeoX RoPE on q and on k (full layers: leading full_rotary_dim dims at
 *           full_rope_theta; sliding layers: all head_dim dims at rope_theta;
 *           the frequency divisor is the rotary width)
 *   a_h   = softmax(scale * K q_h) V over the causal history (full layers) or
 *           the last sliding_window positions read through a ring (sliding)
 *   a_h  *= sigmoid(g_h)           headwise, before the output projection
 *   out_b = W_o a
 *
 * Conventions for every entry point
 *   - Pointers named "device" are device (HBM) addresses; "host" ones are CPU
 *     addresses read before the call returns.  The caller owns all memory; the
 *     library allocates nothing and keeps no state except a thread-local error
 *     string.  Device memory must stay valid until the stream reaches the work.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.  Work
 *     is enqueued asynchronously: a GQA_OK status says the arguments were valid
 *     and the launches were accepted, not that the kernels have finished.
 *   - Every argument is checked on the host BEFORE the first launch, so a call
 *     that returns an error has enqueued nothing.  The library never aborts.
 *   - Device pointers must be 16-byte aligned; row counts and sizes are in
 *     elements unless a name ends in _bytes.
 *   - Dtypes: weights bf16 (raw uint16 bit patterns), KV cache IEEE fp16,
 *     activations and every intermediate fp32, accumulation fp32.
 *   - Kernels specialise head_dim == 256 and num_heads == 4 * num_kv_heads;
 *     other shapes return GQA_ERR_UNSUPPORTED.
 *
 * Precision and range (all within the parity bar of relative L2 error <= 1e-3
 * and max abs error <= 5e-3 max|ref| against an fp64 evaluation; not checked
 * at run time, since the values live on the device):
 *   - Attention runs on fp16 matrix cores with fp32 accumulation.  Each query
 *     element is scaled by attention_scale * log2(e) and carried as an fp16
 *     high part plus an fp16 low part (about 22 significant bits), so every
 *     |q_i| * attention_scale * log2(e) must stay below 65504, the fp16
 *     maximum: |q_i| < 7.2e5 at the published scale 1/16.  Larger values
 *     overflow to inf.  Softmax weights are split the same way and are at
 *     most 2^8.
 *   - In the q_k_v_proj, g_proj, o_proj, MLP down-projection and head GEMVs each
 *     activation element (after the RMSNorm weight, where there is one) is
 *     carried as a bf16 high part plus a bf16 low part, i.e. to within 2^-16
 *     of its magnitude (about 16 significant bits), while the bf16 weights
 *     are exact: below batch 4 on VALU dot products (v_dot2 of bf16 pairs
 *     into fp32), from batch 4 on bf16 matrix cores.  The MLP gate/up GEMV
 *     below batch 4 takes its activations in fp32.
 *   - RoPE angles are formed and reduced mod 2 pi in fp64; sin and cos are
 *     then taken in fp32.  k and v are rounded to fp16 once, after RoPE.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARGUMENT = 1,   /* a value violates the contract below      */
  GQA_ERR_UNSUPPORTED = 2,        /* valid, but a shape the kernels lack      */
  GQA_ERR_WORKSPACE_TOO_SMALL = 3,
  GQA_ERR_GPU = 4                 /* a HIP call failed; see gqa_last_error()  */
} gqa_status;

/* Architecture fields the block reads ([attn] `encode_attention_block` reads
 * hidden size, head counts, head dim, the full-layer mask, both thetas, the
 * sliding window and the attention scale; `full_rotary_dim` comes from the
 * family state).  Published values: num_heads 16, num_kv_heads 4, head_dim
 * 256, full_rotary_dim 64, sliding_window 512, full_rope_theta 5e6,
 * rope_theta 1e4, attention_scale 256^-0.5, rms_eps 1e-6 ([mod] module doc). */
typedef struct {
  int32_t hidden;            /* H: width of x and out                         */
  int32_t num_heads;         /* Hq                                            */
  int32_t num_kv_heads;      /* Hk                                            */
  int32_t head_dim;          /* D                                             */
  int32_t full_rotary_dim;   /* rotary width on full layers (even, <= D)      */
  int32_t sliding_window;    /* attended positions on sliding layers (>= 1)   */
  double full_rope_theta;    /* RoPE base on full layers (> 0)                */
  double rope_theta;         /* RoPE base on sliding layers (> 0)             */
  float attention_scale;     /* softmax scale (> 0, finite)                   */
  float rms_eps;             /* RMSNorm epsilon, used by gqa_rms_norm_bf16w   */
} gqa_arch;

/* One layer's projection weights, bf16, row-major [out][in] so that y = W x
 * ([attn] the GEMV calls pass rows = outputs, cols = inputs). Device, read-only.
 * `sinks` is the attention call's optional sink operand ([attn] the attention
 * step passes none; [kvw] `encode_attention_any` takes one): NULL for this
 * family, else device fp32 [Hq], one logit per query head that joins that
 * head's softmax with no value row, in the units of the scaled scores:
 *   p_t = e^{s_t} / (sum_u e^{s_u} + e^{sinks[h]}),  s_t = attention_scale q.k_t
 * (the pages leave the operand's meaning open; this is the reading taken).
 * A sink logit of -inf is the same as none; non-finite values other than -inf
 * are not checked (the memory is on the device) and give NaN or 0 outputs. */
typedef struct {
  const void *q_k_v_proj;    /* [Hq*D + 2*Hk*D][H], rows q | k | v, head-major */
  const void *g_proj;        /* [Hq][H]                                        */
  const void *o_proj;        /* [H][Hq*D]                                      */
  const float *sinks;        /* [Hq] fp32 sink logits, or NULL (none)          */
} gqa_layer_weights;

/* One sequence's K/V cache for this layer ([kvw] a slot is one position's row
 * of Hk*D fp16 values; attention reads the layer buffer from row 0).
 *   k, v        device fp16 [capacity][Hk][D]; the block WRITES row
 *               gqa_kv_slot(position, ring_capacity) of both (this token's
 *               RoPE'd k and its v) and reads only rows of the window.
 *   capacity    rows allocated (>= 1).
 *   ring_capacity  0: linear addressing, position < capacity required.
 *               > 0: ring of that many slots (sliding layers only), with
 *               sliding_window <= ring_capacity <= capacity.
 *   position    this token's position (>= 0); seq_len = position + 1.
 * Sequential positions and cache advancing stay with the caller. */
typedef struct {
  void *k;
  void *v;
  int32_t capacity;
  int32_t ring_capacity;
  int32_t position;
  int32_t reserved;          /* must be 0 */
} gqa_kv_seq;

/* ---------------------------------------------------------------------------
 * Pure host functions (no device access; usable without a GPU).
 * ------------------------------------------------------------------------- */

/* [attn] `rope_params_for`: full layers rotate the leading full_rotary_dim
 * dims at full_theta; sliding layers rotate all head_dim dims at
 * sliding_theta.  Outputs are host pointers; errors: null outputs, head_dim or
 * full_rotary_dim < 2 or odd, full_rotary_dim > head_dim, a theta <= 0. */
gqa_status gqa_rope_params_for(int is_full, int32_t full_rotary_dim, int32_t head_dim,
                               double full_theta, double sliding_theta,
                               int32_t *rotary_dim, double *theta);

/* [attn] the window/ring step: seq_len = position + 1; full layers read
 * [0, seq_len) linearly; sliding layers read [max(seq_len - window, 0),
 * seq_len) and use ring addressing only when ring_capacity > 0 and
 * seq_len > ring_capacity (active_ring = ring_capacity, else 0).
 * Errors: null outputs, position < 0, sliding_window < 1, ring_capacity < 0,
 * position == INT32_MAX. */
gqa_status gqa_kv_window(int is_full, int32_t position, int32_t sliding_window,
                         int32_t ring_capacity, int32_t *seq_len,
                         int32_t *kv_start, int32_t *active_ring);

/* Physical cache row of `position`: position mod ring_capacity on a ring,
 * position itself when ring_capacity == 0 ([kvw] `kv_write_target` returns
 * the slot of (layer, position)).  Returns -1 if position < 0 or
 * ring_capacity < 0. */
int32_t gqa_kv_slot(int32_t position, int32_t ring_capacity);

/* Bytes of device workspace that gqa_attention_block_decode and
 * gqa_attention_gated need for `batch` sequences whose seq_len is at most
 * max_seq_len (an upper bound valid for every layer class). */
gqa_status gqa_workspace_size(const gqa_arch *arch, int32_t batch, int32_t max_seq_len,
                              size_t *bytes);

/* The split-K plan the attention launches use for these sequences (the
 * library's own schedule, not a step of the pages; exposed so that its
 * invariants can be checked on the host).  The attended rows of sequence i
 * (gqa_kv_window) are cut into ceil(n_i / *chunk_rows) chunks, one workgroup
 * per chunk and KV head; sequences go to launch groups of at most 32.
 *   allow_direct  1: windows of at most 128 rows may run as one chunk that
 *                 the partial pass finishes itself (the block's plan); 0: the
 *                 plan of gqa_attention_partials
 *   chunk_rows    rows per chunk (a multiple of 64)
 *   waves         waves per attention workgroup (4, or 2 for batches)
 *   direct        1 if the plan is the one-chunk direct form
 *   groups        launch groups
 *   max_group_chunks  chunks of the largest launch group
 *   chunk_bound   the chunk count gqa_workspace_size provisions for this
 *                 batch and the longest seq_len; max_group_chunks never
 *                 exceeds it
 * Host only; seqs[].k and .v must be non-null and 16-byte aligned but are not
 * dereferenced.  Errors: as gqa_attention_block_decode's argument checks. */
gqa_status gqa_split_plan(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs, int32_t batch,
                          int allow_direct, int32_t *chunk_rows, int32_t *waves, int32_t *direct,
                          int32_t *groups, int32_t *max_group_chunks, int64_t *chunk_bound);

/* ---------------------------------------------------------------------------
 * The block.
 * ------------------------------------------------------------------------- */

/* [attn] `encode_attention_block`, for `batch` independent sequences that all
 * use this layer's weights and class.
 *   arch, weights   host structs (weights point to device memory)
 *   is_full         1: full (causal) layer; 0: sliding-window layer
 *   seqs            host array [batch] of this layer's caches
 *   x_normed        device fp32 [batch][H]: the already-normed layer input
 *   out             device fp32 [batch][H]: W_o (sigmoid-gated attention)
 *   workspace       device, at least gqa_workspace_size(...) bytes for the
 *                   largest seq_len in `seqs`; its contents on entry are
 *                   ignored (see the one-launch form below)
 * Side effect: each sequence's cache slot row for `position` is written.
 * x_normed and out must not overlap each other, the workspace or a cache.
 * One launch: for one sequence whose window is longer than 128 rows (at most
 * 256 split-K chunks, hidden <= 4096, num_heads * head_dim <= 4096) the whole
 * block runs as ONE persistent launch of one workgroup per CU whose tasks
 * wait for each other through flag words at the start of the workspace.
 * That launch needs its workgroups resident together: a call running
 * concurrently with other work on the same GPU (another stream) is delayed
 * until the CUs it needs are free, and two such calls must not overlap on
 * one GPU (their waits would time out after about a second and the outputs
 * would be wrong).  The flags carry a per-call epoch kept in the workspace,
 * so arbitrary workspace contents are accepted (a false match has
 * probability 2^-64 per flag word).  Other shapes run the projection, the
 * attention + merge and o_proj as separate launches.
 * Determinism: every case is bit-reproducible from run to run, and the
 * output equals, bit for bit, that of the step entry points below run in
 * order on the same inputs (each value is computed by the same code in the
 * same order). */
gqa_status gqa_attention_block_decode(const gqa_arch *arch, const gqa_layer_weights *weights,
                                      int is_full, const gqa_kv_seq *seqs, int32_t batch,
                                      const float *x_normed, float *out, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * block as gqa_attention_block_decode -- the same kernels, the same results --
 * with its workspace in the library's own static device scratch of 8 MiB per
 * GPU instead of a caller buffer.  The scratch is placed on each GPU when the
 * library's code object is loaded there and is held until the process ends;
 * its device address is looked up on the first call on a device (the
 * calling thread's current device, which must own `stream` and the buffers;
 * make that first call outside graph capture).  The call allocates no device
 * memory.
 *   arguments as for gqa_attention_block_decode, without the workspace.
 * Every call on one GPU uses that GPU's one scratch, which keeps the last
 * call's contents (nothing in it needs clearing between calls): calls that
 * overlap on one GPU (other streams, other threads) race on it and must be
 * serialised by the caller.
 * Errors: those of gqa_attention_block_decode; GQA_ERR_WORKSPACE_TOO_SMALL
 * when these sequences need more than the 8 MiB (the need grows with the
 * batch: at the published head counts one sequence of any length takes about
 * 1.5 MiB and 96 sequences about 4.5 MiB; gqa_workspace_size is an upper
 * bound);
 * GQA_ERR_GPU when the scratch's address cannot be obtained. */
gqa_status gqa_attention_block_decode_noalloc(const gqa_arch *arch, const gqa_layer_weights *weights,
                                              int is_full, const gqa_kv_seq *seqs, int32_t batch,
                                              const float *x_normed, float *out, void *stream);

/* M consecutive tokens of ONE sequence in one call: chunked prefill or the
 * verify step of a draft ([mod] the family's `prefill` module; [kvw] module
 * doc: chunked prefill reuses the per-token block, while the M-row path
 * projects K/V for all M rows with one GEMM).  Token t is at position
 * seq->position + t; its result is exactly the single-token block's at that
 * position after tokens 0 .. t-1 have been decoded: the projections run as
 * an M-row product that writes all M cache slots first, then token t attends
 * over its own window, which ends at its position (causal inside the chunk).
 *   seq        host pointer to ONE cache descriptor; position = the first
 *              token's position
 *   m_tokens   M >= 1
 *   x_normed   device fp32 [M][H]: the normed inputs of the M tokens
 *   out        device fp32 [M][H]
 *   workspace  device, at least gqa_workspace_size(arch, M, position + M)
 * Side effect: the cache slots of all M positions are written.
 * Errors: those of gqa_attention_block_decode for each token's position, and
 * INVALID_ARGUMENT when m_tokens < 1, when a linear cache has fewer than
 * position + M rows, or when a ring holds fewer than sliding_window + M - 1
 * slots (a later token's slot would overwrite a row an earlier token reads).
 * Determinism: M == 1 is gqa_attention_block_decode; M > 1 is bit-reproducible. */
gqa_status gqa_attention_block_chunk(const gqa_arch *arch, const gqa_layer_weights *weights,
                                     int is_full, const gqa_kv_seq *seq, int32_t m_tokens,
                                     const float *x_normed, float *out, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The attention half of one decoder layer, in place on the residual stream
 * ([mod] `produce_real_spark_inner`: input RMSNorm with a plain bf16 weight,
 * the block, the raw residual add):
 *   h[b] += block(RMSNorm(h[b]) * w_norm)
 * with RMSNorm(h) = h / sqrt(mean(h^2) + arch->rms_eps).  The norm is folded
 * into the projections (inv_rms(h) * W (h * w_norm)) and the residual add into
 * the o_proj epilogue, so a layer is the block's launches and nothing more.
 *   w_norm     device bf16 [H]
 *   h          device fp32 [batch][H], read and updated in place
 *   weights, is_full, seqs, workspace as for gqa_attention_block_decode (the
 *   workspace size is the block's).
 * Side effect: each sequence's cache slot row for `position` is written.
 * Determinism and the one-launch form as for gqa_attention_block_decode.
 * Errors: those of gqa_attention_block_decode, and rms_eps < 0 or not finite. */
gqa_status gqa_attention_layer_decode(const gqa_arch *arch, const gqa_layer_weights *weights,
                                      const void *w_norm, int is_full, const gqa_kv_seq *seqs,
                                      int32_t batch, float *h, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* One layer of a stack for gqa_attention_stack_decode: its weights, its input
 * RMSNorm weight (device bf16 [H]), its cache of the one sequence (the token's
 * position), and its class. */
typedef struct {
  gqa_layer_weights weights;
  const void *w_norm;
  gqa_kv_seq cache;
  int32_t is_full;
  int32_t reserved;          /* must be 0 */
} gqa_stack_layer;

/* One decode token of ONE sequence through a stack of attention layers, in
 * layer order ([mod] `produce_real_spark_inner`: the layer loop encodes every
 * layer of the token into one pass that is committed once):
 *   for l in 0 .. num_layers-1:  h += block_l(RMSNorm(h) * layers[l].w_norm)
 * i.e. gqa_attention_layer_decode for each layer in turn, with the same
 * result bit for bit.  Consecutive layers that the one-launch block takes
 * (see gqa_attention_block_decode; the window longer than 128 rows) run as
 * ONE persistent launch per up to 40 layers with at most 4 distinct
 * attention shapes (window, chunking, RoPE class), each layer's projections
 * starting as soon as the previous layer's o_proj has finished; other layers
 * run as gqa_attention_layer_decode runs them.
 *   layers     host array of num_layers descriptors (read during the call
 *              only); each layer's weights and cache as for
 *              gqa_attention_layer_decode, batch 1
 *   num_layers >= 0 (0: nothing is done)
 *   h          device fp32 [H], read and updated in place
 *   workspace  device, at least the largest of the layers' block workspaces
 *              (gqa_workspace_size(arch, 1, position + 1) is enough); the
 *              layers run one after another through it
 * Side effect: each layer's cache slot row for its position is written.
 * Residency and overlap: as for the one-launch block (its workgroups, one
 * per CU, must all be resident; calls on one workspace must not overlap).
 * Determinism: bit-reproducible, and equal to the layer-by-layer calls.
 * Errors: those of gqa_attention_layer_decode for any layer (the message
 * names the layer; nothing is enqueued then), INVALID_ARGUMENT for
 * num_layers < 0, a null layers array or a nonzero reserved field. */
gqa_status gqa_attention_stack_decode(const gqa_arch *arch, const gqa_stack_layer *layers,
                                      int32_t num_layers, float *h, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Step entry points: the block's steps one launch each, exposed so each
 * step can be checked and timed on its own.  They run the block's own code:
 * the same kernels where the block launches its steps separately, and, where
 * it runs as one launch, kernels that compute every value as its tasks do
 * (gqa_attention_gated runs the one-launch kernel's attention and merge
 * tasks themselves), so the steps' output equals the block's bit for bit.
 * ------------------------------------------------------------------------- */

/* [attn] the fused q_k_v_proj GEMV and the g_proj GEMV over the same input,
 * the split, the per-class NeoX RoPE of q and k, and the write of k and v
 * into this position's cache slot ([attn] GEMV, split and RoPE steps; [kvw]
 * `kv_write_target`).  k and v are rounded to fp16 once, after RoPE.
 *   x            device fp32 [batch][H]
 *   q_roped      device fp32 [batch][Hq*D]: RoPE'd q, head h at [h*D, (h+1)*D)
 *   gate_logits  device fp32 [batch][Hq] (before the sigmoid)
 *   seqs, is_full as for gqa_attention_block_decode (only the slot is used).
 * Side effect: each sequence's cache slot row for `position` is written. */
gqa_status gqa_qkv_rope_kv(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                           const gqa_kv_seq *seqs, int32_t batch, const float *x, float *q_roped,
                           float *gate_logits, void *stream);

/* [attn] the decode attention over the window (full layers: causal over
 * [0, seq_len); sliding layers: the last sliding_window positions, read
 * through the ring once it has wrapped) and the headwise sigmoid gate.  The
 * cache must already hold this token's row (gqa_qkv_rope_kv writes it).
 *   q_roped      device fp32 [batch][Hq*D]
 *   gate_logits  device fp32 [batch][Hq]
 *   sinks        device fp32 [Hq] or NULL, as gqa_layer_weights.sinks (the
 *                same logits for every sequence)
 *   attn_gated   device fp32 [batch][Hq*D]: head h at [h*D, (h+1)*D)
 *   seqs, is_full, workspace as for gqa_attention_block_decode.
 * One sequence with a window longer than 128 rows runs as one launch of the
 * block's one-launch kernel restricted to its attention and merge tasks
 * (the residency note of gqa_attention_block_decode applies).
 * Reads the caches only. */
gqa_status gqa_attention_gated(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs,
                               int32_t batch, const float *q_roped, const float *gate_logits,
                               const float *sinks, float *attn_gated, void *workspace,
                               size_t workspace_bytes, void *stream);

/* The split-K pass of gqa_attention_gated alone (the dominant kernel of the
 * block), for one launch group of at most 32 sequences; exposed so the pass
 * can be checked and timed by itself.  The attended rows of sequence i are
 * cut into chunks of *chunk_rows rows (the plan the block uses); chunk j of
 * sequence i is flat chunk chunk_begin[i] + j.  For every flat chunk c and
 * query head h it writes the chunk's unnormalised softmax partial, scores in
 * log2 units (s_r = attention_scale * log2(e) * q_h . k_r over the chunk's
 * rows r, [attn] attention step):
 *   part_ml[c][h] = (m, l)  with  l * 2^m = sum_r 2^s_r  (m is a reference
 *                   point within 8 of the chunk's largest s_r)
 *   part_o[c][h][e] = (sum_r 2^(s_r - m) v_r)[16 * (e % 16) + e / 16]
 * so that part_o / l is the attention of q_h over the chunk's rows.  Sink logits do
 * not enter the partials: they join the softmax where the chunks are merged.
 *   q_roped      device fp32 [batch][Hq*D]
 *   part_o       device fp32 [max_chunks][Hq][D]
 *   part_ml      device fp32 [max_chunks][Hq][2]
 *   chunk_rows   host out: rows per chunk (a multiple of 64)
 *   chunk_begin  host out [batch + 1]: first flat chunk of each sequence, then
 *                the total
 * Errors: batch > 32 (UNSUPPORTED), more chunks than max_chunks
 * (WORKSPACE_TOO_SMALL), and the checks of gqa_attention_gated.
 * Reads the caches only. */
gqa_status gqa_attention_partials(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs,
                                  int32_t batch, const float *q_roped, float *part_o,
                                  float *part_ml, int32_t max_chunks, int32_t *chunk_rows,
                                  int32_t *chunk_begin, void *stream);

/* [attn] the o_proj GEMV: out[b] = W_o attn_gated[b].
 *   attn_gated device fp32 [batch][Hq*D]; out device fp32 [batch][H]. */
gqa_status gqa_o_proj_gemv(const gqa_arch *arch, const gqa_layer_weights *weights,
                           int32_t batch, const float *attn_gated, float *out, void *stream);

/* ---------------------------------------------------------------------------
 * Layer-loop helpers around the block ([mod] `produce_real_spark_inner`: the
 * input RMSNorm with a bf16 weight before the block, the raw residual add
 * after it).
 * ------------------------------------------------------------------------- */

/* out[r][c] = h[r][c] / sqrt(mean_c(h[r][c]^2) + eps) * w[c], plain w.
 *   h device fp32 [rows][hidden]; w device bf16 [hidden]; out device fp32
 *   [rows][hidden] (may equal h).  eps >= 0, finite. */
gqa_status gqa_rms_norm_bf16w(const float *h, const void *w, float *out, int32_t rows,
                              int32_t hidden, float eps, void *stream);

/* h[i] += o[i] for i < n (device fp32, n >= 0, no partial overlap). */
gqa_status gqa_residual_add(float *h, const float *o, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * The rest of the decoder layer ([mod] module doc, the transcribed layer's
 * last two lines): after the attention's residual add,
 *   x = rms(h, post_attention_layernorm, rms_eps)   (plain w)
 *   h = h + down_proj(gelu_erf(gate_proj x) * up_proj x)
 * with the exact (erf) GELU, x * Phi(x).  The pages print no intermediate
 * size; any multiple of 8 up to 8192 is taken.
 * ------------------------------------------------------------------------- */

typedef struct {
  const void *post_attention_layernorm; /* bf16 [hidden] */
  const void *gate_proj;                /* bf16 [intermediate][hidden], row-major */
  const void *up_proj;                  /* bf16 [intermediate][hidden] */
  const void *down_proj;                /* bf16 [hidden][intermediate] */
  int32_t intermediate;
  int32_t reserved;                     /* must be 0 */
} gqa_mlp_weights;

/* Workspace bytes gqa_mlp_decode needs for `batch` rows (x, gate and up
 * projections, fp32).  Errors: as for gqa_mlp_decode's shape checks. */
gqa_status gqa_mlp_workspace_size(const gqa_arch *arch, int32_t intermediate, int32_t batch,
                                  size_t *bytes);

/* h[b] += down_proj(gelu_erf(gate_proj x_b) * up_proj x_b), x_b the RMSNorm of
 * h[b] with post_attention_layernorm and arch->rms_eps, for b < batch, in
 * place.  h is device fp32 [batch][hidden]; the weights are device bf16 as
 * above; workspace is device memory of at least gqa_mlp_workspace_size
 * bytes, owned by the caller.  Below batch 4 two launches on `stream`: the
 * norm, both projections and the activation in one, then the down projection
 * with the residual add in its epilogue; from batch 4 (matrix cores) four:
 * the norm, the gate and up projections, the activation, the down projection.
 * Errors: null or misaligned pointers, intermediate not a multiple of 8 or
 * below 8, reserved != 0, rms_eps negative or not finite
 * (INVALID_ARGUMENT); intermediate above 8192 (UNSUPPORTED); a workspace
 * smaller than needed (WORKSPACE_TOO_SMALL); a launch failure (GPU).
 * batch 0 is a no-op. */
gqa_status gqa_mlp_decode(const gqa_arch *arch, const gqa_mlp_weights *weights, int32_t batch,
                          float *h, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * The ends of the decode step ([mod] `produce_real_spark_inner`): the token's
 * embedding row enters the stack raw (no sqrt(hidden) scale, no norm); after
 * the last layer the final RMSNorm (model.norm, plain w) and the TIED head,
 * logits = x @ embed_tokens^T (raw logits, fp32 here).  The pages print no
 * vocabulary size.
 * ------------------------------------------------------------------------- */

/* h[b] = embed_tokens[ids[b]] as fp32, b < batch.
 *   embed_tokens device bf16 [vocab][hidden]; ids HOST int32 [batch], each in
 *   [0, vocab); h device fp32 [batch][hidden].
 * Errors: null or misaligned pointers, vocab < 1, an id out of range
 * (INVALID_ARGUMENT); vocab * hidden * 2 >= 2^31 (UNSUPPORTED).  batch 0 is a
 * no-op. */
gqa_status gqa_embed_tokens(const gqa_arch *arch, const void *embed_tokens, int32_t vocab,
                            const int32_t *ids, int32_t batch, float *h, void *stream);

/* Workspace bytes of gqa_lm_head for `batch` rows (the normed x, fp32). */
gqa_status gqa_lm_head_workspace_size(const gqa_arch *arch, int32_t batch, size_t *bytes);

/* logits[b] = rms(h[b], final_norm, arch->rms_eps) @ embed_tokens^T.
 *   final_norm device bf16 [hidden]; embed_tokens device bf16 [vocab][hidden];
 *   h device fp32 [batch][hidden] (read only); logits device fp32
 *   [batch][vocab]; workspace device, caller-owned.  Two launches: the norm,
 *   the head GEMV (VALU below batch 4, matrix cores from 4).
 * Errors: as gqa_embed_tokens for the table, null or misaligned pointers,
 * rms_eps negative or not finite (INVALID_ARGUMENT), a small workspace
 * (WORKSPACE_TOO_SMALL), launch failures (GPU). */
gqa_status gqa_lm_head(const gqa_arch *arch, const void *final_norm, const void *embed_tokens,
                       int32_t vocab, const float *h, int32_t batch, float *logits, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Diagnostics.
 * ------------------------------------------------------------------------- */
const char *gqa_status_string(gqa_status status);
/* Detail of the last error on this thread ("" if none).  Valid until the next
 * call into the library from this thread. */
const char *gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
