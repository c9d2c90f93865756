// Host side of libgqa: argument checks, the window/slot/RoPE-parameter
// functions, the split-K plan, workspace layout and the extern "C" entry
// points declared in include/gqa.h.
//
// Every entry point validates all of its arguments before the first launch so
// that an error return means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "gqa.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

thread_local std::string g_last_error;

gqa_status fail(gqa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gqa_status ok() {
  g_last_error.clear();
  return GQA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr double kLog2e = 1.4426950408889634;

// ---- architecture ---------------------------------------------------------

gqa_status check_arch(const gqa_arch *a) {
  if (!a) return fail(GQA_ERR_INVALID_ARGUMENT, "arch is null");
  if (a->hidden < 8 || a->hidden % 8 != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "hidden=%d must be a positive multiple of 8", a->hidden);
  if (a->hidden > kMaxHidden)
    return fail(GQA_ERR_UNSUPPORTED, "hidden=%d exceeds the supported %d", a->hidden, kMaxHidden);
  if (a->num_kv_heads < 1 || a->num_heads < 1)
    return fail(GQA_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (num_heads=%d num_kv_heads=%d)",
                a->num_heads, a->num_kv_heads);
  if (a->num_heads % a->num_kv_heads != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "num_heads=%d is not a multiple of num_kv_heads=%d",
                a->num_heads, a->num_kv_heads);
  if (a->num_heads != kGroup * a->num_kv_heads)
    return fail(GQA_ERR_UNSUPPORTED, "kernels need num_heads == 4 * num_kv_heads (got %d, %d)",
                a->num_heads, a->num_kv_heads);
  if (a->head_dim != kHeadDim)
    return fail(GQA_ERR_UNSUPPORTED, "kernels need head_dim == 256 (got %d)", a->head_dim);
  if (a->num_heads * a->head_dim > kMaxHidden)
    return fail(GQA_ERR_UNSUPPORTED, "num_heads*head_dim=%d exceeds %d", a->num_heads * a->head_dim,
                kMaxHidden);
  if (a->full_rotary_dim < 2 || a->full_rotary_dim % 2 != 0 || a->full_rotary_dim > a->head_dim)
    return fail(GQA_ERR_INVALID_ARGUMENT, "full_rotary_dim=%d must be even and in [2, head_dim]",
                a->full_rotary_dim);
  if (a->sliding_window < 1)
    return fail(GQA_ERR_INVALID_ARGUMENT, "sliding_window=%d must be >= 1", a->sliding_window);
  if (!(a->full_rope_theta > 0.0) || !isfinite(a->full_rope_theta) || !(a->rope_theta > 0.0) ||
      !isfinite(a->rope_theta))
    return fail(GQA_ERR_INVALID_ARGUMENT, "rope thetas must be finite and > 0");
  if (!(a->attention_scale > 0.f) || !isfinite(a->attention_scale))
    return fail(GQA_ERR_INVALID_ARGUMENT, "attention_scale must be finite and > 0");
  const size_t qkv_bytes = (size_t)(a->num_heads + 2 * a->num_kv_heads) * a->head_dim * a->hidden * 2u;
  if (qkv_bytes > kMaxBufferBytes)
    return fail(GQA_ERR_UNSUPPORTED, "q_k_v_proj of %zu bytes exceeds the supported %u", qkv_bytes,
                kMaxBufferBytes);
  return GQA_OK;
}

gqa_status check_weights(const gqa_layer_weights *w, bool need_qkv, bool need_o) {
  if (!w) return fail(GQA_ERR_INVALID_ARGUMENT, "weights is null");
  if (need_qkv) {
    if (!w->q_k_v_proj || !w->g_proj)
      return fail(GQA_ERR_INVALID_ARGUMENT, "q_k_v_proj or g_proj is null");
    if (!aligned16(w->q_k_v_proj) || !aligned16(w->g_proj))
      return fail(GQA_ERR_INVALID_ARGUMENT, "q_k_v_proj and g_proj must be 16-byte aligned");
  }
  if (need_o) {
    if (!w->o_proj) return fail(GQA_ERR_INVALID_ARGUMENT, "o_proj is null");
    if (!aligned16(w->o_proj)) return fail(GQA_ERR_INVALID_ARGUMENT, "o_proj must be 16-byte aligned");
  }
  return GQA_OK;
}

gqa_status check_ptr(const void *p, const char *name) {
  if (!p) return fail(GQA_ERR_INVALID_ARGUMENT, "%s is null", name);
  if (!aligned16(p)) return fail(GQA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return GQA_OK;
}

gqa_status check_batch(const gqa_arch *a, int32_t batch) {
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  const size_t widest = (size_t)std::max(a->hidden, a->num_heads * a->head_dim);
  if ((size_t)batch * widest * sizeof(float) > kMaxBufferBytes)
    return fail(GQA_ERR_UNSUPPORTED, "batch=%d makes an activation larger than %u bytes", batch,
                kMaxBufferBytes);
  return GQA_OK;
}

// ---- window, slot, RoPE parameters (pure) ---------------------------------

gqa_status window_of(int is_full, int32_t position, int32_t window, int32_t ring, int32_t *seq_len,
                     int32_t *kv_start, int32_t *active_ring) {
  if (position < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "position=%d must be >= 0", position);
  if (position == INT32_MAX) return fail(GQA_ERR_INVALID_ARGUMENT, "position + 1 overflows");
  if (window < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "sliding_window=%d must be >= 1", window);
  if (ring < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "ring_capacity=%d must be >= 0", ring);
  const int32_t sl = position + 1;
  if (is_full) {
    *seq_len = sl;
    *kv_start = 0;
    *active_ring = 0;
  } else {
    *seq_len = sl;
    *kv_start = sl > window ? sl - window : 0;
    *active_ring = (ring > 0 && sl > ring) ? ring : 0;
  }
  return GQA_OK;
}

// ---- sequences and the split-K plan ----------------------------------------

struct Plan {
  int chunk = kChunkQuantum;
  bool direct = false;   // one chunk per sequence, finished by the partial kernel
  int waves = 4;         // waves per workgroup of the partial kernel (4 or 2)
  struct Group {
    int first = 0, count = 0, total_chunks = 0;
  };
  std::vector<Group> groups;
  size_t max_group_chunks = 0;
};

// Resolve and check every sequence.  Fills one SeqDesc per sequence (without
// chunk_begin) and the attended-row counts.
gqa_status resolve_seqs(const gqa_arch *a, int is_full, const gqa_kv_seq *seqs, int32_t batch,
                        std::vector<SeqDesc> *out) {
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  if (batch > 0 && !seqs) return fail(GQA_ERR_INVALID_ARGUMENT, "seqs is null");
  out->resize(batch);
  for (int32_t b = 0; b < batch; ++b) {
    const gqa_kv_seq &s = seqs[b];
    gqa_status st;
    if ((st = check_ptr(s.k, "seqs[].k")) != GQA_OK) return st;
    if ((st = check_ptr(s.v, "seqs[].v")) != GQA_OK) return st;
    if (s.reserved != 0) return fail(GQA_ERR_INVALID_ARGUMENT, "seqs[%d].reserved must be 0", b);
    if (s.capacity < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "seqs[%d].capacity=%d < 1", b, s.capacity);
    if (s.ring_capacity < 0)
      return fail(GQA_ERR_INVALID_ARGUMENT, "seqs[%d].ring_capacity=%d < 0", b, s.ring_capacity);
    if (s.ring_capacity > 0) {
      if (is_full)
        return fail(GQA_ERR_INVALID_ARGUMENT,
                    "seqs[%d]: a full (causal) layer has no ring (ring_capacity=%d)", b, s.ring_capacity);
      if (s.ring_capacity < a->sliding_window)
        return fail(GQA_ERR_INVALID_ARGUMENT,
                    "seqs[%d].ring_capacity=%d < sliding_window=%d would overwrite rows of the window",
                    b, s.ring_capacity, a->sliding_window);
      if (s.ring_capacity > s.capacity)
        return fail(GQA_ERR_INVALID_ARGUMENT, "seqs[%d].ring_capacity=%d > capacity=%d", b,
                    s.ring_capacity, s.capacity);
    }
    int32_t sl, ks, ar;
    if ((st = window_of(is_full, s.position, a->sliding_window, s.ring_capacity, &sl, &ks, &ar)) != GQA_OK)
      return st;
    if (s.ring_capacity == 0 && s.position >= s.capacity)
      return fail(GQA_ERR_INVALID_ARGUMENT, "seqs[%d].position=%d needs a linear cache of more than %d rows",
                  b, s.position, s.capacity);
    const size_t cache_bytes = (size_t)s.capacity * a->num_kv_heads * a->head_dim * 2u;
    if (cache_bytes > kMaxBufferBytes)
      return fail(GQA_ERR_UNSUPPORTED, "seqs[%d]: a %zu-byte K/V cache exceeds the supported %u bytes", b,
                  cache_bytes, kMaxBufferBytes);
    SeqDesc &d = (*out)[b];
    d.k = static_cast<_Float16 *>(s.k);
    d.v = static_cast<_Float16 *>(s.v);
    d.kv_start = ks;
    d.n = sl - ks;
    d.ring = ar;
    d.slot = s.ring_capacity > 0 ? s.position % s.ring_capacity : s.position;
    d.position = s.position;
    d.chunk_begin = 0;
    d.cache_bytes = (unsigned)cache_bytes;
  }
  return GQA_OK;
}

// Split-K plan.  One attention workgroup covers a chunk of rows for one KV
// head (a quarter of the rows per wave).  The chunk is the largest multiple
// of kChunkQuantum that still gives every launch about kAttnTargetWgs (twice
// that for 2-wave workgroups)
// workgroups (longer chunks spend less on each wave's set-up and on the
// partials; fewer workgroups than the chip holds leave HBM bandwidth unused).
// With C(c) chunks at chunk size c this keeps C <= 2 * target / Hk +
// sequences (see max_chunks).
Plan make_plan(const std::vector<SeqDesc> &seqs, int num_kv_heads, bool allow_direct) {
  Plan plan;
  auto wgs = [&](int chunk) {
    long n = 0;
    for (const SeqDesc &s : seqs) n += (long)ceil_div(s.n, chunk) * num_kv_heads;
    return n;
  };
  int longest = 1;
  long total = 0;
  for (const SeqDesc &s : seqs) {
    longest = std::max(longest, s.n);
    total += s.n;
  }
  // short launches: half the workgroups, two tiles per wave instead of one
  // (measured at 4096 rows: 22.9 against 24.6 us per block; at 8192 rows and
  // beyond the full target is faster)
  const bool direct = allow_direct && longest <= kDirectMaxRows;
  // many long sequences: 2-wave workgroups, twice as many (two resident per CU)
  plan.waves = !direct && (int)seqs.size() >= kNarrowMinSeqs && total > kShortPlanRows ? 2 : 4;
  const int full = plan.waves == 2 ? 2 * kAttnTargetWgs : kAttnTargetWgs;
  const int target = total <= kShortPlanRows ? full / 2 : full;
  const int cap = ceil_div(longest, kChunkQuantum) * kChunkQuantum;
  int chunk = kChunkQuantum;
  if (direct) {
    chunk = cap;
    plan.direct = true;
  } else {
    while (chunk + kChunkQuantum <= cap && wgs(chunk + kChunkQuantum) >= target) chunk += kChunkQuantum;
    // Workgroups past a multiple of the resident slots (one per CU, two with
    // 2-wave workgroups) run as another round of full-length workgroups: from
    // this chunk size up, take the least rounds x rows per chunk (ties: the
    // larger chunk, fewer partials).  A round costs at least its chunk, so
    // the search ends once the chunk alone exceeds the best cost.  Fewer
    // chunks than the loop above chose, so the workspace bound still holds.
    if (total > kShortPlanRows) {
      const long slots = (long)kAttnTargetWgs * (plan.waves == 2 ? 2 : 1);
      auto rounds = [&](int c) { return (wgs(c) + slots - 1) / slots; };
      long best = rounds(chunk) * chunk;
      for (int c = chunk + kChunkQuantum; c <= cap && c <= best; c += kChunkQuantum) {
        const long cost = rounds(c) * c;
        if (cost <= best) {
          best = cost;
          chunk = c;
        }
      }
    }
  }
  plan.chunk = chunk;
  for (int first = 0; first < (int)seqs.size(); first += kMaxSeqPerLaunch) {
    Plan::Group g;
    g.first = first;
    g.count = std::min<int>(kMaxSeqPerLaunch, (int)seqs.size() - first);
    int tot = 0;
    for (int i = 0; i < g.count; ++i) tot += ceil_div(seqs[first + i].n, plan.chunk);
    g.total_chunks = tot;
    plan.max_group_chunks = std::max<size_t>(plan.max_group_chunks, (size_t)tot);
    plan.groups.push_back(g);
  }
  return plan;
}

// Several tokens of one sequence (attn_chunk_kernel): the rows every token
// attends, [r0, position + M), are cut into chunks of a multiple of 32 rows,
// the largest that still gives kAttnTargetWgs workgroups of (chunk, KV head,
// 16 tokens).
struct ChunkPlan {
  int r0 = 0, rows = 0, chunk = 32, nchunks = 1, window = 0;
};

ChunkPlan make_chunk_plan(const gqa_arch *a, int is_full, int32_t first_pos, int32_t m) {
  ChunkPlan cp;
  cp.window = is_full ? first_pos + m : a->sliding_window;
  cp.r0 = std::max(0, first_pos + 1 - cp.window);
  cp.rows = first_pos + m - cp.r0;
  const long groups = (long)a->num_kv_heads * ceil_div(m, 16);
  const int cap = ceil_div(cp.rows, 32) * 32;
  while (cp.chunk + 32 <= cap && (long)ceil_div(cp.rows, cp.chunk + 32) * groups >= kChunkTargetWgs) cp.chunk += 32;
  cp.nchunks = ceil_div(cp.rows, cp.chunk);
  return cp;
}

// Partial rows (token x chunk) of a chunk plan for m tokens: by the argument
// of max_chunks below, nchunks <= 2 * ceil(target / groups) + 1.
size_t chunk_partial_rows(int num_kv_heads, int32_t m, int32_t max_seq_len) {
  if (m < 2) return 0;
  const size_t groups = (size_t)num_kv_heads * ceil_div(m, 16);
  const size_t per = std::min((size_t)ceil_div(max_seq_len, 32),
                              2 * ((kChunkTargetWgs + groups - 1) / groups) + 1);
  return (size_t)m * per;
}

// Upper bound of Plan::max_group_chunks for `batch` sequences of at most
// max_seq_len attended rows.  If the plan stops at chunk c > q (q =
// kChunkQuantum) because C(c + q) * Hk < target, then C(c) <= N / c + B <=
// 2 C(c + q) + B; at c = q, C(q) <= 2 C(2q) likewise; at the cap C = B.
size_t max_chunks(int num_kv_heads, int32_t batch, int32_t max_seq_len) {
  const size_t seqs = (size_t)std::min<int32_t>(batch, kMaxSeqPerLaunch);
  const size_t finest = (size_t)ceil_div(max_seq_len, kChunkQuantum) * seqs;
  const size_t bound = 2 * (size_t)ceil_div(2 * kAttnTargetWgs, num_kv_heads) + seqs;   // the 2-wave target
  return std::max(std::min(finest, bound), chunk_partial_rows(num_kv_heads, batch, max_seq_len));
}

// ---- workspace layout -----------------------------------------------------

struct Layout {
  size_t q = 0, gate = 0, attn = 0, part_o = 0, part_ml = 0, total = 0;
};

size_t partial_bytes_o(const gqa_arch *a, size_t chunks) {
  return round_up(chunks * (size_t)a->num_heads * kHeadDim * sizeof(float), 256);
}
size_t partial_bytes_ml(const gqa_arch *a, size_t chunks) {
  return round_up(chunks * (size_t)a->num_heads * 2 * sizeof(float), 256);
}

// Block layout: [sync | q | gate | attn | part_o | part_ml]; the attention
// step alone uses [sync | part_o | part_ml].  The synchronisation words of
// the one-launch block (kSyncBytes) come first in both, so other paths never
// overwrite them.
Layout block_layout(const gqa_arch *a, int32_t batch, size_t chunks) {
  Layout L;
  const size_t q_dim = (size_t)a->num_heads * a->head_dim;
  L.q = kSyncBytes;
  L.gate = L.q + round_up((size_t)batch * q_dim * sizeof(float), 256);
  L.attn = L.gate + round_up((size_t)batch * a->num_heads * sizeof(float), 256);
  L.part_o = L.attn + round_up((size_t)batch * a->num_heads * a->head_dim * sizeof(float), 256);
  L.part_ml = L.part_o + partial_bytes_o(a, chunks);
  L.total = L.part_ml + partial_bytes_ml(a, chunks);
  return L;
}

// ---- launch helpers -------------------------------------------------------

gqa_status gpu_error(hipError_t e, const char *what) {
  return fail(GQA_ERR_GPU, "%s: %s", what, hipGetErrorString(e));
}

// The fused projection step for every sequence, in launch groups of up to
// kMaxSeqPerLaunch batch rows.
// x is the normed input, or (w_norm set) the raw residual stream h, normed
// on the fly with w_norm.
gqa_status run_qkv_rope(const gqa_arch *a, const gqa_layer_weights *w, int is_full,
                        const std::vector<SeqDesc> &seqs, const float *x, float *q, float *gate,
                        hipStream_t stream, const uint16_t *w_norm = nullptr) {
  int32_t rdim;
  double theta;
  gqa_rope_params_for(is_full, a->full_rotary_dim, a->head_dim, a->full_rope_theta, a->rope_theta, &rdim,
                      &theta);
  const long q_dim = (long)a->num_heads * a->head_dim;
  for (int first = 0; first < (int)seqs.size(); first += kMaxSeqPerLaunch) {
    QkvParams p{};
    p.w_qkv = static_cast<const uint16_t *>(w->q_k_v_proj);
    p.w_g = static_cast<const uint16_t *>(w->g_proj);
    p.hidden = a->hidden;
    p.batch = std::min<int>(kMaxSeqPerLaunch, (int)seqs.size() - first);
    p.x = x + (size_t)first * a->hidden;
    p.ldx = a->hidden;
    p.q_out = q + (size_t)first * q_dim;
    p.ld_q = q_dim;
    p.gate_out = gate + (size_t)first * a->num_heads;
    p.ld_gate = a->num_heads;
    p.num_heads = a->num_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.rotary_dim = rdim;
    p.log2_theta = log2(theta);
    p.w_norm = w_norm;
    p.rms_eps = a->rms_eps;
    for (int i = 0; i < p.batch; ++i) p.seq[i] = seqs[first + i];
    // batched: MFMA (its units pair RoPE tiles, so the rotated width must be
    // whole 32-row tile pairs); batch 1-3: the fused VALU kernel
    const bool mfma = p.batch >= kMfmaMinBatch && rdim % 32 == 0;
    hipError_t e = mfma ? launch_qkv_mfma(p, stream) : launch_qkv_rope(p, stream);
    if (e != hipSuccess) return gpu_error(e, "qkv/RoPE/KV-write launch");
  }
  return GQA_OK;
}

// accumulate: out += W_o attn (the residual add) instead of out = W_o attn
gqa_status run_o_proj(const gqa_arch *a, const gqa_layer_weights *w, int32_t batch, const float *attn,
                      float *out, hipStream_t stream, bool accumulate = false) {
  const int cols = a->num_heads * a->head_dim;
  if (batch >= kMfmaMinBatch) {
    // groups of <= 32 batch rows on MFMA (a small last group on the VALU GEMV)
    for (int first = 0; first < batch; first += 32) {
      GemvParams p{};
      p.w0 = static_cast<const uint16_t *>(w->o_proj);
      p.rows0 = a->hidden;
      p.cols = cols;
      p.batch = std::min(32, batch - first);
      p.x = attn + (size_t)first * cols;
      p.ldx = cols;
      p.y0 = out + (size_t)first * a->hidden;
      p.ldy0 = a->hidden;
      p.accumulate = accumulate ? 1 : 0;
      hipError_t e = p.batch >= kMfmaMinBatch ? launch_proj_mfma(p, stream) : launch_gemv(p, stream);
      if (e != hipSuccess) return gpu_error(e, "o_proj launch");
    }
    return GQA_OK;
  }
  GemvParams p{};
  p.w0 = static_cast<const uint16_t *>(w->o_proj);
  p.w1 = nullptr;
  p.rows0 = a->hidden;
  p.rows1 = 0;
  p.cols = a->num_heads * a->head_dim;
  p.batch = batch;
  p.x = attn;
  p.ldx = p.cols;
  p.y0 = out;
  p.ldy0 = a->hidden;
  p.y1 = nullptr;
  p.ldy1 = 0;
  p.accumulate = accumulate ? 1 : 0;
  hipError_t e = launch_gemv(p, stream);
  return e == hipSuccess ? GQA_OK : gpu_error(e, "o_proj GEMV launch");
}

// Kernel arguments of one launch group.  q, gate and attn point at row 0 of
// the whole batch; gate and attn may be null (the partial pass alone).
AttnParams attn_params(const gqa_arch *a, const std::vector<SeqDesc> &seqs, const Plan &plan,
                       const Plan::Group &g, const float *q, const float *gate, float *attn, float *part_o,
                       float *part_ml) {
  const long q_dim = (long)a->num_heads * a->head_dim;
  AttnParams p{};
  p.q = q + (size_t)g.first * q_dim;
  p.ld_q = q_dim;
  p.gate = gate ? gate + (size_t)g.first * a->num_heads : nullptr;
  p.ld_gate = a->num_heads;
  p.out = attn ? attn + (size_t)g.first * q_dim : nullptr;
  p.ld_out = q_dim;
  p.part_o = part_o;
  p.part_ml = part_ml;
  p.num_kv_heads = a->num_kv_heads;
  p.qscale = (float)((double)a->attention_scale * kLog2e);
  p.chunk = plan.chunk;
  p.direct = plan.direct ? 1 : 0;
  p.waves = plan.waves;
  p.nseq = g.count;
  p.total_chunks = g.total_chunks;
  int cb = 0;
  for (int i = 0; i < g.count; ++i) {
    p.seq[i] = seqs[g.first + i];
    p.seq[i].chunk_begin = cb;
    cb += ceil_div(p.seq[i].n, plan.chunk);
  }
  return p;
}

gqa_status run_attention(const gqa_arch *a, const std::vector<SeqDesc> &seqs, const Plan &plan,
                         const float *q, const float *gate, const float *sinks, float *attn, float *part_o,
                         float *part_ml, hipStream_t stream) {
  for (const Plan::Group &g : plan.groups) {
    AttnParams p = attn_params(a, seqs, plan, g, q, gate, attn, part_o, part_ml);
    p.sinks = sinks;
    hipError_t e = launch_attention(p, a->num_heads, stream);
    if (e != hipSuccess) return gpu_error(e, "attention launch");
  }
  return GQA_OK;
}

// One sequence whose window needs more than one chunk (longer than the
// direct form's 128 rows) runs its attention through block_fused_kernel: the
// whole block in one launch when x fits the kernel's LDS staging and o_proj
// its registers, else its attention + merge phase between the projection and
// o_proj launches.  Either way the merge of the chunks has one fixed order.
bool fused_attention(const gqa_arch *a, const Plan &plan, int32_t batch) {
  return batch == 1 && !plan.direct && plan.groups.size() == 1 &&
         plan.groups[0].total_chunks <= kFusedMaxChunks && a->num_kv_heads <= 8;
}
bool fused_whole(const gqa_arch *a) {
  return a->hidden <= kFusedMaxHidden && a->num_heads * a->head_dim <= kFusedMaxQDim;
}

FusedParams fused_params(const gqa_arch *a, int is_full, const SeqDesc &sd, const Plan &plan, int phases,
                         const float *q, const float *gate, const float *sinks, float *part_o, float *part_ml,
                         float *attn, void *sync) {
  FusedParams p{};
  p.phases = phases;
  p.hidden = a->hidden;
  p.rms_eps = a->rms_eps;
  int32_t rdim;
  double theta;
  gqa_rope_params_for(is_full, a->full_rotary_dim, a->head_dim, a->full_rope_theta, a->rope_theta, &rdim, &theta);
  p.rotary_dim = rdim;
  p.log2_theta = log2(theta);
  p.q = const_cast<float *>(q);
  p.gate = const_cast<float *>(gate);
  p.seq = sd;
  p.seq.chunk_begin = 0;
  p.chunk = plan.chunk;
  p.nchunks = plan.groups[0].total_chunks;
  p.qscale = (float)((double)a->attention_scale * kLog2e);
  p.sinks = sinks;
  p.part_o = part_o;
  p.part_ml = part_ml;
  p.a = attn;
  p.sync = static_cast<unsigned long long *>(sync);
  p.num_heads = a->num_heads;
  p.num_kv_heads = a->num_kv_heads;
  return p;
}

// The block (or, with w_norm, the layer: y is then the residual stream and
// takes y += W_o a) for one sequence through block_fused_kernel.
gqa_status run_fused_block(const gqa_arch *a, const gqa_layer_weights *w, int is_full, const SeqDesc &sd,
                           const Plan &plan, const float *x, const uint16_t *w_norm, float *y, bool accumulate,
                           char *ws, const Layout &L, hipStream_t stream) {
  float *q = reinterpret_cast<float *>(ws + L.q);
  float *gate = reinterpret_cast<float *>(ws + L.gate);
  float *attn = reinterpret_cast<float *>(ws + L.attn);
  float *part_o = reinterpret_cast<float *>(ws + L.part_o);
  float *part_ml = reinterpret_cast<float *>(ws + L.part_ml);
  const bool whole = fused_whole(a);
  FusedParams p = fused_params(a, is_full, sd, plan, whole ? kPhaseQkv | kPhaseAttn | kPhaseOproj : kPhaseAttn, q,
                               gate, w->sinks, part_o, part_ml, attn, ws);
  hipError_t e;
  if (whole) {
    p.w_qkv = static_cast<const uint16_t *>(w->q_k_v_proj);
    p.w_g = static_cast<const uint16_t *>(w->g_proj);
    p.x = x;
    p.w_norm = w_norm;
    p.w_o = static_cast<const uint16_t *>(w->o_proj);
    p.y = y;
    p.accumulate = accumulate ? 1 : 0;
    fused_tasks(p);
    e = launch_block_fused(p, stream);
    return e == hipSuccess ? GQA_OK : gpu_error(e, "one-launch block");
  }
  gqa_status st;
  const std::vector<SeqDesc> one(1, sd);
  if ((st = run_qkv_rope(a, w, is_full, one, x, q, gate, stream, w_norm)) != GQA_OK) return st;
  fused_tasks(p);
  if ((e = launch_block_fused(p, stream)) != hipSuccess) return gpu_error(e, "attention + merge launch");
  return run_o_proj(a, w, 1, attn, y, stream, accumulate);
}

// y0 (= or +=) W0 x and y1 (= or +=) W1 x for `batch` rows of x [batch][cols]
// (y0 [batch][rows0], y1 [batch][rows1]; w1 may be null): the MFMA kernel in
// groups of up to 32 rows from kMfmaMinBatch rows on (a short last group on
// the VALU GEMV), the VALU GEMV for smaller batches.
gqa_status run_proj(const uint16_t *w0, int rows0, const uint16_t *w1, int rows1, int cols, int batch,
                    const float *x, float *y0, float *y1, bool accumulate, hipStream_t stream, const char *what) {
  const int group = batch >= kMfmaMinBatch ? 32 : batch;
  for (int first = 0; first < batch; first += group) {
    GemvParams p{};
    p.w0 = w0;
    p.rows0 = rows0;
    p.w1 = w1;
    p.rows1 = w1 ? rows1 : 0;
    p.cols = cols;
    p.batch = std::min(group, batch - first);
    p.x = x + (size_t)first * cols;
    p.ldx = cols;
    p.y0 = y0 + (size_t)first * rows0;
    p.ldy0 = rows0;
    p.y1 = w1 ? y1 + (size_t)first * rows1 : nullptr;
    p.ldy1 = rows1;
    p.accumulate = accumulate ? 1 : 0;
    hipError_t e = p.batch >= kMfmaMinBatch ? launch_proj_mfma(p, stream) : launch_gemv(p, stream);
    if (e != hipSuccess) return gpu_error(e, what);
  }
  return GQA_OK;
}

// ---- the rest of the decoder layer: post-attention norm + gated MLP --------

gqa_status check_mlp(const gqa_arch *a, const gqa_mlp_weights *w, int32_t batch) {
  gqa_status st;
  if ((st = check_arch(a)) != GQA_OK) return st;
  if (!w) return fail(GQA_ERR_INVALID_ARGUMENT, "mlp weights is null");
  if (w->reserved != 0) return fail(GQA_ERR_INVALID_ARGUMENT, "mlp weights reserved must be 0");
  if (w->intermediate < 8 || w->intermediate % 8 != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "intermediate=%d must be a positive multiple of 8", w->intermediate);
  if (w->intermediate > kMaxHidden)
    return fail(GQA_ERR_UNSUPPORTED, "intermediate=%d exceeds the supported %d", w->intermediate, kMaxHidden);
  if (!(a->rms_eps >= 0.f) || !isfinite(a->rms_eps))
    return fail(GQA_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  if ((size_t)batch * std::max(a->hidden, w->intermediate) * sizeof(float) > kMaxBufferBytes)
    return fail(GQA_ERR_UNSUPPORTED, "batch=%d makes an activation larger than %u bytes", batch, kMaxBufferBytes);
  return GQA_OK;
}

// MLP workspace: [x fp32 [B][H] | gate [B][I] | up [B][I]]
size_t mlp_bytes(const gqa_arch *a, int32_t inter, int32_t batch) {
  return round_up((size_t)batch * a->hidden * sizeof(float), 256) +
         2 * round_up((size_t)batch * inter * sizeof(float), 256);
}

// Two layers of a stack whose attention runs alike: window, slot, chunking, RoPE.
bool same_shape(const StackDesc &a, const StackDesc &b) {
  return a.seq.kv_start == b.seq.kv_start && a.seq.n == b.seq.n && a.seq.ring == b.seq.ring &&
         a.seq.slot == b.seq.slot && a.seq.position == b.seq.position && a.seq.cache_bytes == b.seq.cache_bytes &&
         a.chunk == b.chunk && a.nchunks == b.nchunks && a.rotary_dim == b.rotary_dim &&
         a.log2_theta == b.log2_theta;
}

// The layer (h += block(RMSNorm(h) * w_norm)) for resolved sequences whose
// plan and workspace layout are known: the one-launch block when it takes
// them, else projections -> attention -> o_proj with the residual add.
gqa_status run_layer(const gqa_arch *arch, const gqa_layer_weights *weights, const uint16_t *w_norm, int is_full,
                     const std::vector<SeqDesc> &descs, const Plan &plan, float *h, char *ws, const Layout &L,
                     hipStream_t s) {
  const int32_t batch = (int32_t)descs.size();
  if (fused_attention(arch, plan, batch))
    return run_fused_block(arch, weights, is_full, descs[0], plan, h, w_norm, h, true, ws, L, s);
  float *q = reinterpret_cast<float *>(ws + L.q);
  float *gate = reinterpret_cast<float *>(ws + L.gate);
  float *attn = reinterpret_cast<float *>(ws + L.attn);
  float *part_o = reinterpret_cast<float *>(ws + L.part_o);
  float *part_ml = reinterpret_cast<float *>(ws + L.part_ml);
  gqa_status st;
  if ((st = run_qkv_rope(arch, weights, is_full, descs, h, q, gate, s, w_norm)) != GQA_OK) return st;
  if ((st = run_attention(arch, descs, plan, q, gate, weights->sinks, attn, part_o, part_ml, s)) != GQA_OK) return st;
  return run_o_proj(arch, weights, batch, attn, h, s, true);
}

// The block for resolved sequence descriptors (one per token or sequence):
// pointers and the workspace size are checked here, then qkv -> attention ->
// o_proj are enqueued.
gqa_status run_block(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                     const std::vector<SeqDesc> &descs, const float *x_normed, float *out, void *workspace,
                     size_t workspace_bytes, void *stream) {
  gqa_status st;
  const int32_t batch = (int32_t)descs.size();
  if ((st = check_ptr(x_normed, "x_normed")) != GQA_OK) return st;
  if ((st = check_ptr(out, "out")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const Plan plan = make_plan(descs, arch->num_kv_heads, true);
  const Layout L = block_layout(arch, batch, plan.max_group_chunks);
  if (workspace_bytes < L.total)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the block needs %zu", workspace_bytes,
                L.total);
  char *ws = static_cast<char *>(workspace);
  float *q = reinterpret_cast<float *>(ws + L.q);
  float *gate = reinterpret_cast<float *>(ws + L.gate);
  float *attn = reinterpret_cast<float *>(ws + L.attn);
  float *part_o = reinterpret_cast<float *>(ws + L.part_o);
  float *part_ml = reinterpret_cast<float *>(ws + L.part_ml);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fused_attention(arch, plan, batch))
    return run_fused_block(arch, weights, is_full, descs[0], plan, x_normed, nullptr, out, false, ws, L, s);
  if ((st = run_qkv_rope(arch, weights, is_full, descs, x_normed, q, gate, s)) != GQA_OK) return st;
  if ((st = run_attention(arch, descs, plan, q, gate, weights->sinks, attn, part_o, part_ml, s)) != GQA_OK)
    return st;
  return run_o_proj(arch, weights, batch, attn, out, s);
}
}  // namespace

gqa_status report(gqa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gqa_status block_workspace_need(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                                const gqa_kv_seq *seqs, int32_t batch, size_t *need) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, true, true)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  *need = batch == 0 ? 0 : block_layout(arch, batch, make_plan(descs, arch->num_kv_heads, true).max_group_chunks).total;
  return GQA_OK;
}
}  // namespace gqa

using namespace gqa;

extern "C" {

const char *gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARGUMENT: return "GQA_ERR_INVALID_ARGUMENT";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE_TOO_SMALL: return "GQA_ERR_WORKSPACE_TOO_SMALL";
    case GQA_ERR_GPU: return "GQA_ERR_GPU";
  }
  return "GQA_ERR_UNKNOWN";
}

const char *gqa_last_error(void) { return g_last_error.c_str(); }

gqa_status gqa_rope_params_for(int is_full, int32_t full_rotary_dim, int32_t head_dim, double full_theta,
                               double sliding_theta, int32_t *rotary_dim, double *theta) {
  if (!rotary_dim || !theta) return fail(GQA_ERR_INVALID_ARGUMENT, "null output pointer");
  if (head_dim < 2 || head_dim % 2 != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "head_dim=%d must be even and >= 2", head_dim);
  if (full_rotary_dim < 2 || full_rotary_dim % 2 != 0 || full_rotary_dim > head_dim)
    return fail(GQA_ERR_INVALID_ARGUMENT, "full_rotary_dim=%d must be even and in [2, head_dim]",
                full_rotary_dim);
  if (!(full_theta > 0.0) || !(sliding_theta > 0.0) || !isfinite(full_theta) || !isfinite(sliding_theta))
    return fail(GQA_ERR_INVALID_ARGUMENT, "thetas must be finite and > 0");
  if (is_full) {
    *rotary_dim = full_rotary_dim;
    *theta = full_theta;
  } else {
    *rotary_dim = head_dim;
    *theta = sliding_theta;
  }
  return ok();
}

gqa_status gqa_kv_window(int is_full, int32_t position, int32_t sliding_window, int32_t ring_capacity,
                         int32_t *seq_len, int32_t *kv_start, int32_t *active_ring) {
  if (!seq_len || !kv_start || !active_ring) return fail(GQA_ERR_INVALID_ARGUMENT, "null output pointer");
  gqa_status st = window_of(is_full, position, sliding_window, ring_capacity, seq_len, kv_start, active_ring);
  return st == GQA_OK ? ok() : st;
}

int32_t gqa_kv_slot(int32_t position, int32_t ring_capacity) {
  if (position < 0 || ring_capacity < 0) return -1;
  return ring_capacity > 0 ? position % ring_capacity : position;
}

gqa_status gqa_workspace_size(const gqa_arch *arch, int32_t batch, int32_t max_seq_len, size_t *bytes) {
  if (!bytes) return fail(GQA_ERR_INVALID_ARGUMENT, "bytes is null");
  gqa_status st = check_arch(arch);
  if (st != GQA_OK) return st;
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  if (max_seq_len < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "max_seq_len=%d must be >= 1", max_seq_len);
  // one launch group of kMaxSeqPerLaunch sequences is live at a time
  *bytes = block_layout(arch, batch, max_chunks(arch->num_kv_heads, batch, max_seq_len)).total;
  return ok();
}

gqa_status gqa_split_plan(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs, int32_t batch,
                          int allow_direct, int32_t *chunk_rows, int32_t *waves, int32_t *direct,
                          int32_t *groups, int32_t *max_group_chunks, int64_t *chunk_bound) {
  if (!chunk_rows || !waves || !direct || !groups || !max_group_chunks || !chunk_bound)
    return fail(GQA_ERR_INVALID_ARGUMENT, "null output pointer");
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if (batch < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 1", batch);
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  const Plan plan = make_plan(descs, arch->num_kv_heads, allow_direct != 0);
  int32_t longest = 1;
  for (int32_t b = 0; b < batch; ++b) longest = std::max(longest, seqs[b].position + 1);
  *chunk_rows = plan.chunk;
  *waves = plan.waves;
  *direct = plan.direct ? 1 : 0;
  *groups = (int32_t)plan.groups.size();
  *max_group_chunks = (int32_t)plan.max_group_chunks;
  *chunk_bound = (int64_t)max_chunks(arch->num_kv_heads, batch, longest);
  return ok();
}

gqa_status gqa_qkv_rope_kv(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                           const gqa_kv_seq *seqs, int32_t batch, const float *x, float *q_roped,
                           float *gate_logits, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, true, false)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if ((st = check_ptr(x, "x")) != GQA_OK) return st;
  if ((st = check_ptr(q_roped, "q_roped")) != GQA_OK) return st;
  if ((st = check_ptr(gate_logits, "gate_logits")) != GQA_OK) return st;
  st = run_qkv_rope(arch, weights, is_full, descs, x, q_roped, gate_logits, static_cast<hipStream_t>(stream));
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_o_proj_gemv(const gqa_arch *arch, const gqa_layer_weights *weights, int32_t batch,
                           const float *attn_gated, float *out, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, false, true)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if ((st = check_ptr(attn_gated, "attn_gated")) != GQA_OK) return st;
  if ((st = check_ptr(out, "out")) != GQA_OK) return st;
  st = run_o_proj(arch, weights, batch, attn_gated, out, static_cast<hipStream_t>(stream));
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_attention_gated(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs, int32_t batch,
                               const float *q_roped, const float *gate_logits, const float *sinks,
                               float *attn_gated, void *workspace, size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if ((st = check_ptr(q_roped, "q_roped")) != GQA_OK) return st;
  if ((st = check_ptr(gate_logits, "gate_logits")) != GQA_OK) return st;
  if ((st = check_ptr(attn_gated, "attn_gated")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const Plan plan = make_plan(descs, arch->num_kv_heads, true);
  const size_t need =
      kSyncBytes + partial_bytes_o(arch, plan.max_group_chunks) + partial_bytes_ml(arch, plan.max_group_chunks);
  if (workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the attention needs %zu",
                workspace_bytes, need);
  char *ws = static_cast<char *>(workspace);
  float *part_o = reinterpret_cast<float *>(ws + kSyncBytes);
  float *part_ml = reinterpret_cast<float *>(ws + kSyncBytes + partial_bytes_o(arch, plan.max_group_chunks));
  if (fused_attention(arch, plan, batch)) {
    // the block's attention + merge phase: the same kernel and order as the block
    FusedParams p = fused_params(arch, is_full, descs[0], plan, kPhaseAttn, q_roped, gate_logits, sinks, part_o,
                                 part_ml, attn_gated, ws);
    fused_tasks(p);
    hipError_t e = launch_block_fused(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : gpu_error(e, "attention + merge launch");
  }
  st = run_attention(arch, descs, plan, q_roped, gate_logits, sinks, attn_gated, part_o, part_ml,
                     static_cast<hipStream_t>(stream));
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_attention_partials(const gqa_arch *arch, int is_full, const gqa_kv_seq *seqs, int32_t batch,
                                  const float *q_roped, float *part_o, float *part_ml, int32_t max_chunks,
                                  int32_t *chunk_rows, int32_t *chunk_begin, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  if (batch > kMaxSeqPerLaunch)
    return fail(GQA_ERR_UNSUPPORTED, "batch=%d: the partial pass runs one launch group of at most %d sequences",
                batch, kMaxSeqPerLaunch);
  if (!chunk_rows) return fail(GQA_ERR_INVALID_ARGUMENT, "chunk_rows is null");
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if (!chunk_begin) return fail(GQA_ERR_INVALID_ARGUMENT, "chunk_begin is null");
  if ((st = check_ptr(q_roped, "q_roped")) != GQA_OK) return st;
  if ((st = check_ptr(part_o, "part_o")) != GQA_OK) return st;
  if ((st = check_ptr(part_ml, "part_ml")) != GQA_OK) return st;
  const Plan plan = make_plan(descs, arch->num_kv_heads, false);
  const Plan::Group &g = plan.groups[0];
  if (g.total_chunks > max_chunks)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "the partial pass writes %d chunks, max_chunks is %d", g.total_chunks,
                max_chunks);
  const AttnParams p = attn_params(arch, descs, plan, g, q_roped, nullptr, nullptr, part_o, part_ml);
  *chunk_rows = plan.chunk;
  for (int i = 0; i < batch; ++i) chunk_begin[i] = p.seq[i].chunk_begin;
  chunk_begin[batch] = g.total_chunks;
  hipError_t e = launch_attention_partials(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return gpu_error(e, "attention partial launch");
  return ok();
}

gqa_status gqa_attention_block_decode(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                                      const gqa_kv_seq *seqs, int32_t batch, const float *x_normed,
                                      float *out, void *workspace, size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, true, true)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  if (batch == 0) return ok();
  st = run_block(arch, weights, is_full, descs, x_normed, out, workspace, workspace_bytes, stream);
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_attention_block_chunk(const gqa_arch *arch, const gqa_layer_weights *weights, int is_full,
                                     const gqa_kv_seq *seq, int32_t m_tokens, const float *x_normed, float *out,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, true, true)) != GQA_OK) return st;
  if (!seq) return fail(GQA_ERR_INVALID_ARGUMENT, "seq is null");
  if (m_tokens < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "m_tokens=%d must be >= 1", m_tokens);
  if ((st = check_batch(arch, m_tokens)) != GQA_OK) return st;
  if (seq->position < 0 || seq->position > INT32_MAX - m_tokens)
    return fail(GQA_ERR_INVALID_ARGUMENT, "position=%d with m_tokens=%d: positions out of range", seq->position,
                m_tokens);
  if (seq->ring_capacity > 0 &&
      (int64_t)seq->ring_capacity < (int64_t)arch->sliding_window + m_tokens - 1)
    return fail(GQA_ERR_INVALID_ARGUMENT,
                "ring_capacity=%d < sliding_window + m_tokens - 1 = %lld: a later token's slot would overwrite a "
                "row an earlier token of the chunk reads",
                seq->ring_capacity, (long long)arch->sliding_window + m_tokens - 1);
  std::vector<gqa_kv_seq> toks((size_t)m_tokens, *seq);
  for (int32_t t = 0; t < m_tokens; ++t) toks[t].position = seq->position + t;
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, toks.data(), m_tokens, &descs)) != GQA_OK) return st;
  if (m_tokens == 1) {
    st = run_block(arch, weights, is_full, descs, x_normed, out, workspace, workspace_bytes, stream);
    return st == GQA_OK ? ok() : st;
  }
  if ((st = check_ptr(x_normed, "x_normed")) != GQA_OK) return st;
  if ((st = check_ptr(out, "out")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const ChunkPlan cp = make_chunk_plan(arch, is_full, seq->position, m_tokens);
  const Layout L = block_layout(arch, m_tokens, (size_t)m_tokens * cp.nchunks);
  if (workspace_bytes < L.total)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the chunk needs %zu", workspace_bytes,
                L.total);
  char *ws = static_cast<char *>(workspace);
  float *q = reinterpret_cast<float *>(ws + L.q);
  float *gate = reinterpret_cast<float *>(ws + L.gate);
  float *attn = reinterpret_cast<float *>(ws + L.attn);
  float *part_o = reinterpret_cast<float *>(ws + L.part_o);
  float *part_ml = reinterpret_cast<float *>(ws + L.part_ml);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // M-row projections: q, gate logits, and every token's k, v into its slot
  if ((st = run_qkv_rope(arch, weights, is_full, descs, x_normed, q, gate, s)) != GQA_OK) return st;
  const long q_dim = (long)arch->num_heads * arch->head_dim;
  ChunkAttnParams ca{};
  ca.q = q;
  ca.ld_q = q_dim;
  ca.part_o = part_o;
  ca.part_ml = part_ml;
  ca.num_kv_heads = arch->num_kv_heads;
  ca.qscale = (float)((double)arch->attention_scale * kLog2e);
  ca.m_tokens = m_tokens;
  ca.first_pos = seq->position;
  ca.window = cp.window;
  ca.r0 = cp.r0;
  ca.chunk = cp.chunk;
  ca.nchunks = cp.nchunks;
  ca.seq = descs[0];
  ca.seq.ring = seq->ring_capacity;   // physical row = position mod ring for every row, wrapped or not
  hipError_t e = launch_attention_chunk(ca, s);
  if (e != hipSuccess) return gpu_error(e, "chunk attention launch");
  // merge + gate per token, up to kMaxSeqPerLaunch tokens per launch
  for (int first = 0; first < m_tokens; first += kMaxSeqPerLaunch) {
    AttnParams ap{};
    const int cnt = std::min(kMaxSeqPerLaunch, m_tokens - first);
    const size_t rows0 = (size_t)first * cp.nchunks * arch->num_heads;
    ap.part_o = part_o + rows0 * kHeadDim;
    ap.part_ml = part_ml + rows0 * 2;
    ap.gate = gate + (size_t)first * arch->num_heads;
    ap.ld_gate = arch->num_heads;
    ap.sinks = weights->sinks;
    ap.out = attn + (size_t)first * q_dim;
    ap.ld_out = q_dim;
    ap.num_kv_heads = arch->num_kv_heads;
    ap.chunk = cp.chunk;
    ap.nseq = cnt;
    ap.total_chunks = cnt * cp.nchunks;
    for (int i = 0; i < cnt; ++i) {
      ap.seq[i] = descs[first + i];
      ap.seq[i].n = cp.rows;                  // every token: nchunks partials
      ap.seq[i].chunk_begin = i * cp.nchunks;
    }
    e = launch_combine(ap, arch->num_heads, s);
    if (e != hipSuccess) return gpu_error(e, "chunk merge launch");
  }
  st = run_o_proj(arch, weights, m_tokens, attn, out, s);
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_attention_layer_decode(const gqa_arch *arch, const gqa_layer_weights *weights, const void *w_norm,
                                      int is_full, const gqa_kv_seq *seqs, int32_t batch, float *h, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if ((st = check_weights(weights, true, true)) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  if (!(arch->rms_eps >= 0.f) || !isfinite(arch->rms_eps))
    return fail(GQA_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  std::vector<SeqDesc> descs;
  if ((st = resolve_seqs(arch, is_full, seqs, batch, &descs)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if ((st = check_ptr(w_norm, "w_norm")) != GQA_OK) return st;
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const Plan plan = make_plan(descs, arch->num_kv_heads, true);
  const Layout L = block_layout(arch, batch, plan.max_group_chunks);
  if (workspace_bytes < L.total)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the layer needs %zu", workspace_bytes,
                L.total);
  st = run_layer(arch, weights, static_cast<const uint16_t *>(w_norm), is_full, descs, plan, h,
                 static_cast<char *>(workspace), L, static_cast<hipStream_t>(stream));
  return st == GQA_OK ? ok() : st;
}

gqa_status gqa_attention_stack_decode(const gqa_arch *arch, const gqa_stack_layer *layers, int32_t num_layers,
                                      float *h, void *workspace, size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if (!(arch->rms_eps >= 0.f) || !isfinite(arch->rms_eps))
    return fail(GQA_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (num_layers < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "num_layers=%d must be >= 0", num_layers);
  if (num_layers == 0) return ok();
  if (!layers) return fail(GQA_ERR_INVALID_ARGUMENT, "layers is null");
  // every layer checked before anything is enqueued
  std::vector<std::vector<SeqDesc>> descs(num_layers);
  std::vector<Plan> plans(num_layers);
  size_t max_chunks = 0;
  for (int32_t l = 0; l < num_layers; ++l) {
    const gqa_stack_layer &ly = layers[l];
    if (ly.reserved != 0) return fail(GQA_ERR_INVALID_ARGUMENT, "layers[%d].reserved must be 0", l);
    if ((st = check_weights(&ly.weights, true, true)) != GQA_OK)
      return report(st, "layers[%d]: %s", l, gqa_last_error());
    if ((st = check_ptr(ly.w_norm, "w_norm")) != GQA_OK) return report(st, "layers[%d]: %s", l, gqa_last_error());
    if ((st = resolve_seqs(arch, ly.is_full, &ly.cache, 1, &descs[l])) != GQA_OK)
      return report(st, "layers[%d]: %s", l, gqa_last_error());
    plans[l] = make_plan(descs[l], arch->num_kv_heads, true);
    max_chunks = std::max(max_chunks, plans[l].max_group_chunks);
  }
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const Layout L = block_layout(arch, 1, max_chunks);
  if (workspace_bytes < L.total)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the stack needs %zu", workspace_bytes,
                L.total);
  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // runs of consecutive layers that the one-launch block takes go out as one
  // launch each (at most kStackMaxLayers layers and kStackMaxDescs attention
  // shapes); any other layer runs as gqa_attention_layer_decode runs it
  const bool whole = fused_whole(arch);
  int32_t l = 0;
  while (l < num_layers) {
    if (!whole || !fused_attention(arch, plans[l], 1)) {
      const gqa_stack_layer &ly = layers[l];
      if ((st = run_layer(arch, &ly.weights, static_cast<const uint16_t *>(ly.w_norm), ly.is_full, descs[l], plans[l],
                          h, ws, L, s)) != GQA_OK)
        return st;
      ++l;
      continue;
    }
    StackParams sp{};
    sp.base = fused_params(arch, layers[l].is_full, descs[l][0], plans[l], kPhaseQkv | kPhaseAttn | kPhaseOproj,
                           reinterpret_cast<float *>(ws + L.q), reinterpret_cast<float *>(ws + L.gate), nullptr,
                           reinterpret_cast<float *>(ws + L.part_o), reinterpret_cast<float *>(ws + L.part_ml),
                           reinterpret_cast<float *>(ws + L.attn), ws);
    sp.base.x = h;
    sp.base.y = h;
    sp.base.accumulate = 1;
    fused_tasks(sp.base);
    int nd = 0;
    while (l < num_layers && sp.num_layers < kStackMaxLayers && fused_attention(arch, plans[l], 1)) {
      const gqa_stack_layer &ly = layers[l];
      StackDesc d{};
      d.seq = descs[l][0];
      d.seq.k = nullptr;
      d.seq.v = nullptr;
      d.seq.chunk_begin = 0;
      d.chunk = plans[l].chunk;
      d.nchunks = plans[l].groups[0].total_chunks;
      d.t_attn = d.nchunks * arch->num_kv_heads;
      int32_t rdim;
      double theta;
      gqa_rope_params_for(ly.is_full, arch->full_rotary_dim, arch->head_dim, arch->full_rope_theta,
                          arch->rope_theta, &rdim, &theta);
      d.rotary_dim = rdim;
      d.log2_theta = log2(theta);
      int di = 0;
      while (di < nd && !same_shape(sp.tab.desc[di], d)) ++di;
      if (di == nd) {
        if (nd == kStackMaxDescs) break;   // a fifth shape starts the next launch
        sp.tab.desc[nd++] = d;
      }
      const int n = sp.num_layers++;
      sp.tab.desc_of[n] = (unsigned char)di;
      sp.t_attn_max = std::max(sp.t_attn_max, d.t_attn);
      sp.tab.w_norm[n] = static_cast<const uint16_t *>(ly.w_norm);
      sp.tab.w_qkv[n] = static_cast<const uint16_t *>(ly.weights.q_k_v_proj);
      sp.tab.w_g[n] = static_cast<const uint16_t *>(ly.weights.g_proj);
      sp.tab.w_o[n] = static_cast<const uint16_t *>(ly.weights.o_proj);
      sp.tab.k[n] = descs[l][0].k;
      sp.tab.v[n] = descs[l][0].v;
      sp.tab.sinks[n] = ly.weights.sinks;
      ++l;
    }
    sp.num_descs = nd;
    hipError_t e = launch_stack_fused(sp, s);
    if (e != hipSuccess) return gpu_error(e, "one-launch stack");
  }
  return ok();
}

gqa_status gqa_rms_norm_bf16w(const float *h, const void *w, float *out, int32_t rows, int32_t hidden,
                              float eps, void *stream) {
  gqa_status st;
  if (rows < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "rows=%d must be >= 0", rows);
  if (hidden < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "hidden=%d must be >= 1", hidden);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(GQA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (rows == 0) return ok();
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(w, "w")) != GQA_OK) return st;
  if ((st = check_ptr(out, "out")) != GQA_OK) return st;
  hipError_t e = launch_rms_norm(h, static_cast<const uint16_t *>(w), out, rows, hidden, eps,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : gpu_error(e, "rms_norm launch");
}

gqa_status gqa_residual_add(float *h, const float *o, int64_t n, void *stream) {
  gqa_status st;
  if (n < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (n == 0) return ok();
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(o, "o")) != GQA_OK) return st;
  hipError_t e = launch_residual_add(h, o, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : gpu_error(e, "residual_add launch");
}

}  // extern "C"

extern "C" {

gqa_status gqa_mlp_workspace_size(const gqa_arch *arch, int32_t intermediate, int32_t batch, size_t *bytes) {
  if (!bytes) return fail(GQA_ERR_INVALID_ARGUMENT, "bytes is null");
  gqa_mlp_weights w{};
  w.intermediate = intermediate;
  gqa_status st = check_mlp(arch, &w, batch);
  if (st != GQA_OK) return st;
  *bytes = mlp_bytes(arch, intermediate, batch);
  return ok();
}

gqa_status gqa_mlp_decode(const gqa_arch *arch, const gqa_mlp_weights *weights, int32_t batch, float *h,
                          void *workspace, size_t workspace_bytes, void *stream) {
  gqa_status st;
  if ((st = check_mlp(arch, weights, batch)) != GQA_OK) return st;
  if (batch == 0) return ok();
  if ((st = check_ptr(weights->post_attention_layernorm, "post_attention_layernorm")) != GQA_OK) return st;
  if ((st = check_ptr(weights->gate_proj, "gate_proj")) != GQA_OK) return st;
  if ((st = check_ptr(weights->up_proj, "up_proj")) != GQA_OK) return st;
  if ((st = check_ptr(weights->down_proj, "down_proj")) != GQA_OK) return st;
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  const int H = arch->hidden, I = weights->intermediate;
  const size_t need = mlp_bytes(arch, I, batch);
  if (workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the MLP needs %zu", workspace_bytes, need);
  char *ws = static_cast<char *>(workspace);
  float *x = reinterpret_cast<float *>(ws);
  float *gate = reinterpret_cast<float *>(ws + round_up((size_t)batch * H * sizeof(float), 256));
  float *up = reinterpret_cast<float *>(reinterpret_cast<char *>(gate) +
                                        round_up((size_t)batch * I * sizeof(float), 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (batch < kMfmaMinBatch) {
    // norm, gate and up projections and the activation in one launch, then the
    // down projection with the residual add
    MlpParams mp{};
    mp.w_post = static_cast<const uint16_t *>(weights->post_attention_layernorm);
    mp.w_gate = static_cast<const uint16_t *>(weights->gate_proj);
    mp.w_up = static_cast<const uint16_t *>(weights->up_proj);
    mp.h = h;
    mp.act = gate;
    mp.hidden = H;
    mp.inter = I;
    mp.batch = batch;
    mp.eps = arch->rms_eps;
    if ((e = launch_mlp_gate_up(mp, s)) != hipSuccess) return gpu_error(e, "norm + gate/up + activation launch");
    st = run_proj(static_cast<const uint16_t *>(weights->down_proj), H, nullptr, 0, I, batch, gate, h, nullptr, true,
                  s, "down projection launch");
    return st == GQA_OK ? ok() : st;
  }
  e = launch_rms_norm(h, static_cast<const uint16_t *>(weights->post_attention_layernorm), x, batch, H,
                      arch->rms_eps, s);
  if (e != hipSuccess) return gpu_error(e, "post-attention RMSNorm launch");
  if ((st = run_proj(static_cast<const uint16_t *>(weights->gate_proj), I,
                     static_cast<const uint16_t *>(weights->up_proj), I, H, batch, x, gate, up, false, s,
                     "gate/up projection launch")) != GQA_OK)
    return st;
  if ((e = launch_gelu_mul(gate, up, (int64_t)batch * I, s)) != hipSuccess) return gpu_error(e, "activation launch");
  if ((st = run_proj(static_cast<const uint16_t *>(weights->down_proj), H, nullptr, 0, I, batch, gate, h, nullptr,
                     true, s, "down projection launch")) != GQA_OK)
    return st;
  return ok();
}

}  // extern "C"

// ---- the ends of the decode step: embedding gather, final norm + tied head --

namespace gqa {
namespace {
gqa_status check_table(const gqa_arch *a, const void *table, int32_t vocab) {
  gqa_status st;
  if ((st = check_arch(a)) != GQA_OK) return st;
  if ((st = check_ptr(table, "embed_tokens")) != GQA_OK) return st;
  if (vocab < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "vocab=%d must be >= 1", vocab);
  if ((size_t)vocab * a->hidden * 2u > kMaxBufferBytes)
    return fail(GQA_ERR_UNSUPPORTED, "a %d x %d bf16 table exceeds %u bytes", vocab, a->hidden, kMaxBufferBytes);
  return GQA_OK;
}
}  // namespace
}  // namespace gqa

extern "C" {

gqa_status gqa_embed_tokens(const gqa_arch *arch, const void *embed_tokens, int32_t vocab, const int32_t *ids,
                            int32_t batch, float *h, void *stream) {
  gqa_status st;
  if ((st = check_table(arch, embed_tokens, vocab)) != GQA_OK) return st;
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  if (batch == 0) return ok();
  if (!ids) return fail(GQA_ERR_INVALID_ARGUMENT, "ids is null");
  for (int32_t b = 0; b < batch; ++b)
    if (ids[b] < 0 || ids[b] >= vocab)
      return fail(GQA_ERR_INVALID_ARGUMENT, "ids[%d]=%d is outside [0, %d)", b, ids[b], vocab);
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  for (int32_t first = 0; first < batch; first += kMaxEmbedIds) {
    EmbedParams p{};
    p.table = static_cast<const uint16_t *>(embed_tokens);
    p.h = h + (size_t)first * arch->hidden;
    p.hidden = arch->hidden;
    p.count = std::min<int32_t>(kMaxEmbedIds, batch - first);
    for (int i = 0; i < p.count; ++i) p.ids[i] = ids[first + i];
    hipError_t e = launch_embed_gather(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return gpu_error(e, "embedding gather launch");
  }
  return ok();
}

gqa_status gqa_lm_head_workspace_size(const gqa_arch *arch, int32_t batch, size_t *bytes) {
  if (!bytes) return fail(GQA_ERR_INVALID_ARGUMENT, "bytes is null");
  gqa_status st;
  if ((st = check_arch(arch)) != GQA_OK) return st;
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  *bytes = round_up((size_t)batch * arch->hidden * sizeof(float), 256);
  return ok();
}

gqa_status gqa_lm_head(const gqa_arch *arch, const void *final_norm, const void *embed_tokens, int32_t vocab,
                       const float *h, int32_t batch, float *logits, void *workspace, size_t workspace_bytes,
                       void *stream) {
  gqa_status st;
  if ((st = check_table(arch, embed_tokens, vocab)) != GQA_OK) return st;
  if (!(arch->rms_eps >= 0.f) || !isfinite(arch->rms_eps))
    return fail(GQA_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (batch < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "batch=%d must be >= 0", batch);
  if (batch == 0) return ok();
  if ((st = check_ptr(final_norm, "final_norm")) != GQA_OK) return st;
  if ((st = check_ptr(h, "h")) != GQA_OK) return st;
  if ((st = check_ptr(logits, "logits")) != GQA_OK) return st;
  if ((st = check_ptr(workspace, "workspace")) != GQA_OK) return st;
  if ((st = check_batch(arch, batch)) != GQA_OK) return st;
  if ((size_t)batch * vocab * sizeof(float) > kMaxBufferBytes)
    return fail(GQA_ERR_UNSUPPORTED, "batch=%d x vocab=%d logits exceed %u bytes", batch, vocab, kMaxBufferBytes);
  const size_t need = round_up((size_t)batch * arch->hidden * sizeof(float), 256);
  if (workspace_bytes < need)
    return fail(GQA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the head needs %zu", workspace_bytes, need);
  float *x = static_cast<float *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_rms_norm(h, static_cast<const uint16_t *>(final_norm), x, batch, arch->hidden, arch->rms_eps, s);
  if (e != hipSuccess) return gpu_error(e, "final RMSNorm launch");
  st = run_proj(static_cast<const uint16_t *>(embed_tokens), vocab, nullptr, 0, arch->hidden, batch, x, logits,
                nullptr, false, s, "tied head launch");
  return st == GQA_OK ? ok() : st;
}

}  // extern "C"

