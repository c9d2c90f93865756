"""fp64 CPU oracle of the hybrid-window GQA decode attention block.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library or its binding, and the product path never calls it.

Every function states the plain definition of one step, in float64, from the
same rounded bf16/fp16 inputs the GPU receives.  The sources are three docs.rs
pages of the crate turbospark-runtime 0.3.0, cited below as:

  [attn]  src/families/spark/attn.rs  (`encode_attention_block`,
          `rope_params_for`, its unit test, the module doc)
  [mod]   src/families/spark/mod.rs   (module doc: the transcribed decoder
          layer and the "does not have" list; `produce_real_spark_inner`)
  [kvw]   src/kv_write.rs             (`kv_write_target`, `encode_kv_commit`,
          `encode_attention_any`)

The rest of the decoder layer (post-attention RMSNorm, erf-GELU gated MLP,
residual add) follows [mod]'s transcribed layer; its intermediate size is not
on the pages, so inputs are synthetic (reading O21: W_gate, W_up [inter][hidden],
W_down [hidden][inter], row-major like O1).

Readings where the pages leave a step open (numbered O1..O23 throughout):
  O1 weights are row-major [out][in] and y = W x; O2 head h of a section is the
  contiguous block [256h, 256h+256); O3 query head h reads KV head
  h // (num_heads / num_kv_heads); O4 NeoX pairs (i, i + r/2) over the leading r
  dims with frequency theta^(-2i/r); O6 k and v are rounded to fp16 once, after
  RoPE; O9 the window is the last min(seq_len, 512) positions including this
  token; O10 ring slot = position mod ring_capacity; O13 RMSNorm multiplies by
  plain w.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force, a library SDPA).  The whole block on
trained weights is "parity unpinned" (no checkpoint or printed outputs exist).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf


# ----------------------------------------------------------------------------
# storage types
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of bf16 bit patterns: the high half of an IEEE binary32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_fp16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to IEEE binary16 (round-to-nearest-even, one rounding)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


# ----------------------------------------------------------------------------
# projections  [attn: encode_attention_block, fused QKV and g_proj GEMVs;
#               mod: transcribed layer, qkv = x @ q_k_v_proj, g = x @ g_proj]
# ----------------------------------------------------------------------------

def gemv(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[b, r] = sum_c W[r, c] * x[b, c]  (W row-major [rows][cols], reading O1)."""
    w = np.asarray(w, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ w.T


def split_qkv(qkv_row: np.ndarray, num_heads: int, num_kv_heads: int,
              head_dim: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """[attn: THE SPLIT; mod: rows are q | k | v] -> q [Hq][D], k [Hk][D], v [Hk][D].

    Sections in the order q (Hq*D rows), k (Hk*D), v (Hk*D); inside a section
    head h owns the contiguous rows [h*D, (h+1)*D) (reading O2).
    """
    q_dim = num_heads * head_dim
    kv_dim = num_kv_heads * head_dim
    q = qkv_row[:q_dim].reshape(num_heads, head_dim)
    k = qkv_row[q_dim:q_dim + kv_dim].reshape(num_kv_heads, head_dim)
    v = qkv_row[q_dim + kv_dim:q_dim + 2 * kv_dim].reshape(num_kv_heads, head_dim)
    return q, k, v


# ----------------------------------------------------------------------------
# RoPE  [attn: module doc item 2, `rope_params_for`, the per-class RoPE step]
# ----------------------------------------------------------------------------

def rope_params_for(is_full: bool, full_rotary_dim: int, head_dim: int,
                    full_theta: float, sliding_theta: float) -> Tuple[int, float]:
    """Full layers: (full_rotary_dim, full theta); sliding layers: (head_dim, sliding theta)."""
    if is_full:
        return int(full_rotary_dim), float(full_theta)
    return int(head_dim), float(sliding_theta)


def rope_neox(x: np.ndarray, position: int, rotary_dim: int, theta: float) -> np.ndarray:
    """NeoX rotation of the leading ``rotary_dim`` dims of every head of ``x``.

    x: [heads][head_dim].  Pair i (0 <= i < r/2) joins dims i and i + r/2 and
    turns by the angle position * theta^(-2i/r); the divisor is the rotary
    width r, not the head dim (HF partial-rotary convention).  Dims >= r are
    returned unchanged.  Angles are formed in float64 (reading O5).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    half = rotary_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / rotary_dim)
    angle = np.float64(position) * inv_freq
    c, s = np.cos(angle), np.sin(angle)
    lo = x[:, :half].copy()
    hi = x[:, half:rotary_dim].copy()
    x[:, :half] = lo * c - hi * s
    x[:, half:rotary_dim] = hi * c + lo * s
    return x


# ----------------------------------------------------------------------------
# window / ring  [attn: the window step after RoPE; kvw: `kv_write_target`,
#                 `encode_attention_any` reads the layer buffer from row 0]
# ----------------------------------------------------------------------------

def kv_window(is_full: bool, position: int, sliding_window: int,
              ring_capacity: int) -> Tuple[int, int, int]:
    """(seq_len, kv_start, active_ring) of one decode step.

    seq_len = position + 1.  Full layers attend causally over everything:
    (kv_start, ring) = (0, 0).  Sliding layers start at seq_len - window
    (clamped at 0) and use ring addressing only once the history is longer
    than the ring; before that the ring is identity addressing.
    """
    seq_len = position + 1
    if is_full:
        return seq_len, 0, 0
    kv_start = max(seq_len - sliding_window, 0)
    active = ring_capacity if (ring_capacity > 0 and seq_len > ring_capacity) else 0
    return seq_len, kv_start, active


def kv_slot(position: int, ring_capacity: int) -> int:
    """Physical cache row of ``position`` (reading O10): mod ring, identity if no ring."""
    return position % ring_capacity if ring_capacity > 0 else position


def physical_rows(seq_len: int, kv_start: int, active_ring: int) -> np.ndarray:
    """Physical rows read for logical positions kv_start .. seq_len-1, in order."""
    t = np.arange(kv_start, seq_len, dtype=np.int64)
    return t % active_ring if active_ring > 0 else t


# ----------------------------------------------------------------------------
# attention  [attn: `encode_attention_any` call; kvw: `encode_attention_any`;
#             mod: attention with scale 256^-0.5, window 512 or causal]
# ----------------------------------------------------------------------------

def attention_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     seq_len: int, kv_start: int, active_ring: int,
                     scale: float, sinks=None) -> np.ndarray:
    """Softmax attention of one query per head over the cache window.

    q [Hq][D]; caches [capacity][Hk][D].  Query head h reads KV head
    h // (Hq / Hk) (reading O3).  No softcap, no bias.

    ``sinks`` (optional, [Hq]): the attention-sink operand that the attention
    call takes and the pages leave unset [attn: the attention step passes no
    sinks; kvw: `encode_attention_any` signature].  Reading O23: sink
    sigma_h is one more logit in head h's softmax, in the units of the scaled
    scores, with no value row: p_t = e^{s_t} / (sum_u e^{s_u} + e^{sigma_h}).
    """
    num_heads, head_dim = q.shape
    num_kv = k_cache.shape[1]
    group = num_heads // num_kv
    rows = physical_rows(seq_len, kv_start, active_ring)
    out = np.zeros((num_heads, head_dim), dtype=np.float64)
    for h in range(num_heads):
        g = h // group
        kk = np.asarray(k_cache[rows, g, :], dtype=np.float64)
        vv = np.asarray(v_cache[rows, g, :], dtype=np.float64)
        s = scale * (kk @ np.asarray(q[h], dtype=np.float64))
        if sinks is None:
            p = np.exp(s - s.max())
            p /= p.sum()
        else:
            sig = float(sinks[h])
            ref = max(float(s.max()), sig)
            p = np.exp(s - ref)
            p = p / (p.sum() + np.exp(sig - ref))
        out[h] = p @ vv
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))


def head_gate(attn: np.ndarray, gate_logits: np.ndarray) -> np.ndarray:
    """[attn: module doc item 3, gate step] attn[h, :] * sigmoid(g[h]), before o_proj."""
    return attn * sigmoid(gate_logits)[:, None]


# ----------------------------------------------------------------------------
# the block  [attn: `encode_attention_block`, steps in its order]
# ----------------------------------------------------------------------------

@dataclass
class OracleSeq:
    k: np.ndarray            # float16 [capacity][Hk][D] (copied, updated by the call)
    v: np.ndarray
    ring_capacity: int
    position: int


@dataclass
class AttentionStepResult:
    q_roped: np.ndarray      # [B][Hq][D]
    k16: np.ndarray          # [B][Hk][D] float16: the row written to the slot
    v16: np.ndarray          # [B][Hk][D] float16
    slots: List[int]
    windows: List[Tuple[int, int, int]]
    attn: np.ndarray         # [B][Hq][D] before the gate
    gated: np.ndarray        # [B][Hq*D]
    k_caches: List[np.ndarray]
    v_caches: List[np.ndarray]


@dataclass
class BlockResult(AttentionStepResult):
    qkv: np.ndarray = None          # [B][qkv_rows]
    gate_logits: np.ndarray = None  # [B][Hq]
    out: np.ndarray = None          # [B][hidden]


def attention_step(arch, is_full: bool, qkv: np.ndarray, gate_logits: np.ndarray,
                   seqs: Sequence, sinks=None) -> AttentionStepResult:
    """Everything between the projections and o_proj, per sequence b:

    split qkv[b] [attn: THE SPLIT]; RoPE q and k with the layer class's
    (rotary_dim, theta) [attn: per-class RoPE step] -- v is not rotated;
    write fp16 k and v into the slot of this position [attn: k and v land in
    their cache slots; kvw: `kv_write_target`]; attend over the window
    [attn: window step, `encode_attention_any`]; apply the headwise gate
    [attn: gate step].  Each element of ``seqs`` exposes k, v (fp16 caches),
    ring_capacity and position; caches are copied and the copies updated.
    ``sinks``: optional per-head sink logits (``attention_decode``).
    """
    hq, hk, d = arch.num_heads, arch.num_kv_heads, arch.head_dim
    qkv = np.atleast_2d(np.asarray(qkv, dtype=np.float64))
    gl = np.atleast_2d(np.asarray(gate_logits, dtype=np.float64))
    rotary_dim, theta = rope_params_for(is_full, arch.full_rotary_dim, d,
                                        arch.full_rope_theta, arch.rope_theta)
    res = dict(q_roped=[], k16=[], v16=[], slots=[], windows=[], attn=[],
               gated=[], k_caches=[], v_caches=[])
    for b, seq in enumerate(seqs):
        pos = int(seq.position)
        q, k, v = split_qkv(qkv[b], hq, hk, d)
        q_r = rope_neox(q, pos, rotary_dim, theta)
        k_r = rope_neox(k, pos, rotary_dim, theta)        # v is not rotated
        k16, v16 = to_fp16(k_r), to_fp16(v)
        kc = np.array(seq.k, dtype=np.float16, copy=True)
        vc = np.array(seq.v, dtype=np.float16, copy=True)
        slot = kv_slot(pos, int(seq.ring_capacity))
        kc[slot] = k16
        vc[slot] = v16
        win = kv_window(is_full, pos, arch.sliding_window, int(seq.ring_capacity))
        a = attention_decode(q_r, kc, vc, win[0], win[1], win[2], arch.attention_scale, sinks)
        res["q_roped"].append(q_r)
        res["k16"].append(k16)
        res["v16"].append(v16)
        res["slots"].append(slot)
        res["windows"].append(win)
        res["attn"].append(a)
        res["gated"].append(head_gate(a, gl[b]).reshape(hq * d))
        res["k_caches"].append(kc)
        res["v_caches"].append(vc)
    return AttentionStepResult(
        q_roped=np.stack(res["q_roped"]), k16=np.stack(res["k16"]),
        v16=np.stack(res["v16"]), slots=res["slots"], windows=res["windows"],
        attn=np.stack(res["attn"]), gated=np.stack(res["gated"]),
        k_caches=res["k_caches"], v_caches=res["v_caches"])


def block_decode(arch, is_full: bool, w_qkv_bits, w_g_bits, w_o_bits,
                 x: np.ndarray, seqs: Sequence, sinks=None) -> BlockResult:
    """One decode step of the attention block for B independent sequences
    [attn: `encode_attention_block`, steps in its order].

    ``arch`` exposes num_heads, num_kv_heads, head_dim, full_rotary_dim,
    sliding_window, full_rope_theta, rope_theta and attention_scale.  The fused
    QKV GEMV and the g_proj GEMV read the same normed x; o_proj reads the
    gated attention.  ``sinks``: optional per-head sink logits.
    """
    w_qkv = bf16_bits_to_f64(w_qkv_bits)
    w_g = bf16_bits_to_f64(w_g_bits)
    w_o = bf16_bits_to_f64(w_o_bits)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    qkv = gemv(w_qkv, x)
    gl = gemv(w_g, x)
    st = attention_step(arch, is_full, qkv, gl, seqs, sinks)
    out = gemv(w_o, st.gated)
    return BlockResult(q_roped=st.q_roped, k16=st.k16, v16=st.v16, slots=st.slots,
                       windows=st.windows, attn=st.attn, gated=st.gated,
                       k_caches=st.k_caches, v_caches=st.v_caches, qkv=qkv,
                       gate_logits=gl, out=out)


# ----------------------------------------------------------------------------
# several tokens of one sequence  [mod: the family's `prefill` module; kvw:
#   module doc -- chunked prefill runs the per-token block token after token]
# ----------------------------------------------------------------------------

@dataclass
class ChunkResult:
    out: np.ndarray          # [M][hidden]
    k_cache: np.ndarray      # float16 cache after all M tokens
    v_cache: np.ndarray
    slots: List[int]


def block_chunk(arch, is_full: bool, w_qkv_bits, w_g_bits, w_o_bits,
                x: np.ndarray, seq, m_tokens: int, sinks=None) -> ChunkResult:
    """M consecutive tokens of one sequence at positions seq.position + t.

    Token t is the single-token block at its position, run once tokens
    0 .. t-1 have written their cache slots, so it sees them and nothing
    later.  ``seq`` exposes k, v (fp16 caches), ring_capacity and position;
    the caches are copied.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    k = np.array(seq.k, dtype=np.float16, copy=True)
    v = np.array(seq.v, dtype=np.float16, copy=True)
    outs, slots = [], []
    for t in range(m_tokens):
        cur = OracleSeq(k=k, v=v, ring_capacity=int(seq.ring_capacity),
                        position=int(seq.position) + t)
        r = block_decode(arch, is_full, w_qkv_bits, w_g_bits, w_o_bits, x[t:t + 1], [cur], sinks)
        k, v = r.k_caches[0], r.v_caches[0]
        outs.append(r.out[0])
        slots.append(r.slots[0])
    return ChunkResult(out=np.stack(outs), k_cache=k, v_cache=v, slots=slots)


# ----------------------------------------------------------------------------
# stack harness  [mod: `produce_real_spark_inner` layer loop: input RMSNorm with
#                 bf16 weight and eps 1e-6, the block, raw residual add]
# ----------------------------------------------------------------------------

def rms_norm(h: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * w, with plain w (reading O13)."""
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    w = bf16_bits_to_f64(w_bits)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * w


@dataclass
class StackResult:
    h: np.ndarray                 # [1][hidden] after the last layer
    block_outs: List[np.ndarray]  # per layer o [1][hidden]
    normed: List[np.ndarray]      # per layer block input


def stack_decode(arch, h0: np.ndarray, layers: Sequence) -> StackResult:
    """Attention-only layer stack: h += block(rms(h) * w) per layer, batch 1.

    Each layer exposes is_full, w_norm, w_qkv, w_g, w_o and cache (with k, v,
    ring_capacity, position).
    """
    h = np.atleast_2d(np.asarray(h0, dtype=np.float64)).copy()
    outs, normed = [], []
    for layer in layers:
        xn = rms_norm(h, layer.w_norm, arch.rms_eps)
        r = block_decode(arch, layer.is_full, layer.w_qkv, layer.w_g, layer.w_o,
                         xn, [layer.cache])
        h = h + r.out
        outs.append(r.out)
        normed.append(xn)
    return StackResult(h=h, block_outs=outs, normed=normed)


# ----------------------------------------------------------------------------
# the rest of the decoder layer  [mod: module doc, transcribed layer -- after
#   the attention's raw residual add: x = rms(h, post_attention_layernorm,
#   1e-6); h = h + down(gelu_erf(x @ gate_proj) * (x @ up_proj)); the family's
#   GELU is the erf form (the module doc's closing remark on mlp.rs)]
# ----------------------------------------------------------------------------

def gelu_erf(x: np.ndarray) -> np.ndarray:
    """x * Phi(x) = x / 2 * (1 + erf(x / sqrt(2))): the exact (erf) GELU, not
    the tanh approximation."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


@dataclass
class MlpResult:
    h: np.ndarray        # [B][hidden] residual stream after the MLP's add
    x: np.ndarray        # post-attention-normed input [B][hidden]
    gate: np.ndarray     # x @ gate_proj  [B][inter]
    up: np.ndarray       # x @ up_proj    [B][inter]
    act: np.ndarray      # gelu_erf(gate) * up
    out: np.ndarray      # down(act): the MLP's contribution [B][hidden]


def mlp_decode(h: np.ndarray, w_post_bits, w_gate_bits, w_up_bits, w_down_bits,
               eps: float) -> MlpResult:
    """[mod: transcribed layer, last two lines] for B rows of the residual stream."""
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    x = rms_norm(h, w_post_bits, eps)
    gate = gemv(bf16_bits_to_f64(w_gate_bits), x)
    up = gemv(bf16_bits_to_f64(w_up_bits), x)
    act = gelu_erf(gate) * up
    out = gemv(bf16_bits_to_f64(w_down_bits), act)
    return MlpResult(h=h + out, x=x, gate=gate, up=up, act=act, out=out)


def decoder_stack_decode(arch, h0: np.ndarray, layers: Sequence) -> StackResult:
    """Whole decoder layers, batch 1 [mod: transcribed layer]: per layer
    h += block(rms(h) * w_norm), then h += mlp(h).  Each layer exposes the
    attention fields of ``stack_decode`` plus w_post, w_gate, w_up, w_down.
    ``block_outs`` holds each layer's total contribution (attention + MLP)."""
    h = np.atleast_2d(np.asarray(h0, dtype=np.float64)).copy()
    outs, normed = [], []
    for layer in layers:
        xn = rms_norm(h, layer.w_norm, arch.rms_eps)
        r = block_decode(arch, layer.is_full, layer.w_qkv, layer.w_g, layer.w_o,
                         xn, [layer.cache])
        h_mid = h + r.out
        m = mlp_decode(h_mid, layer.w_post, layer.w_gate, layer.w_up, layer.w_down,
                       arch.rms_eps)
        outs.append(m.h - h)
        normed.append(xn)
        h = m.h
    return StackResult(h=h, block_outs=outs, normed=normed)


# ----------------------------------------------------------------------------
# the ends of the decode step  [mod: `produce_real_spark_inner` -- the token's
#   embedding row is used raw (no sqrt(hidden) scale, no embedding norm); after
#   the last layer the final RMSNorm (model.norm, plain w) and the TIED head,
#   logits = x @ embed_tokens^T, raw logits; vocab is not on the pages
#   (reading O22: synthetic)]
# ----------------------------------------------------------------------------

def embed_gather(e_bits: np.ndarray, ids) -> np.ndarray:
    """h[b] = embed_tokens[ids[b]], the bf16 row as it is."""
    return bf16_bits_to_f64(np.asarray(e_bits)[np.asarray(ids, dtype=np.int64)])


def lm_head(h: np.ndarray, w_final_bits: np.ndarray, e_bits: np.ndarray, eps: float) -> np.ndarray:
    """logits[b] = rms(h[b], model.norm) @ embed_tokens^T  [vocab per row]."""
    x = rms_norm(h, w_final_bits, eps)
    return gemv(bf16_bits_to_f64(e_bits), x)
