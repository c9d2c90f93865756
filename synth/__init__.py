"""Seeded synthetic inputs for the hybrid-window GQA decode attention block.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds BOTH the HIP library and the fp64 oracle.  It therefore holds none of the
block's arithmetic: it only draws random numbers, rounds the drawn fp32 values
to the storage types the block consumes (bf16 weights, fp16 KV cache), and
arranges them in the layouts the boundary documents.

Layouts (all row-major, C order):
  * ``w_qkv``  uint16 bf16 bits ``[q_dim + 2*kv_dim][hidden]`` (rows q | k | v)
  * ``w_g``    uint16 bf16 bits ``[num_heads][hidden]``
  * ``w_o``    uint16 bf16 bits ``[hidden][q_dim]``
  * ``w_norm`` uint16 bf16 bits ``[hidden]`` (stack cases only)
  * MLP (decoder stack cases): ``w_post`` bf16 ``[hidden]``, ``w_gate`` and
    ``w_up`` bf16 ``[inter][hidden]``, ``w_down`` bf16 ``[hidden][inter]``
  * ``x``      float32 ``[batch][hidden]`` (already-normed block input)
  * per sequence ``k``/``v`` float16 ``[capacity][num_kv_heads][head_dim]``

Every tensor has its own stream ``numpy.random.default_rng([seed, case_id,
tensor_id])`` so that adding a tensor never changes another one.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# Model shape of the spark2_5 family block (docs.rs turbospark-runtime 0.3.0,
# src/families/spark/mod.rs module doc: 16 query heads over 4 KV heads at
# head_dim 256, window 512; the per-class RoPE widths/thetas are in
# src/families/spark/attn.rs, `rope_params_for` and its unit test).
NUM_HEADS = 16
NUM_KV_HEADS = 4
HEAD_DIM = 256
FULL_ROTARY_DIM = 64
SLIDING_WINDOW = 512
FULL_ROPE_THETA = 5.0e6
ROPE_THETA = 1.0e4
ATTENTION_SCALE = 0.0625          # 256 ** -0.5, exact in binary
RMS_EPS = 1e-6
Q_DIM = NUM_HEADS * HEAD_DIM      # 4096
KV_DIM = NUM_KV_HEADS * HEAD_DIM  # 1024
QKV_ROWS = Q_DIM + 2 * KV_DIM     # 6144

WEIGHT_STD = 0.02

# tensor ids inside one case (per-layer / per-sequence ids are offset below)
_T_WQKV, _T_WG, _T_WO, _T_WNORM, _T_X, _T_K, _T_V, _T_LEN, _T_H = range(9)


@dataclass
class Arch:
    hidden: int
    num_heads: int = NUM_HEADS
    num_kv_heads: int = NUM_KV_HEADS
    head_dim: int = HEAD_DIM
    full_rotary_dim: int = FULL_ROTARY_DIM
    sliding_window: int = SLIDING_WINDOW
    full_rope_theta: float = FULL_ROPE_THETA
    rope_theta: float = ROPE_THETA
    attention_scale: float = ATTENTION_SCALE
    rms_eps: float = RMS_EPS

    @property
    def q_dim(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return self.q_dim + 2 * self.kv_dim


@dataclass
class SeqCache:
    """One sequence's cache for one layer, before the call writes this token."""
    k: np.ndarray            # float16 [capacity][num_kv_heads][head_dim]
    v: np.ndarray            # float16 [capacity][num_kv_heads][head_dim]
    ring_capacity: int       # 0 = linear addressing, else ring slots
    position: int            # this token's position

    @property
    def capacity(self) -> int:
        return int(self.k.shape[0])


@dataclass
class BlockCase:
    name: str
    arch: Arch
    is_full: bool
    w_qkv: np.ndarray        # uint16 bf16 bits
    w_g: np.ndarray          # uint16 bf16 bits
    w_o: np.ndarray          # uint16 bf16 bits
    x: np.ndarray            # float32 [batch][hidden]
    seqs: List[SeqCache] = field(default_factory=list)

    @property
    def batch(self) -> int:
        return int(self.x.shape[0])


@dataclass
class StackLayer:
    is_full: bool
    w_norm: np.ndarray       # uint16 bf16 bits [hidden]
    w_qkv: np.ndarray
    w_g: np.ndarray
    w_o: np.ndarray
    cache: SeqCache


@dataclass
class StackCase:
    name: str
    arch: Arch
    h: np.ndarray            # float32 [1][hidden] residual stream entering layer 0
    layers: List[StackLayer] = field(default_factory=list)


# ----------------------------------------------------------------------------
# storage rounding of drawn inputs
# ----------------------------------------------------------------------------

def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def round_to_fp16(a: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16, round-to-nearest-even (numpy's cast)."""
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def _rng(seed: int, case_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, case_id, tensor_id])


def _normal(seed, case_id, tensor_id, shape, std=1.0, mean=0.0) -> np.ndarray:
    r = _rng(seed, case_id, tensor_id)
    out = r.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def _weights(arch: Arch, seed: int, case_id: int, base: int):
    w_qkv = round_to_bf16_bits(_normal(seed, case_id, base + _T_WQKV,
                                       (arch.qkv_rows, arch.hidden), WEIGHT_STD))
    w_g = round_to_bf16_bits(_normal(seed, case_id, base + _T_WG,
                                     (arch.num_heads, arch.hidden), WEIGHT_STD))
    w_o = round_to_bf16_bits(_normal(seed, case_id, base + _T_WO,
                                     (arch.hidden, arch.q_dim), WEIGHT_STD))
    return w_qkv, w_g, w_o


def make_cache(arch: Arch, seed: int, case_id: int, tensor_base: int,
               capacity: int, ring_capacity: int, position: int) -> SeqCache:
    """A cache whose every row holds N(0,1) fp16 values.

    Rows that the block reads stand for earlier tokens' keys/values; the row
    at this token's slot is overwritten by the call.
    """
    shape = (capacity, arch.num_kv_heads, arch.head_dim)
    k = round_to_fp16(_normal(seed, case_id, tensor_base + _T_K, shape))
    v = round_to_fp16(_normal(seed, case_id, tensor_base + _T_V, shape))
    return SeqCache(k=k, v=v, ring_capacity=ring_capacity, position=position)


def block_case(name: str, hidden: int, is_full: bool, positions, *,
               capacities=None, ring_capacity: int = 0, seed: int = 0,
               case_id: int = 0, arch: "Arch | None" = None) -> BlockCase:
    """General single-layer case: one cache per entry of ``positions``.

    ``capacities`` defaults to ``position + 1`` (linear) or ``ring_capacity``.
    ``arch`` (its hidden must equal ``hidden``) replaces the family's head counts.
    """
    if arch is None:
        arch = Arch(hidden=hidden)
    assert arch.hidden == hidden
    positions = [int(p) for p in positions]
    w_qkv, w_g, w_o = _weights(arch, seed, case_id, 0)
    x = _normal(seed, case_id, _T_X, (len(positions), hidden))
    seqs = []
    for i, p in enumerate(positions):
        if capacities is not None:
            cap = int(capacities[i])
        elif ring_capacity > 0:
            cap = ring_capacity
        else:
            cap = p + 1
        seqs.append(make_cache(arch, seed, case_id, 100 + 16 * i, cap,
                               ring_capacity, p))
    return BlockCase(name=name, arch=arch, is_full=is_full, w_qkv=w_qkv,
                     w_g=w_g, w_o=w_o, x=x, seqs=seqs)


# ----------------------------------------------------------------------------
# the five named workloads and the long-context headline
# ----------------------------------------------------------------------------

def cfg1_sliding_pos63(seed: int = 0) -> BlockCase:
    """Sliding layer, hidden 1024, position 63, 64-row cache (window not yet full)."""
    return block_case("cfg1_sliding_pos63", 1024, False, [63], capacities=[64],
                      ring_capacity=0, seed=seed, case_id=1)


def cfg2_full_pos4095(seed: int = 0) -> BlockCase:
    """Full layer, hidden 2560, position 4095, 4096-row linear cache."""
    return block_case("cfg2_full_pos4095", 2560, True, [4095], seed=seed, case_id=2)


def cfg3_sliding_ring_pos32767(seed: int = 0) -> BlockCase:
    """Sliding layer, hidden 1024, position 32767 on a wrapped 512-slot ring."""
    return block_case("cfg3_sliding_ring_pos32767", 1024, False, [32767],
                      ring_capacity=SLIDING_WINDOW, seed=seed, case_id=3)


def cfg5_lengths(seed: int = 0, batch: int = 32, max_len: int = 16384) -> np.ndarray:
    """Context lengths of the batched case, uniform on [1, max_len] inclusive."""
    return _rng(seed, 5, _T_LEN).integers(1, max_len + 1, size=batch)


def cfg5_batched_full(seed: int = 0) -> BlockCase:
    """32 independent sequences on one full layer, hidden 2560.

    Sequence i has context length L_i: its position is L_i - 1 and its linear
    cache holds L_i rows (the last row is written by the call).
    """
    lengths = cfg5_lengths(seed)
    return block_case("cfg5_batched_full_m32", 2560, True, [int(n) - 1 for n in lengths],
                      seed=seed, case_id=5)


def headline_full_pos32767(seed: int = 0) -> BlockCase:
    """Full layer at 32K context: hidden 2560, position 32767, 32768-row cache."""
    return block_case("full_layer_h2560_pos32767", 2560, True, [32767], seed=seed,
                      case_id=6)


def stack_layer_is_full(layer: int, phase_full_first: bool = False) -> bool:
    """3 sliding : 1 full pattern; default phase puts the full layer last."""
    return (layer % 4 == 0) if phase_full_first else (layer % 4 == 3)


def cfg4_stack(seed: int = 0, num_layers: int = 36, position: int = 8191,
               hidden: int = 2560, phase_full_first: bool = False,
               case_id: int = 4) -> StackCase:
    """Stack of attention blocks (no MLP) at one position, batch 1."""
    arch = Arch(hidden=hidden)
    h = _normal(seed, case_id, _T_H, (1, hidden))
    layers = []
    for li in range(num_layers):
        base = 1000 + 32 * li
        full = stack_layer_is_full(li, phase_full_first)
        w_qkv, w_g, w_o = _weights(arch, seed, case_id, base)
        w_norm = round_to_bf16_bits(_normal(seed, case_id, base + _T_WNORM,
                                            (hidden,), 0.1, 1.0))
        if full:
            cache = make_cache(arch, seed, case_id, base, position + 1, 0, position)
        else:
            cache = make_cache(arch, seed, case_id, base, SLIDING_WINDOW,
                               SLIDING_WINDOW, position)
        layers.append(StackLayer(is_full=full, w_norm=w_norm, w_qkv=w_qkv,
                                 w_g=w_g, w_o=w_o, cache=cache))
    return StackCase(name=f"cfg4_stack{num_layers}_pos{position}", arch=arch,
                     h=h, layers=layers)


NAMED_BLOCK_CASES = {
    "cfg1": cfg1_sliding_pos63,
    "cfg2": cfg2_full_pos4095,
    "cfg3": cfg3_sliding_ring_pos32767,
    "cfg5": cfg5_batched_full,
    "full32k": headline_full_pos32767,
}


def random_qkv(arch: Arch, batch: int, seed: int, case_id: int) -> np.ndarray:
    """fp32 [batch][qkv_rows] ~ N(0,1): a stand-in projection output for step tests."""
    return _normal(seed, case_id, 900, (batch, arch.qkv_rows))


def random_gate_logits(arch: Arch, batch: int, seed: int, case_id: int) -> np.ndarray:
    return _normal(seed, case_id, 901, (batch, arch.num_heads))


def random_sinks(arch: Arch, seed: int, case_id: int, lo: float = -2.0, hi: float = 14.0) -> np.ndarray:
    """Per-head attention-sink logits, fp32 [num_heads], uniform on [lo, hi).
    The log of a window's partition function runs from about 1 (a few rows)
    to about 11 (32K rows) on these inputs, so across the heads the sink takes
    anything from a negligible share to most of the softmax."""
    return _rng(seed, case_id, 904).uniform(lo, hi, arch.num_heads).astype(np.float32)


def random_hidden(hidden: int, batch: int, seed: int, case_id: int,
                  tensor_id: int = 902, std: float = 1.0) -> np.ndarray:
    return _normal(seed, case_id, tensor_id, (batch, hidden), std)


def random_bf16(shape, seed: int, case_id: int, tensor_id: int,
                std: float = WEIGHT_STD, mean: float = 0.0) -> np.ndarray:
    return round_to_bf16_bits(_normal(seed, case_id, tensor_id, shape, std, mean))


# ----------------------------------------------------------------------------
# the rest of the decoder layer (post-attention norm + gated MLP); the pages
# print no intermediate size, so it is taken as 3 * hidden here
# ----------------------------------------------------------------------------

_T_WPOST, _T_WGATE, _T_WUP, _T_WDOWN = 16, 17, 18, 19   # inside a layer's block of 32 ids


def mlp_inter(hidden: int) -> int:
    return 3 * hidden


@dataclass
class MlpWeights:
    w_post: np.ndarray   # uint16 bf16 bits [hidden] (post_attention_layernorm)
    w_gate: np.ndarray   # uint16 bf16 bits [inter][hidden]
    w_up: np.ndarray     # uint16 bf16 bits [inter][hidden]
    w_down: np.ndarray   # uint16 bf16 bits [hidden][inter]

    @property
    def inter(self) -> int:
        return int(self.w_gate.shape[0])


def make_mlp(hidden: int, inter: int, seed: int, case_id: int, base: int) -> MlpWeights:
    """Norm weight ~ N(1, 0.1), projections ~ N(0, 0.02), rounded to bf16."""
    return MlpWeights(
        w_post=round_to_bf16_bits(_normal(seed, case_id, base + _T_WPOST, (hidden,), 0.1, 1.0)),
        w_gate=round_to_bf16_bits(_normal(seed, case_id, base + _T_WGATE, (inter, hidden), WEIGHT_STD)),
        w_up=round_to_bf16_bits(_normal(seed, case_id, base + _T_WUP, (inter, hidden), WEIGHT_STD)),
        w_down=round_to_bf16_bits(_normal(seed, case_id, base + _T_WDOWN, (hidden, inter), WEIGHT_STD)))


@dataclass
class DecoderLayer:
    """A whole decoder layer: the attention fields of StackLayer plus the MLP."""
    is_full: bool
    w_norm: np.ndarray
    w_qkv: np.ndarray
    w_g: np.ndarray
    w_o: np.ndarray
    cache: SeqCache
    w_post: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


def decoder_stack(seed: int = 0, num_layers: int = 36, position: int = 8191, hidden: int = 2560,
                  inter: Optional[int] = None, phase_full_first: bool = False,
                  case_id: int = 4) -> StackCase:
    """The attention stack of ``cfg4_stack`` (same draws) with each layer's MLP."""
    base_case = cfg4_stack(seed, num_layers, position, hidden, phase_full_first, case_id)
    inter = inter or mlp_inter(hidden)
    layers = []
    for li, L in enumerate(base_case.layers):
        m = make_mlp(hidden, inter, seed, case_id, 1000 + 32 * li)
        layers.append(DecoderLayer(is_full=L.is_full, w_norm=L.w_norm, w_qkv=L.w_qkv, w_g=L.w_g,
                                   w_o=L.w_o, cache=L.cache, w_post=m.w_post, w_gate=m.w_gate,
                                   w_up=m.w_up, w_down=m.w_down))
    return StackCase(name=f"decoder_stack{num_layers}_pos{position}_inter{inter}",
                     arch=base_case.arch, h=base_case.h, layers=layers)


# ----------------------------------------------------------------------------
# the ends of the decode step (embedding / tied head); the pages print no
# vocabulary size, so it is a parameter here (65536 in the benchmark)
# ----------------------------------------------------------------------------

_T_EMBED, _T_WFINAL, _T_IDS = 7001, 7002, 7003


@dataclass
class HeadCase:
    embed: np.ndarray      # uint16 bf16 bits [vocab][hidden] (embed_tokens, tied head)
    w_final: np.ndarray    # uint16 bf16 bits [hidden] (model.norm)
    ids: np.ndarray        # int32 [batch] token ids
    h: np.ndarray          # float32 [batch][hidden] residual stream after the last layer

    @property
    def vocab(self) -> int:
        return int(self.embed.shape[0])


def head_case(hidden: int, vocab: int, batch: int, seed: int = 0, case_id: int = 70) -> HeadCase:
    """Embedding ~ N(0, 0.02), final norm weight ~ N(1, 0.1), ids uniform in
    [0, vocab), h ~ N(0, 1)."""
    ids = _rng(seed, case_id, _T_IDS).integers(0, vocab, size=batch).astype(np.int32)
    return HeadCase(
        embed=round_to_bf16_bits(_normal(seed, case_id, _T_EMBED, (vocab, hidden), WEIGHT_STD)),
        w_final=round_to_bf16_bits(_normal(seed, case_id, _T_WFINAL, (hidden,), 0.1, 1.0)),
        ids=ids, h=_normal(seed, case_id, _T_H, (batch, hidden)))
