"""ctypes binding of libgqa (include/gqa.h).

Argument marshalling only: torch tensors are checked for dtype, device,
contiguity and shape, turned into raw device pointers, and passed with the
current HIP stream.  Every step of the block runs in the library's kernels;
there is no fallback of any kind.  If ``libgqa.so`` has not been built the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")

GQA_OK = 0
_STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARGUMENT", 2: "GQA_ERR_UNSUPPORTED",
           3: "GQA_ERR_WORKSPACE_TOO_SMALL", 4: "GQA_ERR_GPU"}


class GqaError(RuntimeError):
    def __init__(self, status: int, detail: str, call: str):
        self.status = status
        self.status_name = _STATUS.get(status, f"status {status}")
        super().__init__(f"{call}: {self.status_name}: {detail}")


class _Arch(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("full_rotary_dim", ctypes.c_int32), ("sliding_window", ctypes.c_int32),
                ("full_rope_theta", ctypes.c_double), ("rope_theta", ctypes.c_double),
                ("attention_scale", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class _Weights(ctypes.Structure):
    _fields_ = [("q_k_v_proj", ctypes.c_void_p), ("g_proj", ctypes.c_void_p),
                ("o_proj", ctypes.c_void_p), ("sinks", ctypes.c_void_p)]


class _MlpWeights(ctypes.Structure):
    _fields_ = [("post_attention_layernorm", ctypes.c_void_p), ("gate_proj", ctypes.c_void_p),
                ("up_proj", ctypes.c_void_p), ("down_proj", ctypes.c_void_p),
                ("intermediate", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _KvSeq(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("ring_capacity", ctypes.c_int32), ("position", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _StackLayer(ctypes.Structure):
    _fields_ = [("weights", _Weights), ("w_norm", ctypes.c_void_p), ("cache", _KvSeq),
                ("is_full", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python gqa_attention_block_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, D, F, S = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                            ctypes.c_float, ctypes.c_size_t)
    A, W, K = ctypes.POINTER(_Arch), ctypes.POINTER(_Weights), ctypes.POINTER(_KvSeq)
    sig = {
        "gqa_rope_params_for": (ctypes.c_int, [ctypes.c_int, I32, I32, D, D, ctypes.POINTER(I32),
                                               ctypes.POINTER(D)]),
        "gqa_kv_window": (ctypes.c_int, [ctypes.c_int, I32, I32, I32, ctypes.POINTER(I32),
                                         ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "gqa_kv_slot": (I32, [I32, I32]),
        "gqa_workspace_size": (ctypes.c_int, [A, I32, I32, ctypes.POINTER(S)]),
        "gqa_split_plan": (ctypes.c_int, [A, ctypes.c_int, K, I32, ctypes.c_int, ctypes.POINTER(I32),
                                          ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32),
                                          ctypes.POINTER(I32), ctypes.POINTER(I64)]),
        "gqa_attention_block_decode": (ctypes.c_int, [A, W, ctypes.c_int, K, I32, P, P, P, S, P]),
        "gqa_attention_block_decode_noalloc": (ctypes.c_int, [A, W, ctypes.c_int, K, I32, P, P, P]),
        "gqa_attention_layer_decode": (ctypes.c_int, [A, W, P, ctypes.c_int, K, I32, P, P, S, P]),
        "gqa_attention_stack_decode": (ctypes.c_int, [A, ctypes.POINTER(_StackLayer), I32, P, P, S, P]),
        "gqa_attention_block_chunk": (ctypes.c_int, [A, W, ctypes.c_int, K, I32, P, P, P, S, P]),
        "gqa_qkv_rope_kv": (ctypes.c_int, [A, W, ctypes.c_int, K, I32, P, P, P, P]),
        "gqa_attention_gated": (ctypes.c_int, [A, ctypes.c_int, K, I32, P, P, P, P, P, S, P]),
        "gqa_attention_partials": (ctypes.c_int, [A, ctypes.c_int, K, I32, P, P, P, I32,
                                                  ctypes.POINTER(I32), ctypes.POINTER(I32), P]),
        "gqa_o_proj_gemv": (ctypes.c_int, [A, W, I32, P, P, P]),
        "gqa_rms_norm_bf16w": (ctypes.c_int, [P, P, P, I32, I32, F, P]),
        "gqa_mlp_workspace_size": (ctypes.c_int, [A, I32, I32, ctypes.POINTER(S)]),
        "gqa_mlp_decode": (ctypes.c_int, [A, ctypes.POINTER(_MlpWeights), I32, P, P, S, P]),
        "gqa_embed_tokens": (ctypes.c_int, [A, P, I32, ctypes.POINTER(I32), I32, P, P]),
        "gqa_lm_head_workspace_size": (ctypes.c_int, [A, I32, ctypes.POINTER(S)]),
        "gqa_lm_head": (ctypes.c_int, [A, P, P, I32, P, I32, P, P, S, P]),
        "gqa_residual_add": (ctypes.c_int, [P, P, I64, P]),
        "gqa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "gqa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

#: symbols the header declares; tests check the library exports all of them
EXPORTED_SYMBOLS = (
    "gqa_rope_params_for", "gqa_kv_window", "gqa_kv_slot", "gqa_workspace_size", "gqa_split_plan",
    "gqa_attention_block_decode", "gqa_attention_block_decode_noalloc", "gqa_attention_block_chunk",
    "gqa_attention_layer_decode", "gqa_attention_stack_decode", "gqa_qkv_rope_kv",
    "gqa_attention_gated",
    "gqa_attention_partials", "gqa_o_proj_gemv", "gqa_rms_norm_bf16w", "gqa_residual_add", "gqa_status_string",
    "gqa_last_error", "gqa_mlp_workspace_size", "gqa_mlp_decode", "gqa_embed_tokens", "gqa_lm_head_workspace_size",
    "gqa_lm_head",
)


def library_path() -> str:
    return _LIB_PATH


def _check(status: int, call: str):
    if status != GQA_OK:
        raise GqaError(status, _lib.gqa_last_error().decode(), call)


# ----------------------------------------------------------------------------
# plain values
# ----------------------------------------------------------------------------

@dataclass
class Arch:
    """Mirror of gqa_arch.  Defaults are the spark2_5 family's published values."""
    hidden: int
    num_heads: int = 16
    num_kv_heads: int = 4
    head_dim: int = 256
    full_rotary_dim: int = 64
    sliding_window: int = 512
    full_rope_theta: float = 5.0e6
    rope_theta: float = 1.0e4
    attention_scale: float = 0.0625
    rms_eps: float = 1e-6

    def _c(self) -> _Arch:
        return _Arch(self.hidden, self.num_heads, self.num_kv_heads, self.head_dim,
                     self.full_rotary_dim, self.sliding_window, self.full_rope_theta,
                     self.rope_theta, self.attention_scale, self.rms_eps)

    @property
    def q_dim(self) -> int:
        return self.num_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return (self.num_heads + 2 * self.num_kv_heads) * self.head_dim


@dataclass
class KvSeq:
    """One sequence's cache for one layer: fp16 tensors [capacity][Hk][D]."""
    k: torch.Tensor
    v: torch.Tensor
    position: int
    ring_capacity: int = 0


@dataclass
class StackLayer:
    """One layer of a stack for attention_stack_decode: its input-norm weight,
    projection weights (bf16 or raw 16-bit bits), class and cache."""
    w_norm: torch.Tensor
    w_qkv: torch.Tensor
    w_g: torch.Tensor
    w_o: torch.Tensor
    is_full: bool
    seq: KvSeq
    sinks: Optional[torch.Tensor] = None


def rope_params_for(is_full: bool, full_rotary_dim: int, head_dim: int, full_theta: float,
                    sliding_theta: float):
    r, t = ctypes.c_int32(), ctypes.c_double()
    _check(_lib.gqa_rope_params_for(int(is_full), full_rotary_dim, head_dim, full_theta,
                                    sliding_theta, ctypes.byref(r), ctypes.byref(t)),
           "gqa_rope_params_for")
    return r.value, t.value


def kv_window(is_full: bool, position: int, sliding_window: int, ring_capacity: int):
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.gqa_kv_window(int(is_full), position, sliding_window, ring_capacity,
                              ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "gqa_kv_window")
    return a.value, b.value, c.value


def kv_slot(position: int, ring_capacity: int) -> int:
    return int(_lib.gqa_kv_slot(position, ring_capacity))


def workspace_size(arch: Arch, batch: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    a = arch._c()
    _check(_lib.gqa_workspace_size(ctypes.byref(a), batch, max_seq_len, ctypes.byref(n)),
           "gqa_workspace_size")
    return n.value


@dataclass
class SplitPlan:
    """The split-K schedule of one attention launch set (gqa_split_plan)."""
    chunk_rows: int
    waves: int
    direct: bool
    groups: int
    max_group_chunks: int
    chunk_bound: int


def split_plan(arch: Arch, is_full: bool, positions: Sequence[int], ring_capacity: int = 0,
               capacities: Optional[Sequence[int]] = None, allow_direct: bool = True) -> SplitPlan:
    """Host-only: the plan for sequences at ``positions`` (cache capacities
    default to position + 1, or ring_capacity on a ring).  The cache pointers
    handed to the library are placeholders it checks but never dereferences."""
    n = len(positions)
    arr = (_KvSeq * max(1, n))()
    for i, p in enumerate(positions):
        cap = capacities[i] if capacities is not None else (ring_capacity or int(p) + 1)
        arr[i] = _KvSeq(0x1000, 0x2000, int(cap), int(ring_capacity), int(p), 0)
    out = [ctypes.c_int32() for _ in range(5)]
    bound = ctypes.c_int64()
    a = arch._c()
    _check(_lib.gqa_split_plan(ctypes.byref(a), int(is_full), arr, n, int(allow_direct),
                               *[ctypes.byref(o) for o in out], ctypes.byref(bound)), "gqa_split_plan")
    return SplitPlan(out[0].value, out[1].value, bool(out[2].value), out[3].value, out[4].value, bound.value)


# ----------------------------------------------------------------------------
# device calls
# ----------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], dtype, name: str, numel: Optional[int] = None) -> int:
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _wptr(t: Optional[torch.Tensor], name: str, numel: int) -> int:
    """bf16 weights may be passed as bfloat16 or as raw 16-bit integers."""
    if t is None:
        return 0
    if t.dtype not in _BF16_LIKE:
        raise TypeError(f"{name}: dtype {t.dtype}, expected bfloat16 (or raw 16-bit bits)")
    return _ptr(t, t.dtype, name, numel)


def _sinks_ptr(arch: Arch, sinks) -> int:
    """Optional per-head attention-sink logits: fp32 [num_heads] on the device."""
    return 0 if sinks is None else _ptr(sinks, torch.float32, "sinks", arch.num_heads)


def _weights(arch: Arch, w_qkv, w_g, w_o, sinks=None) -> _Weights:
    h = arch.hidden
    return _Weights(_wptr(w_qkv, "w_qkv", arch.qkv_rows * h),
                    _wptr(w_g, "w_g", arch.num_heads * h),
                    _wptr(w_o, "w_o", h * arch.q_dim), _sinks_ptr(arch, sinks))


def _seqs(arch: Arch, seqs: Sequence[KvSeq]):
    arr = (_KvSeq * max(1, len(seqs)))()
    row = arch.num_kv_heads * arch.head_dim
    for i, s in enumerate(seqs):
        if s.k.shape != s.v.shape:
            raise ValueError(f"seqs[{i}]: k and v shapes differ")
        if s.k.numel() % row != 0:
            raise ValueError(f"seqs[{i}]: cache size is not a whole number of rows")
        cap = s.k.numel() // row
        arr[i] = _KvSeq(_ptr(s.k, torch.float16, f"seqs[{i}].k"),
                        _ptr(s.v, torch.float16, f"seqs[{i}].v"), cap, int(s.ring_capacity),
                        int(s.position), 0)
    return arr


def attention_block_decode(arch: Arch, w_qkv, w_g, w_o, is_full: bool, seqs: Sequence[KvSeq],
                           x: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                           stream=None, sinks=None):
    """One decode step of the block; ``sinks``: optional fp32 [num_heads]
    attention-sink logits (None: the family's own block, without sinks)."""
    b = len(seqs)
    a = arch._c()
    w = _weights(arch, w_qkv, w_g, w_o, sinks)
    ks = _seqs(arch, seqs)
    _check(_lib.gqa_attention_block_decode(
        ctypes.byref(a), ctypes.byref(w), int(is_full), ks, b,
        _ptr(x, torch.float32, "x", b * arch.hidden),
        _ptr(out, torch.float32, "out", b * arch.hidden),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "gqa_attention_block_decode")


def attention_block_decode_noalloc(arch: Arch, w_qkv, w_g, w_o, is_full: bool, seqs: Sequence[KvSeq],
                                   x: torch.Tensor, out: torch.Tensor, stream=None, sinks=None):
    """The same block with its workspace in the library's static per-GPU
    scratch (gqa_attention_block_decode_noalloc): no device allocation."""
    b = len(seqs)
    a = arch._c()
    w = _weights(arch, w_qkv, w_g, w_o, sinks)
    ks = _seqs(arch, seqs)
    _check(_lib.gqa_attention_block_decode_noalloc(
        ctypes.byref(a), ctypes.byref(w), int(is_full), ks, b,
        _ptr(x, torch.float32, "x", b * arch.hidden),
        _ptr(out, torch.float32, "out", b * arch.hidden), _stream(stream)),
        "gqa_attention_block_decode_noalloc")


class _Prepared:
    """A library call with its arguments marshalled once.  The object holds
    references to the tensors it was built from (their storage must not be
    resized or moved while it is used); step() updates only the sequences'
    positions and enqueues the call on the current stream (or the stream given
    at construction)."""

    def __init__(self, fn, name: str, ks, args_before_stream, stream, keep=()):
        self._fn, self._name, self._ks = fn, name, ks
        self._keep = tuple(keep)
        self._args = args_before_stream
        self._stream = None if stream is None else _stream(stream)

    def step(self, positions: Optional[Sequence[int]] = None):
        if positions is not None:
            for i, p in enumerate(positions):
                self._ks[i].position = int(p)
        st = self._fn(*self._args, self._stream if self._stream is not None
                      else torch.cuda.current_stream().cuda_stream)
        if st != GQA_OK:
            raise GqaError(st, _lib.gqa_last_error().decode(), self._name)


class PreparedBlock(_Prepared):
    """attention_block_decode with fixed weights, caches, x, out and workspace."""

    def __init__(self, arch: Arch, w_qkv, w_g, w_o, is_full: bool, seqs: Sequence[KvSeq], x: torch.Tensor,
                 out: torch.Tensor, workspace: torch.Tensor, stream=None, sinks=None):
        b = len(seqs)
        self._a = arch._c()
        self._w = _weights(arch, w_qkv, w_g, w_o, sinks)
        ks = _seqs(arch, seqs)
        super().__init__(_lib.gqa_attention_block_decode, "gqa_attention_block_decode", ks,
                         (ctypes.byref(self._a), ctypes.byref(self._w), int(is_full), ks, b,
                          _ptr(x, torch.float32, "x", b * arch.hidden),
                          _ptr(out, torch.float32, "out", b * arch.hidden),
                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel()), stream,
                         keep=(w_qkv, w_g, w_o, sinks, x, out, workspace, *[t for q in seqs for t in (q.k, q.v)]))


class PreparedLayer(_Prepared):
    """attention_layer_decode (h += block(RMSNorm(h) * w_norm), in place) with
    fixed weights, caches, h and workspace."""

    def __init__(self, arch: Arch, w_norm, w_qkv, w_g, w_o, is_full: bool, seqs: Sequence[KvSeq],
                 h: torch.Tensor, workspace: torch.Tensor, stream=None, sinks=None):
        b = len(seqs)
        self._a = arch._c()
        self._w = _weights(arch, w_qkv, w_g, w_o, sinks)
        ks = _seqs(arch, seqs)
        super().__init__(_lib.gqa_attention_layer_decode, "gqa_attention_layer_decode", ks,
                         (ctypes.byref(self._a), ctypes.byref(self._w), _wptr(w_norm, "w_norm", arch.hidden),
                          int(is_full), ks, b, _ptr(h, torch.float32, "h", b * arch.hidden),
                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel()), stream,
                         keep=(w_norm, w_qkv, w_g, w_o, sinks, h, workspace,
                               *[t for q in seqs for t in (q.k, q.v)]))


def _stack_layers(arch: Arch, layers: Sequence[StackLayer]):
    arr = (_StackLayer * max(1, len(layers)))()
    for i, ly in enumerate(layers):
        arr[i] = _StackLayer(_weights(arch, ly.w_qkv, ly.w_g, ly.w_o, ly.sinks),
                             _wptr(ly.w_norm, f"layers[{i}].w_norm", arch.hidden), _seqs(arch, [ly.seq])[0],
                             int(ly.is_full), 0)
    return arr


def _stack_keep(layers: Sequence[StackLayer]):
    return [t for ly in layers for t in (ly.w_norm, ly.w_qkv, ly.w_g, ly.w_o, ly.sinks, ly.seq.k, ly.seq.v)]


class PreparedStack(_Prepared):
    """attention_stack_decode (one token through the layers, h updated in
    place) with fixed layers, h and workspace; step(position) moves every
    layer's cache to that position."""

    def __init__(self, arch: Arch, layers: Sequence[StackLayer], h: torch.Tensor, workspace: torch.Tensor,
                 stream=None):
        self._a = arch._c()
        self._layers = _stack_layers(arch, layers)
        super().__init__(_lib.gqa_attention_stack_decode, "gqa_attention_stack_decode", None,
                         (ctypes.byref(self._a), self._layers, len(layers),
                          _ptr(h, torch.float32, "h", arch.hidden),
                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel()), stream,
                         keep=(h, workspace, *_stack_keep(layers)))

    def step(self, position: Optional[int] = None):
        if position is not None:
            for i in range(self._args[2]):
                self._layers[i].cache.position = int(position)
        super().step()


class PreparedMlp(_Prepared):
    """mlp_decode (h += down(gelu_erf(gate x) * up x), in place) with fixed
    weights, h and workspace."""

    def __init__(self, arch: Arch, w_post, w_gate, w_up, w_down, h: torch.Tensor, workspace: torch.Tensor,
                 stream=None):
        b = h.shape[0] if h.dim() == 2 else 1
        inter = int(w_gate.shape[0])
        hd = arch.hidden
        self._a = arch._c()
        self._w = _MlpWeights(_wptr(w_post, "w_post", hd), _wptr(w_gate, "w_gate", inter * hd),
                              _wptr(w_up, "w_up", inter * hd), _wptr(w_down, "w_down", hd * inter), inter, 0)
        super().__init__(_lib.gqa_mlp_decode, "gqa_mlp_decode", None,
                         (ctypes.byref(self._a), ctypes.byref(self._w), b, _ptr(h, torch.float32, "h", b * hd),
                          _ptr(workspace, torch.uint8, "workspace"), workspace.numel()), stream,
                         keep=(w_post, w_gate, w_up, w_down, h, workspace))


def attention_block_chunk(arch: Arch, w_qkv, w_g, w_o, is_full: bool, seq: KvSeq, x: torch.Tensor,
                          out: torch.Tensor, workspace: torch.Tensor, stream=None, sinks=None):
    """M consecutive tokens of one sequence (x, out: [M][hidden]); seq.position is the first token's."""
    m = x.shape[0] if x.dim() == 2 else 1
    a = arch._c()
    w = _weights(arch, w_qkv, w_g, w_o, sinks)
    ks = _seqs(arch, [seq])
    _check(_lib.gqa_attention_block_chunk(
        ctypes.byref(a), ctypes.byref(w), int(is_full), ks, m,
        _ptr(x, torch.float32, "x", m * arch.hidden),
        _ptr(out, torch.float32, "out", m * arch.hidden),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "gqa_attention_block_chunk")


def attention_layer_decode(arch: Arch, w_norm, w_qkv, w_g, w_o, is_full: bool, seqs: Sequence[KvSeq],
                           h: torch.Tensor, workspace: torch.Tensor, stream=None, sinks=None):
    """h += block(RMSNorm(h) * w_norm), in place (the attention half of a decoder layer)."""
    b = len(seqs)
    a = arch._c()
    w = _weights(arch, w_qkv, w_g, w_o, sinks)
    ks = _seqs(arch, seqs)
    _check(_lib.gqa_attention_layer_decode(
        ctypes.byref(a), ctypes.byref(w), _wptr(w_norm, "w_norm", arch.hidden), int(is_full), ks, b,
        _ptr(h, torch.float32, "h", b * arch.hidden),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "gqa_attention_layer_decode")


def attention_stack_decode(arch: Arch, layers: Sequence[StackLayer], h: torch.Tensor, workspace: torch.Tensor,
                           stream=None):
    """One token of one sequence through the layers in order: for each layer
    h += block(RMSNorm(h) * w_norm), in place (h: [hidden] or [1, hidden])."""
    a = arch._c()
    arr = _stack_layers(arch, layers)
    _check(_lib.gqa_attention_stack_decode(
        ctypes.byref(a), arr, len(layers), _ptr(h, torch.float32, "h", arch.hidden),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "gqa_attention_stack_decode")


def mlp_workspace_size(arch: Arch, intermediate: int, batch: int) -> int:
    n = ctypes.c_size_t()
    a = arch._c()
    _check(_lib.gqa_mlp_workspace_size(ctypes.byref(a), intermediate, batch, ctypes.byref(n)),
           "gqa_mlp_workspace_size")
    return n.value


def mlp_decode(arch: Arch, w_post, w_gate, w_up, w_down, h: torch.Tensor, workspace: torch.Tensor,
               stream=None):
    """h += down(gelu_erf(gate(x)) * up(x)), x = RMSNorm(h) * w_post, in place (the
    rest of the decoder layer); w_gate and w_up are [inter, hidden], w_down
    [hidden, inter], bf16 (or raw 16-bit bits)."""
    b = h.shape[0] if h.dim() == 2 else 1
    inter = int(w_gate.shape[0])
    hd = arch.hidden
    w = _MlpWeights(_wptr(w_post, "w_post", hd), _wptr(w_gate, "w_gate", inter * hd),
                    _wptr(w_up, "w_up", inter * hd), _wptr(w_down, "w_down", hd * inter), inter, 0)
    a = arch._c()
    _check(_lib.gqa_mlp_decode(ctypes.byref(a), ctypes.byref(w), b, _ptr(h, torch.float32, "h", b * hd),
                               _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                               _stream(stream)), "gqa_mlp_decode")


def embed_tokens(arch: Arch, table, ids: Sequence[int], h: torch.Tensor, stream=None):
    """h[b] = table[ids[b]] as fp32 (the raw bf16 row); table [vocab, hidden]."""
    b = len(ids)
    vocab = int(table.shape[0])
    a = arch._c()
    arr = (ctypes.c_int32 * max(1, b))(*[int(i) for i in ids])
    _check(_lib.gqa_embed_tokens(ctypes.byref(a), _wptr(table, "embed_tokens", vocab * arch.hidden), vocab, arr, b,
                                 _ptr(h, torch.float32, "h", b * arch.hidden), _stream(stream)),
           "gqa_embed_tokens")


def lm_head_workspace_size(arch: Arch, batch: int) -> int:
    n = ctypes.c_size_t()
    a = arch._c()
    _check(_lib.gqa_lm_head_workspace_size(ctypes.byref(a), batch, ctypes.byref(n)), "gqa_lm_head_workspace_size")
    return n.value


def lm_head(arch: Arch, final_norm, table, h: torch.Tensor, logits: torch.Tensor, workspace: torch.Tensor,
            stream=None):
    """logits = RMSNorm(h) * final_norm @ table^T (the tied head); h [batch,
    hidden], logits [batch, vocab], fp32."""
    b = h.shape[0]
    vocab = int(table.shape[0])
    a = arch._c()
    _check(_lib.gqa_lm_head(ctypes.byref(a), _wptr(final_norm, "final_norm", arch.hidden),
                            _wptr(table, "embed_tokens", vocab * arch.hidden), vocab,
                            _ptr(h, torch.float32, "h", b * arch.hidden), b,
                            _ptr(logits, torch.float32, "logits", b * vocab),
                            _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
           "gqa_lm_head")


def qkv_rope_kv(arch: Arch, w_qkv, w_g, is_full: bool, seqs: Sequence[KvSeq], x: torch.Tensor,
                q_roped: torch.Tensor, gate_logits: torch.Tensor, stream=None):
    """The projections, split, RoPE and KV-slot write; writes each cache's slot row."""
    b = len(seqs)
    a = arch._c()
    w = _weights(arch, w_qkv, w_g, None)
    ks = _seqs(arch, seqs)
    _check(_lib.gqa_qkv_rope_kv(
        ctypes.byref(a), ctypes.byref(w), int(is_full), ks, b,
        _ptr(x, torch.float32, "x", b * arch.hidden),
        _ptr(q_roped, torch.float32, "q_roped", b * arch.q_dim),
        _ptr(gate_logits, torch.float32, "gate_logits", b * arch.num_heads), _stream(stream)),
        "gqa_qkv_rope_kv")


def attention_gated(arch: Arch, is_full: bool, seqs: Sequence[KvSeq], q_roped: torch.Tensor,
                    gate_logits: torch.Tensor, attn_gated: torch.Tensor,
                    workspace: torch.Tensor, stream=None, sinks=None):
    """Attention over each cache window and the headwise gate (reads the caches
    only); ``sinks``: optional fp32 [num_heads] attention-sink logits."""
    b = len(seqs)
    a = arch._c()
    ks = _seqs(arch, seqs)
    _check(_lib.gqa_attention_gated(
        ctypes.byref(a), int(is_full), ks, b,
        _ptr(q_roped, torch.float32, "q_roped", b * arch.q_dim),
        _ptr(gate_logits, torch.float32, "gate_logits", b * arch.num_heads),
        _sinks_ptr(arch, sinks),
        _ptr(attn_gated, torch.float32, "attn_gated", b * arch.q_dim),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "gqa_attention_gated")


def attention_partials(arch: Arch, is_full: bool, seqs: Sequence[KvSeq], q_roped: torch.Tensor,
                       part_o: torch.Tensor, part_ml: torch.Tensor, stream=None):
    """The split-K pass alone: per chunk and query head the unnormalised
    partial (m, l, O) in log2 units; part_o is [max_chunks, Hq, D] and part_ml
    [max_chunks, Hq, 2], fp32.  Returns (chunk_rows, chunk_begin) where
    chunk_begin has len(seqs) + 1 entries (the last is the chunk count)."""
    b = len(seqs)
    a = arch._c()
    ks = _seqs(arch, seqs)
    per_chunk = arch.num_heads * arch.head_dim
    if part_o.dim() == 0 or part_o.numel() % per_chunk != 0:
        raise ValueError("part_o: must hold whole [Hq, D] chunks")
    max_chunks = part_o.numel() // per_chunk
    rows = ctypes.c_int32(0)
    begin = (ctypes.c_int32 * (b + 1))()
    _check(_lib.gqa_attention_partials(
        ctypes.byref(a), int(is_full), ks, b,
        _ptr(q_roped, torch.float32, "q_roped", b * arch.q_dim),
        _ptr(part_o, torch.float32, "part_o"),
        _ptr(part_ml, torch.float32, "part_ml", max_chunks * arch.num_heads * 2), max_chunks,
        ctypes.byref(rows), begin, _stream(stream)), "gqa_attention_partials")
    return rows.value, [int(begin[i]) for i in range(b + 1)] if b else [0]


def o_proj_gemv(arch: Arch, w_o, attn_gated: torch.Tensor, out: torch.Tensor, stream=None):
    b = attn_gated.shape[0]
    a = arch._c()
    w = _weights(arch, None, None, w_o)
    _check(_lib.gqa_o_proj_gemv(
        ctypes.byref(a), ctypes.byref(w), b,
        _ptr(attn_gated, torch.float32, "attn_gated", b * arch.q_dim),
        _ptr(out, torch.float32, "out", b * arch.hidden), _stream(stream)), "gqa_o_proj_gemv")


def rms_norm_bf16w(h: torch.Tensor, w, out: torch.Tensor, eps: float, stream=None):
    rows, hidden = h.shape
    _check(_lib.gqa_rms_norm_bf16w(
        _ptr(h, torch.float32, "h"), _wptr(w, "w", hidden),
        _ptr(out, torch.float32, "out", rows * hidden), rows, hidden, eps, _stream(stream)),
        "gqa_rms_norm_bf16w")


def residual_add(h: torch.Tensor, o: torch.Tensor, stream=None):
    n = h.numel()
    _check(_lib.gqa_residual_add(_ptr(h, torch.float32, "h"), _ptr(o, torch.float32, "o", n),
                                 n, _stream(stream)), "gqa_residual_add")


def raw_call(name: str, *args):
    """Call a library entry point with already-marshalled ctypes arguments and
    return its raw status (used by the error-path tests)."""
    return getattr(_lib, name)(*args)


def last_error() -> str:
    return _lib.gqa_last_error().decode()


def status_string(status: int) -> str:
    return _lib.gqa_status_string(status).decode()


def c_arch(arch: Arch) -> _Arch:
    return arch._c()


def c_seq_array(n: int):
    return (_KvSeq * max(1, n))()


c_weights = _Weights
c_kv_seq = _KvSeq
c_stack_layer = _StackLayer
