"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/gqa.h declares, its pure functions agree bit for bit with the
oracle and the golden fixtures, and every invalid argument is refused before
anything is launched (a launch here, with no GPU, could only fail as
GQA_ERR_GPU, so an INVALID/UNSUPPORTED/WORKSPACE status proves the check ran
first)."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

import gqa_attention_block_amd as gqa
from gqa_attention_block_amd import binding as B
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

OK, INVALID, UNSUPPORTED, WS_SMALL, GPU = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.library_path())
    names = declared_functions()
    assert len(names) >= 12
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(B.EXPORTED_SYMBOLS) == names


def test_struct_layouts_match_the_header(tmp_path):
    """The binding's ctypes mirrors have the size and field offsets that a C
    compiler gives the header's structs (gcc on the host: plain C, no GPU)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    mirrors = {"gqa_arch": B._Arch, "gqa_layer_weights": B._Weights, "gqa_kv_seq": B._KvSeq,
               "gqa_mlp_weights": B._MlpWeights, "gqa_stack_layer": B._StackLayer}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in mirrors.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    # the header names hipStream_t nowhere (streams are void *), so plain C compiles it
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, val = ln.split()
        got[(cname, field)] = int(val)
    for cname, py in mirrors.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_rope_params_golden():
    for c in json.load(open(os.path.join(GOLDEN, "rope_params_for.json")))["cases"]:
        assert gqa.rope_params_for(c["is_full"], c["full_rotary_dim"], c["head_dim"],
                                   c["full_theta"], c["sliding_theta"]) == (c["rotary_dim"], c["theta"])


def test_kv_window_golden():
    for full, pos, win, ring, sl, ks, ar, slot in json.load(
            open(os.path.join(GOLDEN, "kv_window_cases.json")))["cases"]:
        assert gqa.kv_window(full, pos, win, ring) == (sl, ks, ar)
        assert gqa.kv_slot(pos, 0 if full else ring) == slot


def test_kv_window_and_slot_match_oracle_exhaustively():
    for window, ring in ((512, 512), (512, 0), (512, 640), (6, 6), (1, 1), (7, 30)):
        for pos in range(0, 2100):
            for full in (True, False):
                r = 0 if full else ring
                assert gqa.kv_window(full, pos, window, r) == oracle.kv_window(full, pos, window, r)
            assert gqa.kv_slot(pos, ring) == oracle.kv_slot(pos, ring)
    for pos in (32767, 32768 + 137, 2 ** 31 - 2):
        assert gqa.kv_window(False, pos, 512, 512) == oracle.kv_window(False, pos, 512, 512)


def test_host_function_errors():
    with pytest.raises(gqa.GqaError):
        gqa.kv_window(False, -1, 512, 512)
    with pytest.raises(gqa.GqaError):
        gqa.kv_window(False, 2 ** 31 - 1, 512, 512)
    with pytest.raises(gqa.GqaError):
        gqa.kv_window(False, 5, 0, 512)
    with pytest.raises(gqa.GqaError):
        gqa.rope_params_for(True, 63, 256, 5e6, 1e4)
    with pytest.raises(gqa.GqaError):
        gqa.rope_params_for(True, 512, 256, 5e6, 1e4)
    with pytest.raises(gqa.GqaError):
        gqa.rope_params_for(False, 64, 256, 5e6, -1.0)
    assert gqa.kv_slot(-1, 512) == -1
    assert gqa.kv_slot(5, -1) == -1


def test_workspace_size_grows_with_batch_and_length():
    a = gqa.Arch(hidden=2560)
    s1 = gqa.workspace_size(a, 1, 4096)
    assert gqa.workspace_size(a, 1, 32768) > s1
    assert gqa.workspace_size(a, 32, 4096) > s1
    with pytest.raises(gqa.GqaError):
        gqa.workspace_size(a, 1, 0)
    with pytest.raises(gqa.GqaError):
        gqa.workspace_size(gqa.Arch(hidden=2560, head_dim=128), 1, 10)


# ----------------------------------------------------------------------------
# argument validation of the device entry points, with fake device pointers
# that are never dereferenced (the checks must fail first)
# ----------------------------------------------------------------------------

FAKE = 0x7F0000000000          # 16-byte aligned, never touched
MISALIGNED = FAKE + 8


def _call_block(arch=None, is_full=1, seqs=None, batch=1, x=FAKE, out=FAKE + 0x100000,
                ws=FAKE + 0x200000, ws_bytes=1 << 30, weights=None):
    a = B.c_arch(arch or gqa.Arch(hidden=1024))
    w = weights or B.c_weights(FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000)
    if seqs is None:
        seqs = [B.c_kv_seq(FAKE + 0x600000, FAKE + 0x700000, 100, 0, 50, 0)]
    arr = B.c_seq_array(len(seqs))
    for i, s in enumerate(seqs):
        arr[i] = s
    st = B.raw_call("gqa_attention_block_decode", ctypes.byref(a), ctypes.byref(w), is_full, arr,
                    batch, x, out, ws, ws_bytes, None)
    return st, B.last_error()


def _seq(k=FAKE + 0x600000, v=FAKE + 0x700000, cap=100, ring=0, pos=50, reserved=0):
    return B.c_kv_seq(k, v, cap, ring, pos, reserved)


@pytest.mark.parametrize("kw,status", [
    (dict(arch=gqa.Arch(hidden=1024, head_dim=128)), UNSUPPORTED),
    (dict(arch=gqa.Arch(hidden=1024, num_heads=8)), UNSUPPORTED),
    (dict(arch=gqa.Arch(hidden=1024, num_heads=15)), INVALID),
    (dict(arch=gqa.Arch(hidden=1020)), INVALID),
    (dict(arch=gqa.Arch(hidden=16384)), UNSUPPORTED),
    (dict(arch=gqa.Arch(hidden=1024, full_rotary_dim=63)), INVALID),
    (dict(arch=gqa.Arch(hidden=1024, full_rotary_dim=512)), INVALID),
    (dict(arch=gqa.Arch(hidden=1024, sliding_window=0)), INVALID),
    (dict(arch=gqa.Arch(hidden=1024, rope_theta=0.0)), INVALID),
    (dict(arch=gqa.Arch(hidden=1024, attention_scale=float("inf"))), INVALID),
    (dict(batch=-1), INVALID),
    (dict(x=0), INVALID),
    (dict(x=MISALIGNED), INVALID),
    (dict(out=0), INVALID),
    (dict(ws=0), INVALID),
    (dict(ws_bytes=1024), WS_SMALL),
    (dict(weights=B.c_weights(0, FAKE, FAKE)), INVALID),
    (dict(weights=B.c_weights(FAKE, FAKE, MISALIGNED)), INVALID),
    (dict(seqs=[_seq(pos=100, cap=100)]), INVALID),            # linear cache too short
    (dict(seqs=[_seq(pos=-1)]), INVALID),
    (dict(seqs=[_seq(k=0)]), INVALID),
    (dict(seqs=[_seq(v=MISALIGNED)]), INVALID),
    (dict(seqs=[_seq(reserved=1)]), INVALID),
    (dict(seqs=[_seq(cap=0)]), INVALID),
    (dict(is_full=1, seqs=[_seq(cap=512, ring=512)]), INVALID),   # full layers have no ring
    (dict(is_full=0, seqs=[_seq(cap=511, ring=511)]), INVALID),   # ring < window
    (dict(is_full=0, seqs=[_seq(cap=512, ring=600)]), INVALID),   # ring > capacity
    (dict(is_full=1, seqs=[_seq(cap=2 ** 20 + 1, pos=5)]), UNSUPPORTED),  # > 2 GiB cache
    (dict(is_full=1, seqs=[_seq(), _seq(pos=200)]), INVALID),  # second sequence bad
])
def test_block_rejects_before_launch(kw, status):
    batch = len(kw.get("seqs", [None]))
    if "batch" in kw:
        batch = kw.pop("batch")
    st, msg = _call_block(batch=batch, **kw)
    assert st == status, (st, msg)
    assert msg, "an error must leave a message"


def test_null_seqs_and_null_arch():
    a = B.c_arch(gqa.Arch(hidden=1024))
    w = B.c_weights(FAKE, FAKE, FAKE)
    assert B.raw_call("gqa_attention_block_decode", None, ctypes.byref(w), 1, None, 1, FAKE, FAKE,
                      FAKE, 1 << 30, None) == INVALID
    assert B.raw_call("gqa_attention_block_decode", ctypes.byref(a), ctypes.byref(w), 1, None, 1,
                      FAKE, FAKE, FAKE, 1 << 30, None) == INVALID


def test_step_entry_points_validate():
    a = B.c_arch(gqa.Arch(hidden=1024))
    w = B.c_weights(FAKE, FAKE, FAKE)
    arr = B.c_seq_array(1)
    arr[0] = _seq()
    assert B.raw_call("gqa_qkv_rope_kv", ctypes.byref(a), ctypes.byref(w), 1, arr, 1, MISALIGNED,
                      FAKE, FAKE, None) == INVALID
    arr[0] = _seq(pos=100, cap=100)
    assert B.raw_call("gqa_qkv_rope_kv", ctypes.byref(a), ctypes.byref(w), 1, arr, 1, FAKE,
                      FAKE, FAKE, None) == INVALID
    assert B.raw_call("gqa_qkv_rope_kv", ctypes.byref(a), ctypes.byref(w), 1, None, 0, 0, 0, 0,
                      None) == OK
    assert B.raw_call("gqa_o_proj_gemv", ctypes.byref(a), ctypes.byref(B.c_weights(FAKE, FAKE, 0)),
                      1, FAKE, FAKE, None) == INVALID
    arr = B.c_seq_array(1)
    arr[0] = _seq(pos=100, cap=100)
    assert B.raw_call("gqa_attention_gated", ctypes.byref(a), 1, arr, 1, FAKE, FAKE, None, FAKE, FAKE,
                      1 << 30, None) == INVALID
    arr[0] = _seq()
    assert B.raw_call("gqa_attention_gated", ctypes.byref(a), 1, arr, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                      16, None) == WS_SMALL
    assert B.raw_call("gqa_rms_norm_bf16w", FAKE, FAKE, FAKE, 1, 0, ctypes.c_float(1e-6),
                      None) == INVALID
    assert B.raw_call("gqa_rms_norm_bf16w", FAKE, FAKE, FAKE, 1, 8, ctypes.c_float(-1.0),
                      None) == INVALID
    assert B.raw_call("gqa_rms_norm_bf16w", FAKE, FAKE, FAKE, 0, 8, ctypes.c_float(1e-6),
                      None) == OK
    assert B.raw_call("gqa_residual_add", FAKE, MISALIGNED, 10, None) == INVALID
    assert B.raw_call("gqa_residual_add", FAKE, FAKE, -1, None) == INVALID
    assert B.raw_call("gqa_residual_add", 0, 0, 0, None) == OK


def test_partials_entry_validates():
    a = B.c_arch(gqa.Arch(hidden=1024))
    arr = B.c_seq_array(33)
    for i in range(33):
        arr[i] = _seq()
    rows = ctypes.c_int32(0)
    begin = (ctypes.c_int32 * 34)()
    call = lambda batch, rows_p, begin_p, q=FAKE, mc=1024: B.raw_call(  # noqa: E731
        "gqa_attention_partials", ctypes.byref(a), 1, arr, batch, q, FAKE, FAKE, mc, rows_p, begin_p, None)
    assert call(33, ctypes.byref(rows), begin) == UNSUPPORTED       # one launch group only
    assert call(1, None, begin) == INVALID                           # chunk_rows is null
    assert call(1, ctypes.byref(rows), None) == INVALID              # chunk_begin is null
    assert call(1, ctypes.byref(rows), begin, q=MISALIGNED) == INVALID
    assert call(1, ctypes.byref(rows), begin, mc=0) == WS_SMALL
    assert call(0, ctypes.byref(rows), None) == OK                  # nothing to do
    arr[0] = _seq(pos=100, cap=100)
    assert call(1, ctypes.byref(rows), begin) == INVALID             # linear cache too short


def test_layer_entry_validates():
    a = B.c_arch(gqa.Arch(hidden=1024))
    w = B.c_weights(FAKE, FAKE, FAKE)
    arr = B.c_seq_array(1)
    arr[0] = _seq()
    call = lambda arch, wn, h: B.raw_call("gqa_attention_layer_decode", ctypes.byref(arch),  # noqa: E731
                                          ctypes.byref(w), wn, 1, arr, 1, h, FAKE, 1 << 30, None)
    assert call(a, 0, FAKE) == INVALID                 # w_norm is null
    assert call(a, MISALIGNED, FAKE) == INVALID
    assert call(a, FAKE, MISALIGNED) == INVALID        # h misaligned
    assert call(B.c_arch(gqa.Arch(hidden=1024, rms_eps=-1.0)), FAKE, FAKE) == INVALID
    assert call(B.c_arch(gqa.Arch(hidden=1024, rms_eps=float("nan"))), FAKE, FAKE) == INVALID
    assert B.raw_call("gqa_attention_layer_decode", ctypes.byref(a), ctypes.byref(w), FAKE, 1, arr, 1,
                      FAKE, FAKE, 1024, None) == WS_SMALL
    assert B.raw_call("gqa_attention_layer_decode", ctypes.byref(a), ctypes.byref(w), 0, 1, None, 0,
                      0, 0, 0, None) == OK                  # batch 0: nothing to do


def test_stack_entry_validates():
    """gqa_attention_stack_decode checks every layer before it enqueues
    anything (FAKE device pointers are never touched: a GQA_OK with layers
    would mean a launch), and names the failing layer."""
    a = B.c_arch(gqa.Arch(hidden=1024))

    def layer(**kw):
        w = B.c_weights(FAKE + 0x300000, FAKE + 0x400000, FAKE + 0x500000)
        ly = B.c_stack_layer(w, FAKE, _seq(pos=300, cap=400), 1, 0)
        for k, v in kw.items():
            setattr(ly, k, v)
        return ly

    def call(layers, n=None, h=FAKE, ws_bytes=1 << 30, arch=a):
        arr = (B.c_stack_layer * max(1, len(layers)))(*layers)
        return B.raw_call("gqa_attention_stack_decode", ctypes.byref(arch), arr if layers else None,
                          len(layers) if n is None else n, h, FAKE + 0x200000, ws_bytes, None)

    assert call([]) == OK                                     # nothing to do
    assert call([], n=-1) == INVALID
    assert call([], n=2) == INVALID                           # layers is null
    assert call([layer(), layer(reserved=1)]) == INVALID
    assert "layers[1]" in B.last_error()
    assert call([layer(), layer(w_norm=0)]) == INVALID
    assert "layers[1]" in B.last_error()
    assert call([layer(), layer(w_norm=MISALIGNED)]) == INVALID
    bad = layer()
    bad.cache = _seq(pos=400, cap=400)                        # linear cache too short
    assert call([layer(), layer(), bad]) == INVALID
    assert "layers[2]" in B.last_error()
    bad = layer()
    bad.weights = B.c_weights(FAKE, 0, FAKE)                  # no g_proj
    assert call([bad]) == INVALID
    assert call([layer()], h=MISALIGNED) == INVALID
    assert call([layer()], ws_bytes=1024) == WS_SMALL
    assert call([layer()], arch=B.c_arch(gqa.Arch(hidden=1024, rms_eps=-1.0))) == INVALID
    assert call([layer()], arch=B.c_arch(gqa.Arch(hidden=1024, head_dim=128))) == UNSUPPORTED


def test_chunk_entry_validates():
    """gqa_attention_block_chunk: every check before any launch (FAKE device
    pointers are never touched, so a GQA_OK here would mean a launch)."""
    a = B.c_arch(gqa.Arch(hidden=1024))
    w = B.c_weights(FAKE, FAKE, FAKE)
    seq = B.c_seq_array(1)

    def call(m, ws_bytes=1 << 30, seq_p=seq, x=FAKE):
        return B.raw_call("gqa_attention_block_chunk", ctypes.byref(a), ctypes.byref(w), 0, seq_p, m, x,
                          FAKE, FAKE, ws_bytes, None)

    seq[0] = _seq(pos=100, cap=200)
    assert call(0) == INVALID                          # m_tokens < 1
    assert call(-3) == INVALID
    assert call(4, seq_p=None) == INVALID              # no descriptor
    assert call(4, x=MISALIGNED) == INVALID
    assert call(4, ws_bytes=1024) == WS_SMALL
    seq[0] = _seq(pos=197, cap=200)
    assert call(4) == INVALID                          # last token at 200 needs a 201-row cache
    seq[0] = _seq(pos=1000, cap=520, ring=519)         # window 512 + 8 - 1 = 519 slots: enough
    assert call(8, ws_bytes=1024) == WS_SMALL          # got as far as the workspace check
    assert call(9) == INVALID                          # 512 + 9 - 1 = 520 > 519
    seq[0] = _seq(pos=2 ** 31 - 4, cap=200, ring=519)
    assert call(8) == INVALID                          # positions overflow int32


def test_status_strings():
    assert B.status_string(0) == "GQA_OK"
    assert B.status_string(3) == "GQA_ERR_WORKSPACE_TOO_SMALL"
    assert B.status_string(99) == "GQA_ERR_UNKNOWN"


def test_mlp_entry_validates():
    """gqa_mlp_decode / gqa_mlp_workspace_size: every check before any launch."""
    a = B.c_arch(gqa.Arch(hidden=1024))

    def w(inter=3072, reserved=0, post=FAKE, gate=FAKE, up=FAKE, down=FAKE):
        return B._MlpWeights(post, gate, up, down, inter, reserved)

    def call(weights, batch=1, h=FAKE, ws=FAKE, nbytes=1 << 30, arch=a):
        return B.raw_call("gqa_mlp_decode", ctypes.byref(arch), ctypes.byref(weights) if weights else None,
                          batch, h, ws, nbytes, None)
    assert call(None) == INVALID
    assert call(w(inter=0)) == INVALID
    assert call(w(inter=3070)) == INVALID
    assert call(w(inter=8200)) == UNSUPPORTED
    assert call(w(reserved=1)) == INVALID
    assert call(w(post=0)) == INVALID
    assert call(w(gate=MISALIGNED)) == INVALID
    assert call(w(up=0)) == INVALID
    assert call(w(down=MISALIGNED)) == INVALID
    assert call(w(), h=MISALIGNED) == INVALID
    assert call(w(), ws=0) == INVALID
    assert call(w(), batch=-1) == INVALID
    assert call(w(), nbytes=16) == WS_SMALL
    assert call(w(), arch=B.c_arch(gqa.Arch(hidden=1024, rms_eps=-1.0))) == INVALID
    assert call(w(), batch=0, h=0, ws=0) == OK                  # nothing to do
    n = ctypes.c_size_t()
    assert B.raw_call("gqa_mlp_workspace_size", ctypes.byref(a), 3072, 2, ctypes.byref(n)) == OK
    assert n.value >= (2 * 1024 + 2 * 2 * 3072) * 4
    assert B.raw_call("gqa_mlp_workspace_size", ctypes.byref(a), 3072, 2, None) == INVALID


def test_head_entries_validate():
    """gqa_embed_tokens / gqa_lm_head: every check before any launch."""
    a = B.c_arch(gqa.Arch(hidden=1024))
    ids = (ctypes.c_int32 * 3)(0, 5, 9)

    def emb(table=FAKE, vocab=10, idp=ids, batch=3, h=FAKE):
        return B.raw_call("gqa_embed_tokens", ctypes.byref(a), table, vocab, idp, batch, h, None)
    assert emb(table=0) == INVALID
    assert emb(table=MISALIGNED) == INVALID
    assert emb(vocab=0) == INVALID
    assert emb(vocab=9) == INVALID                 # id 9 out of range
    assert emb(idp=None) == INVALID
    assert emb(h=MISALIGNED) == INVALID
    assert emb(batch=-1) == INVALID
    assert emb(vocab=1 << 20) == UNSUPPORTED       # table beyond 2 GiB at hidden 1024
    assert emb(batch=0, idp=None, h=0) == OK
    neg = (ctypes.c_int32 * 1)(-1)
    assert emb(idp=neg, batch=1) == INVALID

    def head(norm=FAKE, table=FAKE, vocab=10, h=FAKE, batch=2, logits=FAKE, ws=FAKE, n=1 << 20, arch=a):
        return B.raw_call("gqa_lm_head", ctypes.byref(arch), norm, table, vocab, h, batch, logits, ws, n, None)
    assert head(norm=0) == INVALID
    assert head(table=MISALIGNED) == INVALID
    assert head(vocab=0) == INVALID
    assert head(h=0) == INVALID
    assert head(logits=MISALIGNED) == INVALID
    assert head(ws=0) == INVALID
    assert head(n=16) == WS_SMALL
    assert head(arch=B.c_arch(gqa.Arch(hidden=1024, rms_eps=float("inf")))) == INVALID
    assert head(batch=0, norm=0, h=0, logits=0, ws=0) == OK
    n = ctypes.c_size_t()
    assert B.raw_call("gqa_lm_head_workspace_size", ctypes.byref(a), 3, ctypes.byref(n)) == OK
    assert n.value >= 3 * 1024 * 4
