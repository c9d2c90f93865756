"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X).

Floating point is held to rel-L2 <= 1e-3 and max-abs <= 5e-3 * max|ref|; the
split, slot and ring/window indexing is held bit-exact (cache rows other than
the slot are untouched bit for bit; the slot row is this token's k and v; the
set of rows read is exactly the window).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import gqa_attention_block_amd as gqa
import oracle
import synth
from tests.gpu_util import (DevBlock, arch_of, assert_fp16_within_one_ulp, assert_parity, bits_to_dev,
                            check_caches, f16_to_dev, f32_to_dev, say)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a CPU host only with -m gpu
    pytest.skip("needs a GPU", allow_module_level=True)


# ----------------------------------------------------------------------------
# projections
# ----------------------------------------------------------------------------

# (hidden, is_full, positions, ring_capacity)
QKV_CASES = [
    (1024, False, [63], 0), (2560, True, [4095], 0), (1024, False, [32767], 512),
    (776, True, [5, 900, 17], 0), (264, False, [0, 511, 512, 513, 2000], 512),
    (2560, True, [int(n) - 1 for n in synth.cfg5_lengths()], 0), (8192, True, [100], 0),
    (4096, False, [1000, 31], 0), (2560, True, list(range(3, 3 + 40 * 5, 5)), 0),
    # batched (MFMA) edges: 4 rows, 17 rows (second batch tile), a tiny hidden
    (1024, True, [7, 63, 64, 3000], 0), (2560, False, list(range(100, 100 + 17 * 61, 61)), 512),
    (8, True, [1, 2, 3, 4, 5], 0),
    # VALU batch 2-3 with x too wide to stage two rows per pass (hidden > 4096)
    (6144, True, [10, 2000, 77], 0),
]


@pytest.mark.parametrize("hidden,is_full,positions,ring", QKV_CASES,
                         ids=[f"h{c[0]}_{'full' if c[1] else 'sliding'}_b{len(c[2])}" for c in QKV_CASES])
def test_qkv_rope_kv(hidden, is_full, positions, ring):
    """Projections + split + RoPE + fp16 KV-slot write against the oracle."""
    say(f"qkv_rope_kv hidden={hidden} full={is_full} batch={len(positions)} ring={ring}")
    case = synth.block_case("qkv", hidden, is_full, positions, ring_capacity=ring, seed=0,
                            case_id=12)
    dev = DevBlock(case)
    a = dev.arch
    b = case.batch
    q = torch.empty((b, a.q_dim), dtype=torch.float32, device="cuda")
    gl = torch.empty((b, a.num_heads), dtype=torch.float32, device="cuda")
    gqa.qkv_rope_kv(a, dev.w_qkv, dev.w_g, is_full, dev.seqs(), dev.x, q, gl)
    torch.cuda.synchronize()
    ref = oracle.block_decode(case.arch, is_full, case.w_qkv, case.w_g, case.w_o, case.x,
                              case.seqs)
    assert_parity(q.cpu().numpy(), ref.q_roped.reshape(b, -1), "RoPE'd q")
    assert_parity(gl.cpu().numpy(), ref.gate_logits, "gate logits")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, "qkv_rope_kv")


def test_qkv_rope_kv_rotary_width_off_the_tile_grid():
    """A full-layer rotary width that is not a multiple of 32 keeps batches on
    the VALU kernel (the MFMA units pair whole 16-row tiles); batch 5 walks
    the batch two rows per pass."""
    arch = synth.Arch(hidden=1024, full_rotary_dim=48)
    positions = [3, 700, 64, 4095, 31]
    case = synth.block_case("qkv_r48", 1024, True, positions, seed=0, case_id=13, arch=arch)
    say(f"qkv_rope_kv full_rotary_dim=48 batch={len(positions)}")
    dev = DevBlock(case)
    a = dev.arch
    q = torch.empty((case.batch, a.q_dim), dtype=torch.float32, device="cuda")
    gl = torch.empty((case.batch, a.num_heads), dtype=torch.float32, device="cuda")
    gqa.qkv_rope_kv(a, dev.w_qkv, dev.w_g, True, dev.seqs(), dev.x, q, gl)
    torch.cuda.synchronize()
    ref = oracle.block_decode(case.arch, True, case.w_qkv, case.w_g, case.w_o, case.x, case.seqs)
    assert_parity(q.cpu().numpy(), ref.q_roped.reshape(case.batch, -1), "RoPE'd q (r = 48)")
    assert_parity(gl.cpu().numpy(), ref.gate_logits, "gate logits")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, "qkv_rope_kv r=48")


@pytest.mark.parametrize("hidden,batch", [(1024, 1), (2560, 1), (776, 3), (2560, 32), (6144, 2),
                                          (776, 5), (1024, 17), (2560, 33), (8, 4)])
def test_o_proj_gemv(hidden, batch):
    say(f"o_proj_gemv hidden={hidden} batch={batch}")
    a = synth.Arch(hidden=hidden)
    w_o = synth.random_bf16((hidden, a.q_dim), 0, 11, hidden)
    attn = synth.random_hidden(a.q_dim, batch, 0, 11)
    out = torch.empty((batch, hidden), dtype=torch.float32, device="cuda")
    gqa.o_proj_gemv(arch_of(a), bits_to_dev(w_o), f32_to_dev(attn), out)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle.gemv(oracle.bf16_bits_to_f64(w_o), attn), "o_proj")


# ----------------------------------------------------------------------------
# attention + gate over the cache window, from a given RoPE'd q
# ----------------------------------------------------------------------------

# (name, is_full, positions, ring_capacity, capacities or None)
ATTN_CASES = [
    ("full_pos0_single_key", True, [0], 0, None),
    ("full_pos1", True, [1], 0, None),
    ("full_pos63", True, [63], 0, None),
    ("full_pos64", True, [64], 0, None),
    ("full_pos1000_ragged", True, [1000], 0, None),
    ("full_pos4095", True, [4095], 0, None),
    ("full_pos20000_multitile", True, [20000], 0, None),
    ("full_pos32767", True, [32767], 0, None),
    ("full_pos100000", True, [100000], 0, None),
    ("full_cap_larger", True, [700], 0, [2048]),
    ("sliding_linear_pos63", False, [63], 0, [64]),
    ("sliding_linear_pos1000", False, [1000], 0, None),
    ("ring_pos0", False, [0], 512, None),
    ("ring_pos100", False, [100], 512, None),
    ("ring_pos510", False, [510], 512, None),
    ("ring_pos511", False, [511], 512, None),
    ("ring_pos512", False, [512], 512, None),
    ("ring_pos513", False, [513], 512, None),
    ("ring_pos1000", False, [1000], 512, None),
    ("ring_pos32767", False, [32767], 512, None),
    ("ring_pos32905", False, [32768 + 137], 512, None),
    ("ring640_pos2000", False, [2000], 640, None),
    ("ring_cap_larger", False, [3000], 512, [1024]),
    ("full_batch_mixed", True, [0, 5, 63, 64, 65, 1000, 4095], 0, None),
    ("ring_batch_mixed", False, [3, 511, 512, 777, 32767], 512, None),
    ("full_batch33_two_launches", True, list(range(7, 7 + 33 * 37, 37)), 0, None),
    ("full_batch_long", True, [20000, 3000, 40000, 100], 0, None),
    # several long sequences: the split-K pass runs 2-wave workgroups
    ("full_batch16_two_wave", True, list(range(700, 700 + 16 * 553, 553)), 0, None),
    ("full_batch15_two_wave", True, list(range(700, 700 + 15 * 553, 553)), 0, None),
    ("ring_batch16_two_wave", False, list(range(400, 400 + 16 * 2001, 2001)), 512, None),
]


def _attn_inputs(name, is_full, positions, ring, caps, case_id):
    arch = synth.Arch(hidden=1024)
    seqs = []
    for i, p in enumerate(positions):
        cap = caps[i] if caps else (ring if ring else p + 1)
        seqs.append(synth.make_cache(arch, 0, case_id, 100 + 16 * i, cap, ring, p))
    case = synth.BlockCase(name=name, arch=arch, is_full=is_full, w_qkv=None, w_g=None,
                           w_o=None, x=np.zeros((len(positions), 1), np.float32), seqs=seqs)
    q = synth.random_hidden(arch.q_dim, len(positions), 0, case_id, tensor_id=903)
    gl = synth.random_gate_logits(arch, len(positions), 0, case_id)
    return arch, case, q, gl


def _oracle_attention(arch, case, q, gl, sinks=None):
    """Attention over each cache as it is (the slot row already written) + gate."""
    out = []
    for i, s in enumerate(case.seqs):
        sl, ks, ar = oracle.kv_window(case.is_full, s.position, arch.sliding_window,
                                      s.ring_capacity)
        att = oracle.attention_decode(np.asarray(q[i], np.float64).reshape(arch.num_heads, -1),
                                      s.k, s.v, sl, ks, ar, arch.attention_scale, sinks)
        out.append(oracle.head_gate(att, gl[i]).reshape(-1))
    return np.stack(out)


def _run_attention(arch, case, q, gl, sinks=None):
    ga = arch_of(arch)
    k = [f16_to_dev(s.k) for s in case.seqs]
    v = [f16_to_dev(s.v) for s in case.seqs]
    seqs = [gqa.KvSeq(k=k[i], v=v[i], position=s.position, ring_capacity=s.ring_capacity)
            for i, s in enumerate(case.seqs)]
    ws = torch.empty(gqa.workspace_size(ga, len(seqs), max(s.position + 1 for s in case.seqs)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((len(seqs), ga.q_dim), dtype=torch.float32, device="cuda")
    gqa.attention_gated(ga, case.is_full, seqs, f32_to_dev(q), f32_to_dev(gl), out, ws,
                        sinks=None if sinks is None else f32_to_dev(sinks))
    torch.cuda.synchronize()
    return out.cpu().numpy(), k, v


@pytest.mark.parametrize("name,is_full,positions,ring,caps", ATTN_CASES,
                         ids=[c[0] for c in ATTN_CASES])
def test_attention_gated(name, is_full, positions, ring, caps):
    say(f"attention_gated {name} positions={positions[:8]} ring={ring}")
    arch, case, q, gl = _attn_inputs(name, is_full, positions, ring, caps, 20)
    got, k, v = _run_attention(arch, case, q, gl)
    ref = _oracle_attention(arch, case, q, gl)
    for b in range(len(positions)):
        assert_parity(got[b], ref[b], f"{name}[{b}] gated attention")
    for i, s in enumerate(case.seqs):   # the attention step only reads the caches
        assert np.array_equal(k[i].cpu().numpy().view(np.int16), s.k.view(np.int16))
        assert np.array_equal(v[i].cpu().numpy().view(np.int16), s.v.view(np.int16))


@pytest.mark.parametrize("qmax", [1e3, 6e5])
@pytest.mark.parametrize("name,is_full,positions,ring", [("full_pos4095", True, [4095], 0),
                                                          ("ring_pos32767", False, [32767], 512),
                                                          ("full_batch_long", True, [20000, 3000, 40000, 100], 0)])
def test_attention_large_q_in_range(name, is_full, positions, ring, qmax):
    """Query elements far from the N(0,1) of the other cases but inside the
    documented range (|q_i| * scale * log2(e) below the fp16 maximum; 6e5 is
    0.83 of that bound): the scores span thousands of log2 units and the
    softmax is nearly one-hot, yet the output meets the same bar."""
    say(f"attention_gated large q {name} qmax={qmax:g}")
    arch, case, q, gl = _attn_inputs(name, is_full, positions, ring, None, 21)
    q = (q / np.max(np.abs(q), axis=1, keepdims=True) * qmax).astype(np.float32)
    assert float(np.max(np.abs(q))) * arch.attention_scale * 1.4426950408889634 < 65504.0
    got, _, _ = _run_attention(arch, case, q, gl)
    ref = _oracle_attention(arch, case, q, gl)
    for b in range(len(positions)):
        assert_parity(got[b], ref[b], f"{name}[{b}] gated attention, |q| up to {qmax:g}")


# ----------------------------------------------------------------------------
# the split-K pass alone: every chunk's partial against the oracle's attention
# over that chunk's rows, and its partition function
# ----------------------------------------------------------------------------

PARTIAL_CASES = ["full_pos0_single_key", "full_pos1000_ragged", "full_pos32767", "ring_pos513",
                 "ring_pos32905", "full_batch_mixed", "ring_batch_mixed", "full_batch_long",
                 "full_batch16_two_wave", "ring_batch16_two_wave"]
# stored element e of a partial holds dim 16 * (e % 16) + e // 16
_PERM = np.array([16 * (e % 16) + e // 16 for e in range(256)])


@pytest.mark.parametrize("name", PARTIAL_CASES)
def test_attention_partials_per_chunk(name):
    _, is_full, positions, ring, caps = next(c for c in ATTN_CASES if c[0] == name)
    say(f"attention_partials {name} positions={positions[:8]} ring={ring}")
    arch, case, q, _ = _attn_inputs(name, is_full, positions, ring, caps, 21)
    ga = arch_of(arch)
    k = [f16_to_dev(s.k) for s in case.seqs]
    v = [f16_to_dev(s.v) for s in case.seqs]
    seqs = [gqa.KvSeq(k=k[i], v=v[i], position=s.position, ring_capacity=s.ring_capacity)
            for i, s in enumerate(case.seqs)]
    max_chunks = 1024
    part_o = torch.full((max_chunks, ga.num_heads, ga.head_dim), float("nan"), device="cuda")
    part_ml = torch.full((max_chunks, ga.num_heads, 2), float("nan"), device="cuda")
    rows, begin = gqa.attention_partials(ga, is_full, seqs, f32_to_dev(q), part_o, part_ml)
    torch.cuda.synchronize()
    assert rows % 64 == 0 and begin[0] == 0 and begin[-1] <= max_chunks
    po, pml = part_o.cpu().numpy().astype(np.float64), part_ml.cpu().numpy().astype(np.float64)
    log2e = 1.0 / np.log(2.0)
    group = arch.num_heads // arch.num_kv_heads
    for i, s in enumerate(case.seqs):
        sl, ks, ar = oracle.kv_window(is_full, s.position, arch.sliding_window, s.ring_capacity)
        qi = np.asarray(q[i], np.float64).reshape(arch.num_heads, -1)
        nch = begin[i + 1] - begin[i]
        assert nch == -(-(sl - ks) // rows)
        for j in range(nch):
            c0, c1 = ks + j * rows, min(ks + (j + 1) * rows, sl)
            ref = oracle.attention_decode(qi, s.k, s.v, c1, c0, ar, arch.attention_scale)
            phys = oracle.physical_rows(c1, c0, ar)
            c = begin[i] + j
            for h in range(arch.num_heads):
                m, l = pml[c, h]
                o = np.empty(256)
                o[_PERM] = po[c, h]
                assert_parity(o / l, ref[h], f"{name}[{i}] chunk {j} head {h}")
                # l * 2^m is the chunk's partition function in log2 units
                sc = arch.attention_scale * log2e * (s.k[phys, h // group].astype(np.float64) @ qi[h])
                z = sc.max() + np.log2(np.sum(np.exp2(sc - sc.max())))
                assert abs(np.log2(l) + m - z) <= 1e-4, (name, i, j, h, np.log2(l) + m, z)
                assert sc.max() - 8 - 1e-3 <= m <= sc.max() + 1e-3, (name, i, j, h, m, sc.max())
    assert np.all(np.isnan(pml[begin[-1]:])), "wrote past the last chunk"


@pytest.mark.parametrize("num_kv_heads,positions", [(1, [700]), (2, [3000, 64]), (3, [1000, 130]),
                                                    (5, [2047]), (8, [500])])
def test_attention_other_kv_head_counts(num_kv_heads, positions):
    """Head counts other than the spark2_5 family's 4 (one attention
    workgroup per chunk and KV head, whatever their number)."""
    say(f"attention_gated num_kv_heads={num_kv_heads} positions={positions}")
    arch = synth.Arch(hidden=1024, num_heads=4 * num_kv_heads, num_kv_heads=num_kv_heads)
    seqs = [synth.make_cache(arch, 0, 22, 100 + 16 * i, p + 1, 0, p) for i, p in enumerate(positions)]
    case = synth.BlockCase(name="kv_heads", arch=arch, is_full=True, w_qkv=None, w_g=None, w_o=None,
                           x=np.zeros((len(positions), 1), np.float32), seqs=seqs)
    q = synth.random_hidden(arch.q_dim, len(positions), 0, 22, tensor_id=903)
    gl = synth.random_gate_logits(arch, len(positions), 0, 22)
    got, _, _ = _run_attention(arch, case, q, gl)
    ref = _oracle_attention(arch, case, q, gl)
    for b in range(len(positions)):
        assert_parity(got[b], ref[b], f"Hk={num_kv_heads}[{b}] gated attention")


def test_attention_partials_rejects_two_launch_groups():
    arch = synth.Arch(hidden=1024)
    ga = arch_of(arch)
    cap = 8
    k = torch.zeros((cap, arch.num_kv_heads, arch.head_dim), dtype=torch.float16, device="cuda")
    seqs = [gqa.KvSeq(k=k, v=k, position=3, ring_capacity=0)] * 33
    q = torch.zeros((33, ga.q_dim), device="cuda")
    part_o = torch.empty((64, ga.num_heads, ga.head_dim), device="cuda")
    part_ml = torch.empty((64, ga.num_heads, 2), device="cuda")
    with pytest.raises(gqa.GqaError) as e:
        gqa.attention_partials(ga, True, seqs, q, part_o, part_ml)
    assert e.value.status == 2
    with pytest.raises(gqa.GqaError) as e:
        gqa.attention_partials(ga, True, seqs[:32], q, part_o[:16], part_ml)
    assert e.value.status == 3


# ----------------------------------------------------------------------------
# bit-exact row set: which rows are read, and how many
# ----------------------------------------------------------------------------

ROWSET_CASES = [
    ("full_pos300_cap512", True, 300, 0, 512),
    ("full_pos5000", True, 5000, 0, 5001),
    ("sliding_linear_pos1000", False, 1000, 0, 1001),
    ("ring_pos511", False, 511, 512, 512),
    ("ring_pos512", False, 512, 512, 512),
    ("ring_pos513", False, 513, 512, 512),
    ("ring_pos1000", False, 1000, 512, 512),
    ("ring_pos32905", False, 32768 + 137, 512, 512),
    ("ring640_pos1500", False, 1500, 640, 640),
    ("full_pos0", True, 0, 0, 4),
    ("full_pos32767", True, 32767, 0, 32768),
]


def _rowset_inputs(is_full, pos, ring, cap, onehot_row=None):
    """q = 0, gate logit +30 (sigmoid rounds to 1.0f), V = 1 on every row of the
    window (or one-hot on one row), NaN on every row outside it."""
    arch = synth.Arch(hidden=1024)
    hk, d = arch.num_kv_heads, arch.head_dim
    sl, ks, ar = oracle.kv_window(is_full, pos, arch.sliding_window, ring)
    owner = {}
    for t in range(pos + 1):                   # rows written up to this token
        owner[t % ring if ring else t] = t
    rng = np.random.default_rng([3, pos, ring, cap])
    k = rng.standard_normal((cap, hk, d)).astype(np.float16)
    v = np.ones((cap, hk, d), np.float16)
    for r in range(cap):
        t = owner.get(r, -1)
        if not (ks <= t < sl):
            k[r] = np.nan
            v[r] = np.nan
    if onehot_row is not None:
        v[:] = np.where(np.isnan(v), v, np.float16(0))
        v[onehot_row] = 1.0
    q = np.zeros((1, arch.q_dim), np.float32)
    gl = np.full((1, arch.num_heads), 30.0, np.float32)
    seq = synth.SeqCache(k=k, v=v, ring_capacity=ring, position=pos)
    case = synth.BlockCase(name="rowset", arch=arch, is_full=is_full, w_qkv=None, w_g=None,
                           w_o=None, x=np.zeros((1, 1), np.float32), seqs=[seq])
    return arch, case, q, gl, sl - ks, owner, (ks, sl)


@pytest.mark.parametrize("name,is_full,pos,ring,cap", ROWSET_CASES, ids=[c[0] for c in ROWSET_CASES])
def test_rows_read_are_exactly_the_window(name, is_full, pos, ring, cap):
    say(f"rowset {name}")
    arch, case, q, gl, n, owner, (ks, sl) = _rowset_inputs(is_full, pos, ring, cap)
    got, _, _ = _run_attention(arch, case, q, gl)
    # any row outside the window would bring a NaN in; all in-window rows are 1
    assert np.array_equal(got[0], np.ones_like(got[0])), f"{name}: {got[0][:4]}"
    # one-hot V on the oldest in-window row: the output 1/n recovers n exactly
    oldest = [r for r, t in owner.items() if t == ks][0]
    arch, case, q, gl, n2, _, _ = _rowset_inputs(is_full, pos, ring, cap, onehot_row=oldest)
    got, _, _ = _run_attention(arch, case, q, gl)
    assert np.all(np.abs(got[0] * n - 1.0) < 4e-7), f"{name}: {got[0][0]} vs 1/{n}"
    assert int(round(1.0 / float(got[0][0]))) == n


@pytest.mark.parametrize("pos", [511, 512, 513, 1000, 32768 + 137])
def test_ring_equals_linear_bitwise(pos):
    """The same last-512 rows through a 512-slot ring and through a linear
    cache give bit-identical results (one reduction order)."""
    say(f"ring==linear pos={pos}")
    arch = synth.Arch(hidden=1024)
    hk, d = arch.num_kv_heads, arch.head_dim
    rng = np.random.default_rng([4, pos])
    lo = max(0, pos - 511)
    lin_k = np.zeros((pos + 1, hk, d), np.float16)
    lin_v = np.zeros((pos + 1, hk, d), np.float16)
    lin_k[lo:] = rng.standard_normal((pos + 1 - lo, hk, d))
    lin_v[lo:] = rng.standard_normal((pos + 1 - lo, hk, d))
    ring_k = np.zeros((512, hk, d), np.float16)
    ring_v = np.zeros((512, hk, d), np.float16)
    for t in range(lo, pos + 1):
        ring_k[t % 512], ring_v[t % 512] = lin_k[t], lin_v[t]
    q = synth.random_hidden(arch.q_dim, 1, 0, 30, tensor_id=903)
    gl = synth.random_gate_logits(arch, 1, 0, 30)
    outs = []
    for k, v, ring in ((lin_k, lin_v, 0), (ring_k, ring_v, 512)):
        seq = synth.SeqCache(k=k, v=v, ring_capacity=ring, position=pos)
        case = synth.BlockCase(name="rl", arch=arch, is_full=False, w_qkv=None, w_g=None,
                               w_o=None, x=np.zeros((1, 1), np.float32), seqs=[seq])
        outs.append(_run_attention(arch, case, q, gl)[0])
    assert np.array_equal(outs[0].view(np.int32), outs[1].view(np.int32))


# ----------------------------------------------------------------------------
# the whole block on the named workloads
# ----------------------------------------------------------------------------

BLOCK_CASES = ["cfg1", "cfg2", "cfg3", "cfg5", "full32k"]


@pytest.mark.parametrize("name", BLOCK_CASES)
def test_block_matches_oracle(name):
    case = synth.NAMED_BLOCK_CASES[name]()
    say(f"block {case.name} batch={case.batch} positions={[s.position for s in case.seqs][:6]}")
    dev = DevBlock(case)
    out = dev.run_block()
    ref = oracle.block_decode(case.arch, case.is_full, case.w_qkv, case.w_g, case.w_o, case.x,
                              case.seqs)
    assert_parity(out, ref.out, f"{name} block output")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, name)


def _one_launch(case) -> bool:
    """One sequence whose window is longer than the partial kernel finishes by
    itself (128 rows): the block runs as one persistent launch (or, past its
    shape limits, as projections + its attention/merge phase + o_proj)."""
    if case.batch != 1:
        return False
    s = case.seqs[0]
    n = s.position + 1 if case.is_full else min(s.position + 1, case.arch.sliding_window)
    return n > 128


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "full32k"])
def test_block_equals_its_steps(name):
    """The block entry point and the three step entry points (projections,
    gated attention, o_proj) run on the same data.  The block's output is
    bit-identical to the steps' in every case -- also when the block runs as
    one launch (cfg2, cfg3, the 32K layer), whose tasks compute each value
    with the steps' code in the steps' order -- and bit-identical from one run
    to the next.  The KV cache rows are bit-identical too."""
    case = synth.NAMED_BLOCK_CASES[name]()
    say(f"block==steps {case.name} one_launch={_one_launch(case)}")
    dev = DevBlock(case)
    out_block = dev.run_block()
    dev2 = DevBlock(case)
    a = dev2.arch
    b = case.batch
    q = torch.empty((b, a.q_dim), dtype=torch.float32, device="cuda")
    gl = torch.empty((b, a.num_heads), dtype=torch.float32, device="cuda")
    attn = torch.empty((b, a.q_dim), dtype=torch.float32, device="cuda")
    out = torch.empty((b, a.hidden), dtype=torch.float32, device="cuda")
    gqa.qkv_rope_kv(a, dev2.w_qkv, dev2.w_g, case.is_full, dev2.seqs(), dev2.x, q, gl)
    gqa.attention_gated(a, case.is_full, dev2.seqs(), q, gl, attn, dev2.ws)
    gqa.o_proj_gemv(a, dev2.w_o, attn, out)
    torch.cuda.synchronize()
    out_steps = out.cpu().numpy()
    for i in range(b):
        assert torch.equal(dev.k[i], dev2.k[i]) and torch.equal(dev.v[i], dev2.v[i])
    assert np.array_equal(out_steps.view(np.int32), out_block.view(np.int32)), \
        f"block and steps differ: max |diff| {np.abs(out_steps - out_block).max():.3e}"
    dev3 = DevBlock(case)
    for rep in range(3):   # one workspace, three calls: the one-launch block re-arms its counters
        out_again = dev3.run_block()
        assert np.array_equal(out_again.view(np.int32), out_block.view(np.int32)), f"run {rep} differs"


@pytest.mark.parametrize("num_kv_heads,position,hidden", [(1, 8191, 1024), (2, 5000, 1024), (8, 3000, 1024),
                                                           (4, 3000, 6144), (4, 20000, 4096), (4, 700, 8),
                                                           (1, 200, 1024), (2, 300, 1024), (4, 1023, 2560)])
def test_block_one_launch_other_shapes(num_kv_heads, position, hidden):
    """One sequence on a full layer with shapes other than the family's: the
    one-launch block over Hq query heads with 256 chunks at Hk = 1 (the merge
    past one wave's 64 lanes), q_dim 2048, the widest x it stages (hidden
    4096) and a tiny one (8); with few chunks (positions 200, 300, 1023: 4 to
    16 chunks), where the last attention task of each KV head group merges
    it, at Hk = 1, 2 and 4; and its fallback, projections + its
    attention/merge phase + o_proj, for q_dim 8192 (Hk = 8) and hidden 6144."""
    arch = synth.Arch(hidden=hidden, num_heads=4 * num_kv_heads, num_kv_heads=num_kv_heads)
    case = synth.block_case(f"fused_hk{num_kv_heads}_h{hidden}", hidden, True, [position], seed=0, case_id=31,
                            arch=arch)
    say(f"block one launch Hk={num_kv_heads} position={position} hidden={hidden}")
    dev = DevBlock(case)
    out = dev.run_block()
    ref = oracle.block_decode(case.arch, case.is_full, case.w_qkv, case.w_g, case.w_o, case.x, case.seqs)
    assert_parity(out, ref.out, f"Hk={num_kv_heads} block output")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, case.name)


CHUNK_CASES = [
    # (name, hidden, is_full, first position, tokens, ring)
    ("full_h1024_p100_m5", 1024, True, 100, 5, 0),
    ("full_h264_p300_m40", 264, True, 300, 40, 0),           # two launch groups of 32 tokens
    ("sliding_ring_h1024_p1035_m9", 1024, False, 1035, 9, 520),   # slots 515..519 then 0..3
    ("sliding_linear_h1024_p600_m8", 1024, False, 600, 8, 0),
    ("full_h2560_p4090_m1", 2560, True, 4090, 1, 0),          # one token: the single-token block
]


@pytest.mark.parametrize("name,hidden,is_full,p0,m,ring", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_block_chunk_matches_oracle(name, hidden, is_full, p0, m, ring):
    """M consecutive tokens of one sequence in one call against the oracle's
    token-after-token chunk: outputs, the M written slots, and every other
    cache row untouched."""
    cap = ring if ring else p0 + m
    case = synth.block_case(name, hidden, is_full, [p0], capacities=[cap], ring_capacity=ring, seed=0,
                            case_id=32)
    x = synth.random_hidden(hidden, m, 0, 32, tensor_id=90)
    say(f"block_chunk {name}")
    a = arch_of(case.arch)
    k = f16_to_dev(case.seqs[0].k)
    v = f16_to_dev(case.seqs[0].v)
    ws = torch.empty(gqa.workspace_size(a, m, p0 + m), dtype=torch.uint8, device="cuda")
    out = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
    gqa.attention_block_chunk(a, bits_to_dev(case.w_qkv), bits_to_dev(case.w_g), bits_to_dev(case.w_o), is_full,
                              gqa.KvSeq(k=k, v=v, position=p0, ring_capacity=ring), f32_to_dev(x), out, ws)
    torch.cuda.synchronize()
    ref = oracle.block_chunk(case.arch, is_full, case.w_qkv, case.w_g, case.w_o, x, case.seqs[0], m)
    assert_parity(out.cpu().numpy(), ref.out, f"{name} chunk output")
    kg, vg = k.cpu().numpy(), v.cpu().numpy()
    rest = np.ones(cap, bool)
    rest[ref.slots] = False
    assert np.array_equal(kg[rest].view(np.int16), case.seqs[0].k[rest].view(np.int16)), "K rows outside the chunk"
    assert np.array_equal(vg[rest].view(np.int16), case.seqs[0].v[rest].view(np.int16)), "V rows outside the chunk"
    for s in ref.slots:   # fp32 sums near zero: one ulp plus 2^-18 of the row's scale, as for one token
        kscale = float(np.max(np.abs(ref.k_cache[s].astype(np.float64))))
        vscale = float(np.max(np.abs(ref.v_cache[s].astype(np.float64))))
        assert_fp16_within_one_ulp(kg[s], ref.k_cache[s], f"{name} K slot {s}", kscale)
        assert_fp16_within_one_ulp(vg[s], ref.v_cache[s], f"{name} V slot {s}", vscale)


def test_batch_zero_is_a_no_op():
    say("batch 0")
    a = gqa.Arch(hidden=1024)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    x = torch.full((1, 1024), 7.0, dtype=torch.float32, device="cuda")
    w_qkv = torch.zeros((a.qkv_rows, 1024), dtype=torch.int16, device="cuda")
    w_g = torch.zeros((a.num_heads, 1024), dtype=torch.int16, device="cuda")
    w_o = torch.zeros((1024, a.q_dim), dtype=torch.int16, device="cuda")
    gqa.attention_block_decode(a, w_qkv, w_g, w_o, True, [], x, x, ws)
    torch.cuda.synchronize()
    assert torch.all(x == 7.0)


# ----------------------------------------------------------------------------
# the 36-layer attention-only stack (config 4): compare the residual delta
# ----------------------------------------------------------------------------

def _run_stack(case: synth.StackCase):
    a = arch_of(case.arch)
    hid = a.hidden
    h = f32_to_dev(case.h)
    h0 = h.clone()
    xn = torch.empty_like(h)
    o = torch.empty_like(h)
    ws = torch.empty(gqa.workspace_size(a, 1, case.layers[0].cache.position + 1),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for li, L in enumerate(case.layers):
        k, v = f16_to_dev(L.cache.k), f16_to_dev(L.cache.v)
        gqa.rms_norm_bf16w(h, bits_to_dev(L.w_norm), xn, a.rms_eps)
        gqa.attention_block_decode(a, bits_to_dev(L.w_qkv), bits_to_dev(L.w_g), bits_to_dev(L.w_o),
                                   L.is_full, [gqa.KvSeq(k=k, v=v, position=L.cache.position,
                                                         ring_capacity=L.cache.ring_capacity)],
                                   xn, o, ws)
        outs.append(o.cpu().numpy().copy())
        gqa.residual_add(h, o)
    torch.cuda.synchronize()
    return (h - h0).cpu().numpy(), outs


_STACKS = {}


def _stack_and_ref(kind: str, phase_full_first: bool):
    """The 36-layer stacks at position 8191 (the configuration the stack
    benchmarks time) and their oracle results, generated once per session:
    each takes about a minute to draw on the host."""
    key = (kind, phase_full_first)
    if key not in _STACKS:
        if kind == "attention":
            case = synth.cfg4_stack(phase_full_first=phase_full_first)
            ref = oracle.stack_decode(case.arch, case.h, case.layers)
        else:
            case = synth.decoder_stack(phase_full_first=phase_full_first)
            ref = oracle.decoder_stack_decode(case.arch, case.h, case.layers)
        for other in [k for k in _STACKS if k[0] != kind]:
            del _STACKS[other]   # one kind of stack (both phases) in host memory at a time
        _STACKS[key] = (case, ref)
    return _STACKS[key]


@pytest.mark.parametrize("phase_full_first", [False, True])
def test_stack_delta_matches_oracle(phase_full_first):
    case, ref = _stack_and_ref("attention", phase_full_first)
    say(f"stack {case.name} phase_full_first={phase_full_first}")
    delta, outs = _run_stack(case)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "stack residual delta")
    for li in range(len(case.layers)):
        assert_parity(outs[li], ref.block_outs[li], f"stack layer {li} block output")


# ----------------------------------------------------------------------------
# the fused layer entry: h += block(RMSNorm(h) * w_norm)
# ----------------------------------------------------------------------------

LAYER_CASES = [
    ("full_h2560_pos4095_b1", 2560, True, [4095], 0),
    ("full_h2560_pos4100_b1", 2560, True, [4100], 0),   # 65 chunks: one past a wave's lanes
    ("ring_h1024_pos1000_b1", 1024, False, [1000], 512),
    ("full_h1024_b2", 1024, True, [63, 700], 0),
    ("full_h1024_b5", 1024, True, [7, 63, 200, 1000, 4095], 0),
    ("ring_h2560_b17", 2560, False, list(range(300, 300 + 17 * 97, 97)), 512),
]


@pytest.mark.parametrize("name,hidden,is_full,positions,ring", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
def test_layer_decode_matches_oracle(name, hidden, is_full, positions, ring):
    say(f"attention_layer_decode {name}")
    case = synth.block_case(name, hidden, is_full, positions, ring_capacity=ring, seed=0, case_id=30)
    w_norm = synth.random_bf16((hidden,), 0, 30, 77, std=0.1, mean=1.0)
    h0 = synth.random_hidden(hidden, case.batch, 0, 30, tensor_id=78)
    dev = DevBlock(case)
    h = f32_to_dev(h0)
    gqa.attention_layer_decode(dev.arch, bits_to_dev(w_norm), dev.w_qkv, dev.w_g, dev.w_o, is_full,
                               dev.seqs(), h, dev.ws)
    torch.cuda.synchronize()
    delta = h.cpu().numpy().astype(np.float64) - h0.astype(np.float64)
    xn = oracle.rms_norm(h0, w_norm, case.arch.rms_eps)
    ref = oracle.block_decode(case.arch, is_full, case.w_qkv, case.w_g, case.w_o, xn, case.seqs)
    assert_parity(delta, ref.out, f"{name} residual delta")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, name)


# ----------------------------------------------------------------------------
# attention sinks: one more logit per query head in each softmax, no value row
# ----------------------------------------------------------------------------

def _sinks(arch, case_id):
    s = synth.random_sinks(arch, 0, case_id)
    s[0] = -np.inf          # the same as no sink
    s[1] = 200.0            # past fp32's exp range: the head's attention is 0
    return s


# every merge: in the partial kernel (<= 128 rows), small, mid and wide
# combines, two launch groups
SINK_ATTN_CASES = ["full_pos0_single_key", "full_pos63", "ring_pos513", "full_pos4095", "full_pos32767",
                   "full_batch_mixed", "ring_batch_mixed", "full_batch33_two_launches", "full_batch_long",
                   "full_batch16_two_wave"]


@pytest.mark.parametrize("name", SINK_ATTN_CASES)
def test_attention_gated_with_sinks(name):
    _, is_full, positions, ring, caps = next(c for c in ATTN_CASES if c[0] == name)
    say(f"attention_gated with sinks {name} positions={positions[:8]} ring={ring}")
    arch, case, q, gl = _attn_inputs(name, is_full, positions, ring, caps, 20)
    sinks = _sinks(arch, 21)
    got, _, _ = _run_attention(arch, case, q, gl, sinks)
    ref = _oracle_attention(arch, case, q, gl, sinks)
    for b in range(len(positions)):
        assert_parity(got[b], ref[b], f"{name}[{b}] gated attention with sinks")
    assert not np.any(got[:, arch.head_dim:2 * arch.head_dim]), "head 1's sink must take all the weight"
    plain, _, _ = _run_attention(arch, case, q, gl)
    assert np.array_equal(got[:, :arch.head_dim].view(np.int32), plain[:, :arch.head_dim].view(np.int32)), \
        "a sink of -inf must change nothing"


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg5", "full32k"])
def test_block_with_sinks_matches_oracle(name):
    """The block's own merges (in the partial kernel, the merge tasks of the
    one-launch block, the batched combine) with sink logits."""
    case = synth.NAMED_BLOCK_CASES[name]()
    say(f"block with sinks {case.name} batch={case.batch}")
    sinks = _sinks(case.arch, 22)
    dev = DevBlock(case)
    out = dev.run_block(sinks)
    ref = oracle.block_decode(case.arch, case.is_full, case.w_qkv, case.w_g, case.w_o, case.x,
                              case.seqs, sinks)
    assert_parity(out, ref.out, f"{name} block output with sinks")
    check_caches(case, dev.k, dev.v, ref.k16, ref.v16, ref.slots, name)


@pytest.mark.parametrize("name", ["full_h264_p300_m40", "sliding_ring_h1024_p1035_m9"])
def test_block_chunk_with_sinks_matches_oracle(name):
    _, hidden, is_full, p0, m, ring = next(c for c in CHUNK_CASES if c[0] == name)
    cap = ring if ring else p0 + m
    case = synth.block_case(name, hidden, is_full, [p0], capacities=[cap], ring_capacity=ring, seed=0,
                            case_id=32)
    x = synth.random_hidden(hidden, m, 0, 32, tensor_id=90)
    sinks = _sinks(case.arch, 23)
    say(f"block_chunk with sinks {name}")
    a = arch_of(case.arch)
    k = f16_to_dev(case.seqs[0].k)
    v = f16_to_dev(case.seqs[0].v)
    ws = torch.empty(gqa.workspace_size(a, m, p0 + m), dtype=torch.uint8, device="cuda")
    out = torch.empty((m, hidden), dtype=torch.float32, device="cuda")
    gqa.attention_block_chunk(a, bits_to_dev(case.w_qkv), bits_to_dev(case.w_g), bits_to_dev(case.w_o), is_full,
                              gqa.KvSeq(k=k, v=v, position=p0, ring_capacity=ring), f32_to_dev(x), out, ws,
                              sinks=f32_to_dev(sinks))
    torch.cuda.synchronize()
    ref = oracle.block_chunk(case.arch, is_full, case.w_qkv, case.w_g, case.w_o, x, case.seqs[0], m, sinks)
    assert_parity(out.cpu().numpy(), ref.out, f"{name} chunk output with sinks")


@pytest.mark.parametrize("name", ["full_h2560_pos4100_b1", "full_h1024_b5"])
def test_layer_decode_with_sinks_matches_oracle(name):
    _, hidden, is_full, positions, ring = next(c for c in LAYER_CASES if c[0] == name)
    say(f"attention_layer_decode with sinks {name}")
    case = synth.block_case(name, hidden, is_full, positions, ring_capacity=ring, seed=0, case_id=30)
    w_norm = synth.random_bf16((hidden,), 0, 30, 77, std=0.1, mean=1.0)
    h0 = synth.random_hidden(hidden, case.batch, 0, 30, tensor_id=78)
    sinks = _sinks(case.arch, 24)
    dev = DevBlock(case)
    h = f32_to_dev(h0)
    gqa.attention_layer_decode(dev.arch, bits_to_dev(w_norm), dev.w_qkv, dev.w_g, dev.w_o, is_full,
                               dev.seqs(), h, dev.ws, sinks=f32_to_dev(sinks))
    torch.cuda.synchronize()
    delta = h.cpu().numpy().astype(np.float64) - h0.astype(np.float64)
    xn = oracle.rms_norm(h0, w_norm, case.arch.rms_eps)
    ref = oracle.block_decode(case.arch, is_full, case.w_qkv, case.w_g, case.w_o, xn, case.seqs, sinks)
    assert_parity(delta, ref.out, f"{name} residual delta with sinks")


def _run_fused_layer_stack(case):
    """gqa_attention_layer_decode once per layer on one residual stream;
    returns the total delta and each layer's contribution."""
    a = arch_of(case.arch)
    h = f32_to_dev(case.h)
    ws = torch.empty(gqa.workspace_size(a, 1, case.layers[0].cache.position + 1), dtype=torch.uint8,
                     device="cuda")
    contrib = []
    for L in case.layers:
        k, v = f16_to_dev(L.cache.k), f16_to_dev(L.cache.v)
        before = h.clone()
        gqa.attention_layer_decode(a, bits_to_dev(L.w_norm), bits_to_dev(L.w_qkv), bits_to_dev(L.w_g),
                                   bits_to_dev(L.w_o), L.is_full,
                                   [gqa.KvSeq(k=k, v=v, position=L.cache.position,
                                              ring_capacity=L.cache.ring_capacity)], h, ws)
        contrib.append((h.double() - before.double()).cpu().numpy())
    torch.cuda.synchronize()
    delta = h.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    return delta, contrib


@pytest.mark.parametrize("phase_full_first", [False, True])
def test_stack36_of_fused_layers_matches_oracle(phase_full_first):
    """The benchmarked stack path at its own configuration: 36 layers of
    gqa_attention_layer_decode at position 8191 (9 full layers over 8192
    rows, 27 sliding layers over wrapped 512-slot rings), both phases of the
    3:1 pattern; the total delta and every layer's contribution against the
    oracle's block outputs."""
    case, ref = _stack_and_ref("attention", phase_full_first)
    say(f"fused-layer stack {case.name} phase_full_first={phase_full_first}")
    delta, contrib = _run_fused_layer_stack(case)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "36-layer fused stack residual delta")
    for li in range(len(case.layers)):
        assert_parity(contrib[li], ref.block_outs[li], f"36-layer fused stack layer {li} contribution")


def _stack_layers_dev(case, sinks=False):
    """The case's layers on the device (caches included) as StackLayer records."""
    out = []
    for li, L in enumerate(case.layers):
        out.append(gqa.StackLayer(
            w_norm=bits_to_dev(L.w_norm), w_qkv=bits_to_dev(L.w_qkv), w_g=bits_to_dev(L.w_g),
            w_o=bits_to_dev(L.w_o), is_full=L.is_full,
            seq=gqa.KvSeq(k=f16_to_dev(L.cache.k), v=f16_to_dev(L.cache.v), position=L.cache.position,
                          ring_capacity=L.cache.ring_capacity),
            sinks=torch.from_numpy(synth.random_sinks(case.arch, 0, 40 + li)).cuda() if sinks else None))
    return out


def _stack_vs_layers(case, sinks=False):
    """h after gqa_attention_stack_decode, after gqa_attention_layer_decode
    layer by layer, and after the stack call once more (same device caches:
    each call rewrites every layer's slot row with the same values)."""
    a = arch_of(case.arch)
    layers = _stack_layers_dev(case, sinks)
    ws = torch.empty(gqa.workspace_size(a, 1, max(L.cache.position for L in case.layers) + 1),
                     dtype=torch.uint8, device="cuda")
    h_stack = f32_to_dev(case.h)
    gqa.attention_stack_decode(a, layers, h_stack, ws)
    h_layers = f32_to_dev(case.h)
    for ly in layers:
        gqa.attention_layer_decode(a, ly.w_norm, ly.w_qkv, ly.w_g, ly.w_o, ly.is_full, [ly.seq], h_layers, ws,
                                   sinks=ly.sinks)
    h_again = f32_to_dev(case.h)
    gqa.attention_stack_decode(a, layers, h_again, ws)
    torch.cuda.synchronize()
    return h_stack, h_layers, h_again


def _assert_same_bits(got: torch.Tensor, ref: torch.Tensor, what: str):
    g, r = got.view(torch.int32).cpu(), ref.view(torch.int32).cpu()
    n = int((g != r).sum())
    assert n == 0, f"{what}: {n} of {g.numel()} values differ in their bits"


@pytest.mark.parametrize("phase_full_first", [False, True])
def test_stack36_one_launch_matches_oracle(phase_full_first):
    """The one-launch stack at the benchmarked configuration (36 layers at
    position 8191, 9 full over 8192 rows, 27 sliding over wrapped 512-slot
    rings): the residual delta against the oracle, and bit-identical to the
    36 layer calls and to itself run again."""
    case, ref = _stack_and_ref("attention", phase_full_first)
    say(f"one-launch stack {case.name} phase_full_first={phase_full_first}")
    h_stack, h_layers, h_again = _stack_vs_layers(case)
    delta = h_stack.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "one-launch 36-layer stack residual delta")
    _assert_same_bits(h_stack, h_layers, "one-launch stack vs its layer calls")
    _assert_same_bits(h_again, h_stack, "one-launch stack run twice")


def _stack_case_positions(num_layers, position, hidden, positions=None, sliding_window=None):
    case = synth.cfg4_stack(num_layers=num_layers, position=position, hidden=hidden, case_id=41)
    if sliding_window is not None:
        case.arch = dataclasses.replace(case.arch, sliding_window=sliding_window)
    if positions is not None:
        for L, p in zip(case.layers, positions):
            L.cache.position = p
    return case


STACK_SPLIT_CASES = [
    # 45 layers: a launch of 40, then one of 5
    ("layers45_pos1000", dict(num_layers=45, position=1000, hidden=1024)),
    # sliding layers over 96 rows (the direct form, one layer each) between
    # full layers over 301 rows (one-launch runs of one layer)
    ("window96_mixed", dict(num_layers=8, position=300, hidden=1024, sliding_window=96)),
    # 6 distinct positions over 10 layers: more shapes than one launch holds
    ("positions6", dict(num_layers=10, position=1200, hidden=1024,
                        positions=[1200, 1100, 1000, 900, 800, 700, 1200, 1100, 1000, 900])),
    # hidden 2560, 12 layers at a position whose full window is 65 chunks
    ("h2560_pos4100", dict(num_layers=12, position=4100, hidden=2560)),
]


@pytest.mark.parametrize("name,kw", STACK_SPLIT_CASES, ids=[c[0] for c in STACK_SPLIT_CASES])
def test_stack_launch_runs_match_oracle(name, kw):
    """How the stack entry splits its layers into launches (the 40-layer and
    4-shape limits, layers the one-launch block does not take): each case
    against the oracle and bit-identical to the layer calls."""
    case = _stack_case_positions(**kw)
    say(f"stack runs {name}")
    ref = oracle.stack_decode(case.arch, case.h, case.layers)
    h_stack, h_layers, h_again = _stack_vs_layers(case)
    delta = h_stack.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), f"stack {name} residual delta")
    _assert_same_bits(h_stack, h_layers, f"stack {name} vs its layer calls")
    _assert_same_bits(h_again, h_stack, f"stack {name} run twice")


def test_stack_with_sinks_equals_layer_calls():
    """Per-layer sink logits reach each layer of a one-launch stack: the
    result is bit-identical to the layer calls with the same sinks (those are
    checked against the oracle with sinks elsewhere)."""
    case = _stack_case_positions(num_layers=6, position=2000, hidden=1024)
    say("stack with sinks")
    h_stack, h_layers, h_again = _stack_vs_layers(case, sinks=True)
    h_plain = f32_to_dev(case.h)
    a = arch_of(case.arch)
    gqa.attention_stack_decode(a, _stack_layers_dev(case), h_plain,
                               torch.empty(gqa.workspace_size(a, 1, 2001), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    _assert_same_bits(h_stack, h_layers, "stack with sinks vs its layer calls")
    _assert_same_bits(h_again, h_stack, "stack with sinks run twice")
    assert not torch.equal(h_plain, h_stack), "the sinks changed nothing"


@pytest.mark.parametrize("phase_full_first", [False, True])
def test_stack_of_fused_layers_matches_oracle(phase_full_first):
    case = synth.cfg4_stack(num_layers=8, position=1000, phase_full_first=phase_full_first)
    say(f"fused-layer stack {case.name} phase_full_first={phase_full_first}")
    a = arch_of(case.arch)
    h = f32_to_dev(case.h)
    ws = torch.empty(gqa.workspace_size(a, 1, case.layers[0].cache.position + 1), dtype=torch.uint8,
                     device="cuda")
    for L in case.layers:
        k, v = f16_to_dev(L.cache.k), f16_to_dev(L.cache.v)
        gqa.attention_layer_decode(a, bits_to_dev(L.w_norm), bits_to_dev(L.w_qkv), bits_to_dev(L.w_g),
                                   bits_to_dev(L.w_o), L.is_full,
                                   [gqa.KvSeq(k=k, v=v, position=L.cache.position,
                                              ring_capacity=L.cache.ring_capacity)], h, ws)
    torch.cuda.synchronize()
    ref = oracle.stack_decode(case.arch, case.h, case.layers)
    delta = h.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "fused-layer stack residual delta")


# ----------------------------------------------------------------------------
# the rest of the decoder layer: post-attention norm + erf-GELU gated MLP
# ----------------------------------------------------------------------------

MLP_CASES = [(1024, 3072, 1), (1024, 3072, 3), (776, 1160, 2), (2560, 7680, 1), (2560, 7680, 5),
             (2560, 7680, 32), (1024, 8192, 37)]


@pytest.mark.parametrize("hidden,inter,batch", MLP_CASES, ids=[f"h{c[0]}_i{c[1]}_b{c[2]}" for c in MLP_CASES])
def test_mlp_decode_matches_oracle(hidden, inter, batch):
    """gqa_mlp_decode: h += down(gelu_erf(gate x) * up x), x = rms(h) w_post, on the
    VALU GEMV (batch 1-3), the MFMA projections (4 and more, in groups of 32),
    and a ragged shape; compared on the MLP's contribution h_out - h_in."""
    say(f"mlp hidden={hidden} inter={inter} batch={batch}")
    arch = synth.Arch(hidden=hidden)
    m = synth.make_mlp(hidden, inter, 0, 60 + batch, 2000)
    h0 = synth.random_hidden(hidden, batch, 0, 60 + batch, tensor_id=950)
    a = arch_of(arch)
    h = f32_to_dev(h0)
    ws = torch.empty(gqa.mlp_workspace_size(a, inter, batch), dtype=torch.uint8, device="cuda")
    gqa.mlp_decode(a, bits_to_dev(m.w_post), bits_to_dev(m.w_gate), bits_to_dev(m.w_up),
                   bits_to_dev(m.w_down), h, ws)
    torch.cuda.synchronize()
    ref = oracle.mlp_decode(h0, m.w_post, m.w_gate, m.w_up, m.w_down, arch.rms_eps)
    got = h.cpu().numpy().astype(np.float64) - np.asarray(h0, np.float64)
    for b in range(batch):
        assert_parity(got[b], ref.out[b], f"mlp row {b} contribution")


def test_mlp_batch_zero_is_a_no_op():
    arch = synth.Arch(hidden=1024)
    a = arch_of(arch)
    h = torch.ones((0, 1024), dtype=torch.float32, device="cuda")
    w = torch.zeros((8, 1024), dtype=torch.int16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    gqa.mlp_decode(a, torch.zeros(1024, dtype=torch.int16, device="cuda"), w, w,
                   torch.zeros((1024, 8), dtype=torch.int16, device="cuda"), h, ws)


@pytest.mark.parametrize("phase_full_first", [False, True])
def test_decoder_stack_matches_oracle(phase_full_first):
    """Whole decoder layers, batch 1: gqa_attention_layer_decode then
    gqa_mlp_decode per layer, against the oracle's layer order."""
    case = synth.decoder_stack(num_layers=4, position=1000, phase_full_first=phase_full_first)
    say(f"decoder stack {case.name} phase_full_first={phase_full_first}")
    a = arch_of(case.arch)
    h = f32_to_dev(case.h)
    inter = case.layers[0].w_gate.shape[0]
    ws = torch.empty(gqa.workspace_size(a, 1, case.layers[0].cache.position + 1), dtype=torch.uint8,
                     device="cuda")
    ws_mlp = torch.empty(gqa.mlp_workspace_size(a, inter, 1), dtype=torch.uint8, device="cuda")
    for L in case.layers:
        k, v = f16_to_dev(L.cache.k), f16_to_dev(L.cache.v)
        gqa.attention_layer_decode(a, bits_to_dev(L.w_norm), bits_to_dev(L.w_qkv), bits_to_dev(L.w_g),
                                   bits_to_dev(L.w_o), L.is_full,
                                   [gqa.KvSeq(k=k, v=v, position=L.cache.position,
                                              ring_capacity=L.cache.ring_capacity)], h, ws)
        gqa.mlp_decode(a, bits_to_dev(L.w_post), bits_to_dev(L.w_gate), bits_to_dev(L.w_up),
                       bits_to_dev(L.w_down), h, ws_mlp)
    torch.cuda.synchronize()
    ref = oracle.decoder_stack_decode(case.arch, case.h, case.layers)
    delta = h.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "decoder stack residual delta")


def test_decoder_stack36_matches_oracle():
    """The benchmarked whole-decoder path at its own configuration: 36 layers
    of gqa_attention_layer_decode then gqa_mlp_decode (intermediate 7680) at
    position 8191; the total delta and every layer's contribution (attention
    plus MLP) against the oracle."""
    case, ref = _stack_and_ref("decoder", False)
    say(f"decoder stack {case.name}")
    a = arch_of(case.arch)
    h = f32_to_dev(case.h)
    inter = case.layers[0].w_gate.shape[0]
    ws = torch.empty(gqa.workspace_size(a, 1, case.layers[0].cache.position + 1), dtype=torch.uint8,
                     device="cuda")
    ws_mlp = torch.empty(gqa.mlp_workspace_size(a, inter, 1), dtype=torch.uint8, device="cuda")
    contrib = []
    for L in case.layers:
        k, v = f16_to_dev(L.cache.k), f16_to_dev(L.cache.v)
        before = h.clone()
        gqa.attention_layer_decode(a, bits_to_dev(L.w_norm), bits_to_dev(L.w_qkv), bits_to_dev(L.w_g),
                                   bits_to_dev(L.w_o), L.is_full,
                                   [gqa.KvSeq(k=k, v=v, position=L.cache.position,
                                              ring_capacity=L.cache.ring_capacity)], h, ws)
        gqa.mlp_decode(a, bits_to_dev(L.w_post), bits_to_dev(L.w_gate), bits_to_dev(L.w_up),
                       bits_to_dev(L.w_down), h, ws_mlp)
        contrib.append((h.double() - before.double()).cpu().numpy())
    torch.cuda.synchronize()
    delta = h.cpu().numpy().astype(np.float64) - np.asarray(case.h, np.float64)
    assert_parity(delta, ref.h - np.asarray(case.h, np.float64), "36-layer decoder residual delta")
    for li in range(len(case.layers)):
        assert_parity(contrib[li], ref.block_outs[li], f"36-layer decoder layer {li} contribution")
    _STACKS.clear()


# ----------------------------------------------------------------------------
# the ends of the decode step: embedding gather (bit-exact), final norm + tied head
# ----------------------------------------------------------------------------

HEAD_CASES = [(1024, 1000, 1), (1024, 1000, 3), (2560, 32768, 1), (2560, 65536, 5), (776, 4099, 70)]


@pytest.mark.parametrize("hidden,vocab,batch", HEAD_CASES, ids=[f"h{c[0]}_v{c[1]}_b{c[2]}" for c in HEAD_CASES])
def test_embed_and_head_match_oracle(hidden, vocab, batch):
    say(f"embed + head hidden={hidden} vocab={vocab} batch={batch}")
    arch = synth.Arch(hidden=hidden)
    hc = synth.head_case(hidden, vocab, batch)
    a = arch_of(arch)
    table = bits_to_dev(hc.embed)
    h = torch.full((batch, hidden), float("nan"), dtype=torch.float32, device="cuda")
    gqa.embed_tokens(a, table, hc.ids.tolist(), h)
    torch.cuda.synchronize()
    # the gather is a copy of bf16 values into fp32: bit-exact
    want = oracle.embed_gather(hc.embed, hc.ids)
    assert np.array_equal(h.cpu().numpy().astype(np.float64), want), "embedding rows differ"
    hs = f32_to_dev(hc.h)
    logits = torch.empty((batch, vocab), dtype=torch.float32, device="cuda")
    ws = torch.empty(gqa.lm_head_workspace_size(a, batch), dtype=torch.uint8, device="cuda")
    gqa.lm_head(a, bits_to_dev(hc.w_final), table, hs, logits, ws)
    torch.cuda.synchronize()
    ref = oracle.lm_head(hc.h, hc.w_final, hc.embed, arch.rms_eps)
    got = logits.cpu().numpy().astype(np.float64)
    for b in range(batch):
        assert_parity(got[b], ref[b], f"logits row {b}")
    assert np.array_equal(hs.cpu().numpy(), hc.h), "the head must not write h"


def test_prepared_calls_equal_the_plain_calls():
    """PreparedBlock / PreparedLayer / PreparedMlp enqueue the same entry points
    with arguments marshalled once; step(positions) moves the token."""
    case = synth.block_case("prepared_ring", 1024, False, [700], ring_capacity=512, seed=0, case_id=80)
    a = arch_of(case.arch)
    s = case.seqs[0]
    x, w_qkv, w_g, w_o = f32_to_dev(case.x), bits_to_dev(case.w_qkv), bits_to_dev(case.w_g), bits_to_dev(case.w_o)
    ws = torch.empty(gqa.workspace_size(a, 1, 2048), dtype=torch.uint8, device="cuda")
    outs = []
    for prepared in (False, True):
        k, v = f16_to_dev(s.k), f16_to_dev(s.v)
        out = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
        seqs = [gqa.KvSeq(k=k, v=v, position=700, ring_capacity=512)]
        if prepared:
            pb = gqa.PreparedBlock(a, w_qkv, w_g, w_o, False, seqs, x, out, ws)
            pb.step()
            first = out.clone()
            pb.step([701])
        else:
            gqa.attention_block_decode(a, w_qkv, w_g, w_o, False, seqs, x, out, ws)
            first = out.clone()
            gqa.attention_block_decode(a, w_qkv, w_g, w_o, False,
                                       [gqa.KvSeq(k=k, v=v, position=701, ring_capacity=512)], x, out, ws)
        torch.cuda.synchronize()
        outs.append((first.cpu().numpy(), out.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()))
    # every path is deterministic: outputs and cache rows bitwise
    for i in range(4):
        assert np.array_equal(outs[0][i].view(np.uint8), outs[1][i].view(np.uint8)), \
            f"prepared block differs in item {i}"
    # layer + MLP on a residual stream
    m = synth.make_mlp(1024, 3072, 0, 81, 2000)
    wn = bits_to_dev(synth.round_to_bf16_bits(np.ones(1024, np.float32)))
    wsm = torch.empty(gqa.mlp_workspace_size(a, 3072, 1), dtype=torch.uint8, device="cuda")
    res = []
    for prepared in (False, True):
        k, v = f16_to_dev(s.k), f16_to_dev(s.v)
        h = f32_to_dev(case.x)
        seqs = [gqa.KvSeq(k=k, v=v, position=700, ring_capacity=512)]
        mw = (bits_to_dev(m.w_post), bits_to_dev(m.w_gate), bits_to_dev(m.w_up), bits_to_dev(m.w_down))
        if prepared:
            gqa.PreparedLayer(a, wn, w_qkv, w_g, w_o, False, seqs, h, ws).step()
            gqa.PreparedMlp(a, *mw, h, wsm).step()
        else:
            gqa.attention_layer_decode(a, wn, w_qkv, w_g, w_o, False, seqs, h, ws)
            gqa.mlp_decode(a, *mw, h, wsm)
        torch.cuda.synchronize()
        res.append(h.cpu().numpy())
    assert np.array_equal(res[1].view(np.uint32), res[0].view(np.uint32)), "prepared layer + MLP differ"


def test_prepared_calls_with_sinks_match_the_oracle():
    """PreparedBlock and PreparedLayer pass the sink logits on (a full layer,
    one sequence: the one-launch block), against the oracle."""
    case = synth.block_case("prepared_sinks", 2560, True, [5000], seed=0, case_id=82)
    sinks = _sinks(case.arch, 25)
    dev = DevBlock(case)
    out = torch.empty((1, 2560), dtype=torch.float32, device="cuda")
    pb = gqa.PreparedBlock(dev.arch, dev.w_qkv, dev.w_g, dev.w_o, True, dev.seqs(), dev.x, out, dev.ws,
                           sinks=f32_to_dev(sinks))
    pb.step()
    torch.cuda.synchronize()
    ref = oracle.block_decode(case.arch, True, case.w_qkv, case.w_g, case.w_o, case.x, case.seqs, sinks)
    assert_parity(out.cpu().numpy(), ref.out, "prepared block with sinks")
    w_norm = synth.random_bf16((2560,), 0, 82, 77, std=0.1, mean=1.0)
    h0 = synth.random_hidden(2560, 1, 0, 82, tensor_id=78)
    dev2 = DevBlock(case)
    h = f32_to_dev(h0)
    gqa.PreparedLayer(dev2.arch, bits_to_dev(w_norm), dev2.w_qkv, dev2.w_g, dev2.w_o, True, dev2.seqs(), h,
                      dev2.ws, sinks=f32_to_dev(sinks)).step()
    torch.cuda.synchronize()
    xn = oracle.rms_norm(h0, w_norm, case.arch.rms_eps)
    ref2 = oracle.block_decode(case.arch, True, case.w_qkv, case.w_g, case.w_o, xn, case.seqs, sinks)
    assert_parity(h.cpu().numpy().astype(np.float64) - h0.astype(np.float64), ref2.out,
                  "prepared layer with sinks")


def test_graph_replays_match_eager():
    """A block (one sequence: the one-launch block, whose flag words need no
    clearing), a whole decoder layer and a one-launch stack captured in HIP
    graphs: every replay, with eager work and synchronisations in between,
    equals the eager result bit for bit (outputs and cache rows)."""
    case = synth.block_case("graph_full", 1024, True, [6000], seed=0, case_id=82)
    a = arch_of(case.arch)
    s = case.seqs[0]
    x, w_qkv, w_g, w_o = f32_to_dev(case.x), bits_to_dev(case.w_qkv), bits_to_dev(case.w_g), bits_to_dev(case.w_o)
    ws = torch.empty(gqa.workspace_size(a, 1, 8192), dtype=torch.uint8, device="cuda")
    k, v = f16_to_dev(s.k), f16_to_dev(s.v)
    out = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
    pb = gqa.PreparedBlock(a, w_qkv, w_g, w_o, True, [gqa.KvSeq(k=k, v=v, position=6000)], x, out, ws)
    pb.step()
    torch.cuda.synchronize()
    eager, k_eager = out.clone(), k.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            pb.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))              # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32)), f"block replay {rep}"
        assert torch.equal(k, k_eager), f"cache rows after replay {rep}"
    # a whole decoder layer (attention layer + MLP) on the residual stream
    m = synth.make_mlp(1024, 3072, 0, 83, 2000)
    wn = bits_to_dev(synth.round_to_bf16_bits(np.ones(1024, np.float32)))
    wsm = torch.empty(gqa.mlp_workspace_size(a, 3072, 1), dtype=torch.uint8, device="cuda")
    h0 = f32_to_dev(case.x)
    h = h0.clone()
    calls = [gqa.PreparedLayer(a, wn, w_qkv, w_g, w_o, True, [gqa.KvSeq(k=k, v=v, position=6000)], h, ws),
             gqa.PreparedMlp(a, bits_to_dev(m.w_post), bits_to_dev(m.w_gate), bits_to_dev(m.w_up),
                             bits_to_dev(m.w_down), h, wsm)]
    for c in calls:
        c.step()
    torch.cuda.synchronize()
    eager_h = h.clone()
    with torch.cuda.stream(side):
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=side):
            for c in calls:
                c.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        h.copy_(h0)                          # eager work between replays
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), eager_h.view(torch.int32)), f"decoder layer replay {rep}"
    # a one-launch stack of 6 layers (hidden 1024, position 1000)
    st = synth.cfg4_stack(num_layers=6, position=1000, hidden=1024, case_id=84)
    layers = _stack_layers_dev(st)
    hs0 = f32_to_dev(st.h)
    hs = hs0.clone()
    a_s = arch_of(st.arch)
    wss = torch.empty(gqa.workspace_size(a_s, 1, 1001), dtype=torch.uint8, device="cuda")
    stack = gqa.PreparedStack(a_s, layers, hs, wss)
    stack.step()
    torch.cuda.synchronize()
    eager_s = hs.clone()
    with torch.cuda.stream(side):
        g3 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g3, stream=side):
            stack.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        hs.copy_(hs0)                        # eager work between replays
        torch.cuda.synchronize()
        g3.replay()
        torch.cuda.synchronize()
        assert torch.equal(hs.view(torch.int32), eager_s.view(torch.int32)), f"stack replay {rep}"


def test_rms_norm_and_residual_add():
    say("rms_norm + residual_add")
    hidden, rows = 2560, 3
    h = synth.random_hidden(hidden, rows, 0, 40)
    w = synth.random_bf16((hidden,), 0, 40, 7, std=0.1, mean=1.0)
    out = torch.empty((rows, hidden), dtype=torch.float32, device="cuda")
    hd = f32_to_dev(h)
    gqa.rms_norm_bf16w(hd, bits_to_dev(w), out, 1e-6)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle.rms_norm(h, w, 1e-6), "rms_norm")
    o = synth.random_hidden(hidden, rows, 0, 41)
    gqa.residual_add(hd, f32_to_dev(o))
    torch.cuda.synchronize()
    assert np.array_equal(hd.cpu().numpy(), (h + o).astype(np.float32))
