"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``pin_*`` takes the oracle module as ``O`` so the same checks run on the
real oracle (all must pass) and on deliberately broken copies of it (at least
one must fail; see ``test_oracle_pins.py``).  The pins use: values printed on
the pages (golden fixtures), hand-worked integer cases, closed forms,
mathematical invariants, brute force on tiny inputs, and a library SDPA.
"""
from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def tiny_arch(window=6, full_rotary_dim=4):
    """A small GQA shape: 4 query heads over 2 KV heads, head_dim 8."""
    return SimpleNamespace(num_heads=4, num_kv_heads=2, head_dim=8,
                           full_rotary_dim=full_rotary_dim, sliding_window=window,
                           full_rope_theta=5e6, rope_theta=1e4,
                           attention_scale=1.0 / math.sqrt(8.0), rms_eps=1e-6,
                           hidden=16)


def _bf16(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def _rng(seed):
    return np.random.default_rng([7, seed])


def _tiny_weights(arch, rng):
    rows = (arch.num_heads + 2 * arch.num_kv_heads) * arch.head_dim
    w_qkv = _bf16(rng.standard_normal((rows, arch.hidden)).astype(np.float32) * 0.3)
    w_g = _bf16(rng.standard_normal((arch.num_heads, arch.hidden)).astype(np.float32) * 0.3)
    w_o = _bf16(rng.standard_normal((arch.hidden, arch.num_heads * arch.head_dim))
                .astype(np.float32) * 0.3)
    return w_qkv, w_g, w_o


def _seq(k, v, ring, pos):
    return SimpleNamespace(k=k, v=v, ring_capacity=ring, position=pos)


def _cache(arch, rng, cap):
    shape = (cap, arch.num_kv_heads, arch.head_dim)
    return (rng.standard_normal(shape).astype(np.float16),
            rng.standard_normal(shape).astype(np.float16))


# ----------------------------------------------------------------------------
# storage types
# ----------------------------------------------------------------------------

def pin_bf16_decode(O):
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3E80], np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -133, 0.25]
    got = O.bf16_bits_to_f64(bits)
    assert np.array_equal(got, np.array(want)), got


def pin_fp16_round_to_nearest_even(O):
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -30,
                  65504.0, -2.5 * 2.0 ** -24, 0.1], np.float64)
    want = [1.0, 1 + 2.0 ** -9, 1 + 2.0 ** -10, 65504.0, -2.0 * 2.0 ** -24,
            0.0999755859375]
    got = O.to_fp16(x).astype(np.float64)
    assert np.array_equal(got, np.array(want)), got


# ----------------------------------------------------------------------------
# projections
# ----------------------------------------------------------------------------

def pin_gemv_brute_force(O):
    rng = _rng(1)
    w = _bf16(rng.standard_normal((5, 7)).astype(np.float32))
    x = rng.standard_normal((2, 7))
    wf = O.bf16_bits_to_f64(w)
    got = O.gemv(wf, x)
    assert got.shape == (2, 5)
    for b in range(2):
        for r in range(5):
            acc = 0.0
            for c in range(7):
                acc += float(wf[r][c]) * float(x[b][c])
            assert abs(got[b][r] - acc) <= 1e-12 * (1 + abs(acc)), (b, r)


def pin_split_offsets(O):
    """x = one-hot e_j makes qkv the j-th weight column; at position 0 RoPE is
    the identity, so the slot rows are fp16 of the k and v column sections."""
    arch = tiny_arch()
    rng = _rng(2)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    wq = O.bf16_bits_to_f64(w_qkv)
    qd, kd = arch.num_heads * arch.head_dim, arch.num_kv_heads * arch.head_dim
    for j in (0, 5):
        x = np.zeros((1, arch.hidden))
        x[0, j] = 1.0
        k, v = _cache(arch, rng, 4)
        r = O.block_decode(arch, False, w_qkv, w_g, w_o, x, [_seq(k, v, 0, 0)])
        col = wq[:, j]
        assert np.array_equal(r.qkv[0], col)
        assert np.array_equal(r.q_roped[0], col[:qd].reshape(arch.num_heads, arch.head_dim))
        assert np.array_equal(r.k16[0].astype(np.float64),
                              col[qd:qd + kd].astype(np.float16).astype(np.float64)
                              .reshape(arch.num_kv_heads, arch.head_dim))
        assert np.array_equal(r.v16[0].astype(np.float64),
                              col[qd + kd:].astype(np.float16).astype(np.float64)
                              .reshape(arch.num_kv_heads, arch.head_dim))
        assert r.slots[0] == 0
        assert np.array_equal(r.k_caches[0][0], r.k16[0])
        assert np.array_equal(r.v_caches[0][0], r.v16[0])
        assert np.array_equal(r.k_caches[0][1:], k[1:])


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------

def pin_rope_params_printed(O):
    for c in _golden("rope_params_for.json")["cases"]:
        got = O.rope_params_for(c["is_full"], c["full_rotary_dim"], c["head_dim"],
                                c["full_theta"], c["sliding_theta"])
        assert tuple(got) == (c["rotary_dim"], c["theta"]), (c, got)


def _x(rng, heads=4, d=256):
    return rng.standard_normal((heads, d))


def pin_rope_identity_at_position_zero(O):
    x = _x(_rng(3))
    for r, th in ((64, 5e6), (256, 1e4)):
        assert np.array_equal(O.rope_neox(x, 0, r, th), x)


def pin_rope_pair_norm_preserved(O):
    x = _x(_rng(4))
    for r, th in ((64, 5e6), (256, 1e4)):
        h = r // 2
        for pos in (1, 63, 4095, 32767):
            y = O.rope_neox(x, pos, r, th)
            n0 = x[:, :h] ** 2 + x[:, h:r] ** 2
            n1 = y[:, :h] ** 2 + y[:, h:r] ** 2
            assert np.allclose(n0, n1, rtol=1e-12, atol=1e-14)


def pin_rope_leaves_tail_dims(O):
    x = _x(_rng(5))
    y = O.rope_neox(x, 777, 64, 5e6)
    assert np.array_equal(y[:, 64:], x[:, 64:])
    assert not np.allclose(y[:, :64], x[:, :64])


def pin_rope_angle_closed_forms(O):
    """A unit vector on dim i turns to (cos a, sin a) on dims (i, i + r/2):
    pair 0 turns by exactly the position, pair r/4 by position / sqrt(theta)."""
    for r, th in ((64, 5e6), (256, 1e4)):
        h = r // 2
        for pos in (3, 100, 32767):
            for i, ang in ((0, float(pos)), (r // 4, pos / math.sqrt(th))):
                x = np.zeros((1, 256))
                x[0, i] = 1.0
                y = O.rope_neox(x, pos, r, th)
                assert abs(y[0, i] - math.cos(ang)) < 1e-9, (r, pos, i)
                assert abs(y[0, i + h] - math.sin(ang)) < 1e-9, (r, pos, i)


def pin_rope_whole_head_is_complex_rotation(O):
    """r = D: the head is 128 complex numbers x[j] + i x[j+128], each multiplied
    by a unit phasor whose frequency falls geometrically by theta^(-1/128)."""
    x = _x(_rng(6))
    th = 1e4
    ratio = th ** (-1.0 / 128.0)
    freq = np.ones(128)
    for j in range(1, 128):
        freq[j] = freq[j - 1] * ratio
    for pos in (1, 511, 32767):
        z = (x[:, :128] + 1j * x[:, 128:]) * np.exp(1j * pos * freq)
        y = O.rope_neox(x, pos, 256, th)
        assert np.allclose(y[:, :128], z.real, atol=1e-8)
        assert np.allclose(y[:, 128:], z.imag, atol=1e-8)


def pin_rope_composition(O):
    x = _x(_rng(7))
    for r, th in ((64, 5e6), (256, 1e4)):
        a, b = 1234, 777
        y = O.rope_neox(O.rope_neox(x, a, r, th), b, r, th)
        assert np.allclose(y, O.rope_neox(x, a + b, r, th), atol=1e-9)


def pin_rope_relative_position(O):
    rng = _rng(8)
    q, k = _x(rng, 1), _x(rng, 1)
    for r, th in ((64, 5e6), (256, 1e4)):
        base = float(np.sum(O.rope_neox(q, 900, r, th) * O.rope_neox(k, 100, r, th)))
        for shift in (1, 37, 20000):
            s = float(np.sum(O.rope_neox(q, 900 + shift, r, th)
                             * O.rope_neox(k, 100 + shift, r, th)))
            assert abs(s - base) < 1e-8 * (1 + abs(base))


# ----------------------------------------------------------------------------
# window / ring
# ----------------------------------------------------------------------------

def pin_window_worked_cases(O):
    g = _golden("kv_window_cases.json")
    for full, pos, win, ring, sl, ks, ar, slot in g["cases"]:
        assert tuple(O.kv_window(full, pos, win, ring)) == (sl, ks, ar), (full, pos, ring)
        assert O.kv_slot(pos, ring if not full else 0) == slot, (pos, ring)


def pin_ring_brute_force(O):
    """Simulate a ring buffer written one position at a time; the rows read at
    each step must hold exactly the last min(seq_len, window) positions."""
    for window, ring in ((512, 512), (512, 640), (6, 6), (6, 9)):
        owner = [-1] * ring
        for pos in range(0, 3 * ring + 5):
            owner[O.kv_slot(pos, ring)] = pos
            sl, ks, ar = O.kv_window(False, pos, window, ring)
            rows = O.physical_rows(sl, ks, ar)
            assert [owner[int(r)] for r in rows] == list(range(max(0, pos - window + 1), pos + 1)), \
                (window, ring, pos)
    for pos in (0, 5, 100):
        sl, ks, ar = O.kv_window(True, pos, 6, 0)
        assert list(O.physical_rows(sl, ks, ar)) == list(range(pos + 1))


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def _sdpa_fp64(q, k_cache, v_cache, mask, scale, group):
    import torch
    kk = torch.from_numpy(k_cache.astype(np.float64)).permute(1, 0, 2)   # [Hk][cap][D]
    vv = torch.from_numpy(v_cache.astype(np.float64)).permute(1, 0, 2)
    kk = kk.repeat_interleave(group, dim=0).unsqueeze(0)
    vv = vv.repeat_interleave(group, dim=0).unsqueeze(0)
    qq = torch.from_numpy(q).unsqueeze(0).unsqueeze(2)                     # [1][Hq][1][D]
    m = torch.from_numpy(mask).view(1, 1, 1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m,
                                                           scale=scale)
    return out[0, :, 0, :].numpy()


def pin_attention_matches_library_sdpa(O):
    rng = _rng(9)
    hq, hk, d = 16, 4, 64
    for full, pos, ring in ((True, 40, 0), (False, 40, 0), (False, 40, 16), (False, 12, 16)):
        window = 10
        cap = ring if ring else pos + 1
        k = rng.standard_normal((cap, hk, d)).astype(np.float16)
        v = rng.standard_normal((cap, hk, d)).astype(np.float16)
        q = rng.standard_normal((hq, d))
        sl, ks, ar = O.kv_window(full, pos, window, ring)
        # which physical rows are in the window, by simulating the writes
        owner = {}
        for t in range(pos + 1):
            owner[t % ring if ring else t] = t
        lo = 0 if full else max(0, pos - window + 1)
        mask = np.array([owner.get(r, -1) >= lo for r in range(cap)])
        got = O.attention_decode(q, k, v, sl, ks, ar, 0.125)
        want = _sdpa_fp64(q, k, v, mask, 0.125, hq // hk)
        assert np.allclose(got, want, rtol=1e-11, atol=1e-12), (full, pos, ring)


def pin_attention_zero_query_is_window_mean(O):
    rng = _rng(10)
    hq, hk, d = 8, 2, 16
    k = rng.standard_normal((20, hk, d)).astype(np.float16)
    v = rng.standard_normal((20, hk, d)).astype(np.float16)
    got = O.attention_decode(np.zeros((hq, d)), k, v, 20, 13, 0, 0.25)
    for h in range(hq):
        want = v[13:20, h // 4].astype(np.float64).mean(axis=0)
        assert np.allclose(got[h], want, rtol=1e-13, atol=1e-14)


def pin_attention_gqa_head_map(O):
    """KV head g holds the constant g + 1: query head h must return h // 4 + 1."""
    rng = _rng(11)
    hq, hk, d, n = 16, 4, 32, 9
    k = rng.standard_normal((n, hk, d)).astype(np.float16)
    v = np.zeros((n, hk, d), np.float16)
    for g in range(hk):
        v[:, g, :] = g + 1
    got = O.attention_decode(rng.standard_normal((hq, d)), k, v, n, 0, 0, 0.2)
    for h in range(hq):
        assert np.allclose(got[h], h // 4 + 1, rtol=1e-13)


def pin_attention_scale(O):
    """Two keys: the weight ratio of their probabilities is exp(scale * dq)."""
    d = 4
    k = np.zeros((2, 1, d), np.float16)
    k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, d), np.float16)
    v[1, 0, 0] = 1.0                      # output dim 0 = p(row 1)
    q = np.zeros((1, d))
    q[0, 0] = 3.0
    a = O.attention_decode(q, k, v, 2, 0, 0, 0.5)
    p1 = math.exp(1.5) / (1 + math.exp(1.5))
    assert abs(a[0, 0] - p1) < 1e-14


def pin_single_key_returns_its_value(O):
    """Position 0: the only key is this token's, so attention returns v16
    exactly, and a zero gate logit (g_proj = 0) halves it exactly."""
    arch = tiny_arch()
    rng = _rng(12)
    w_qkv, _, w_o = _tiny_weights(arch, rng)
    w_g = np.zeros((arch.num_heads, arch.hidden), np.uint16)
    x = rng.standard_normal((1, arch.hidden))
    for full in (True, False):
        k, v = _cache(arch, rng, 3)
        r = O.block_decode(arch, full, w_qkv, w_g, w_o, x, [_seq(k, v, 0, 0)])
        for h in range(arch.num_heads):
            vv = r.v16[0][h // 2].astype(np.float64)
            assert np.array_equal(r.attn[0][h], vv)
            assert np.array_equal(r.gated[0].reshape(arch.num_heads, -1)[h], 0.5 * vv)


def pin_zero_gate_logit_is_half(O):
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    a = _rng(13).standard_normal((4, 8))
    assert np.array_equal(O.head_gate(a, np.zeros(4)), 0.5 * a)


def pin_gate_is_headwise_and_before_o_proj(O):
    """Gate logits +60 on head 0 and -60 elsewhere: the output is W_o applied
    to head 0's attention alone (other heads scaled by ~1e-26)."""
    arch = tiny_arch()
    rng = _rng(14)
    w_qkv, _, w_o = _tiny_weights(arch, rng)
    x = rng.standard_normal((1, arch.hidden))
    # build g_proj rows so that g = W_g x takes the wanted values exactly enough
    target = np.array([60.0, -60.0, -60.0, -60.0])
    w_g_f = np.outer(target, x[0]) / float(x[0] @ x[0])
    w_g = _bf16(w_g_f.astype(np.float32))
    k, v = _cache(arch, rng, 9)
    r = O.block_decode(arch, True, w_qkv, w_g, w_o, x, [_seq(k, v, 0, 8)])
    assert r.gate_logits[0][0] > 50 and np.all(r.gate_logits[0][1:] < -50)
    d = arch.head_dim
    wo = O.bf16_bits_to_f64(w_o)
    want = wo[:, :d] @ r.attn[0][0]
    assert np.allclose(r.out[0], want, rtol=1e-9, atol=1e-12)


def pin_ring_equals_linear(O):
    """Window-512 attention through a 512-slot ring equals, bitwise, linear
    addressing over the same last 512 positions."""
    rng = _rng(15)
    hq, hk, d = 16, 4, 32
    q = rng.standard_normal((hq, d))
    for pos in (511, 512, 513, 1000, 32768 + 137):
        lo = max(0, pos - 511)
        rows_k = rng.standard_normal((pos + 1 - lo, hk, d)).astype(np.float16)
        rows_v = rng.standard_normal((pos + 1 - lo, hk, d)).astype(np.float16)
        lin_k = np.zeros((pos + 1, hk, d), np.float16)
        lin_v = np.zeros((pos + 1, hk, d), np.float16)
        lin_k[lo:], lin_v[lo:] = rows_k, rows_v
        ring_k = np.full((512, hk, d), np.nan, np.float16)
        ring_v = np.full((512, hk, d), np.nan, np.float16)
        for t in range(lo, pos + 1):
            ring_k[t % 512], ring_v[t % 512] = lin_k[t], lin_v[t]
        sl, ks, ar = O.kv_window(False, pos, 512, 512)
        a_ring = O.attention_decode(q, ring_k, ring_v, sl, ks, ar, 0.0625)
        sl2, ks2, ar2 = O.kv_window(False, pos, 512, 0)
        a_lin = O.attention_decode(q, lin_k, lin_v, sl2, ks2, ar2, 0.0625)
        assert np.array_equal(a_ring, a_lin), pos


def pin_block_reads_only_the_window(O):
    """Rows outside the window are NaN; the block output stays finite."""
    arch = tiny_arch(window=6)
    rng = _rng(16)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    x = rng.standard_normal((1, arch.hidden))
    for pos, ring in ((20, 0), (20, 6), (20, 8), (3, 6)):
        cap = ring if ring else pos + 1
        k, v = _cache(arch, rng, cap)
        lo = max(0, pos - 5)
        for r in range(cap):
            owner = [t for t in range(pos + 1) if (t % ring if ring else t) == r]
            if not owner or owner[-1] < lo:
                k[r], v[r] = np.nan, np.nan
        res = O.block_decode(arch, False, w_qkv, w_g, w_o, x, [_seq(k, v, ring, pos)])
        assert np.all(np.isfinite(res.out)), (pos, ring)


def pin_block_q_k_rotated_v_not(O):
    """x = e_j at position p > 0: q and the written k row are the q and k
    columns turned as complex numbers (sliding layer, r = D; k then rounded to
    fp16), while the v row is the unturned v column in fp16."""
    arch = tiny_arch()
    rng = _rng(17)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    wq = O.bf16_bits_to_f64(w_qkv)
    d, hk = arch.head_dim, arch.num_kv_heads
    qd = arch.num_heads * d
    j, pos = 3, 5
    x = np.zeros((1, arch.hidden))
    x[0, j] = 1.0
    k, v = _cache(arch, rng, pos + 1)
    r = O.block_decode(arch, False, w_qkv, w_g, w_o, x, [_seq(k, v, 0, pos)])
    kcol = wq[qd:qd + hk * d, j].reshape(hk, d)
    half = d // 2
    freq = np.array([arch.rope_theta ** (-(2.0 * i) / d) for i in range(half)])
    z = (kcol[:, :half] + 1j * kcol[:, half:]) * np.exp(1j * pos * freq)
    want = np.concatenate([z.real, z.imag], axis=1).astype(np.float16).astype(np.float64)
    got = r.k16[0].astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp), np.max(np.abs(got - want))
    vcol = wq[qd + hk * d:, j].reshape(hk, d).astype(np.float16)
    assert np.array_equal(r.v16[0], vcol)
    qcol = wq[:qd, j].reshape(arch.num_heads, d)
    zq = (qcol[:, :half] + 1j * qcol[:, half:]) * np.exp(1j * pos * freq)
    assert np.allclose(r.q_roped[0], np.concatenate([zq.real, zq.imag], axis=1),
                       rtol=1e-12, atol=1e-12)


def pin_block_zero_input(O):
    """x = 0: q = k = v = 0 and the gate logits are 0, so each head returns half
    the mean of its KV head's V rows over the window (this token's row is 0)."""
    arch = tiny_arch(window=6)
    rng = _rng(18)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    pos = 10
    k, v = _cache(arch, rng, pos + 1)
    r = O.block_decode(arch, False, w_qkv, w_g, w_o, np.zeros((1, arch.hidden)),
                       [_seq(k, v, 0, pos)])
    vv = v.astype(np.float64).copy()
    vv[pos] = 0.0
    wo = O.bf16_bits_to_f64(w_o)
    gated = np.concatenate([0.5 * vv[5:11, h // 2].mean(axis=0) for h in range(4)])
    assert np.allclose(r.gated[0], gated, rtol=1e-13, atol=1e-15)
    assert np.allclose(r.out[0], wo @ gated, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# several tokens of one sequence
# ----------------------------------------------------------------------------

def pin_chunk_of_one_is_the_block(O):
    """A one-token chunk is the single-token block (output and cache)."""
    arch = tiny_arch(window=6)
    rng = _rng(20)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    x = rng.standard_normal((1, arch.hidden))
    k, v = _cache(arch, rng, 12)
    c = O.block_chunk(arch, True, w_qkv, w_g, w_o, x, _seq(k, v, 0, 9), 1)
    b = O.block_decode(arch, True, w_qkv, w_g, w_o, x, [_seq(k, v, 0, 9)])
    assert np.array_equal(c.out, b.out)
    assert np.array_equal(c.k_cache, b.k_caches[0]) and np.array_equal(c.v_cache, b.v_caches[0])


def pin_chunk_is_causal(O):
    """Token t's output does not depend on the inputs of later tokens, and it
    does depend on every earlier token's input (through the k, v rows that
    token wrote)."""
    arch = tiny_arch(window=6)
    rng = _rng(21)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    m, pos = 4, 7
    x = rng.standard_normal((m, arch.hidden))
    k, v = _cache(arch, rng, pos + m)
    for is_full in (True, False):
        base = O.block_chunk(arch, is_full, w_qkv, w_g, w_o, x, _seq(k, v, 0, pos), m)
        for t in range(m):
            x2 = x.copy()
            x2[t] += 1.0
            r = O.block_chunk(arch, is_full, w_qkv, w_g, w_o, x2, _seq(k, v, 0, pos), m)
            assert np.array_equal(r.out[:t], base.out[:t]), (is_full, t)
            assert np.all(np.abs(r.out[t:] - base.out[t:]).max(axis=1) > 1e-9), (is_full, t)


def pin_chunk_ring_equals_linear(O):
    """A chunk through a ring of sliding_window + M - 1 slots equals, bitwise,
    the chunk over a linear cache holding the same history."""
    arch = tiny_arch(window=6)
    rng = _rng(22)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    m, ring = 3, 8
    for pos in (2, 9, 30):
        x = rng.standard_normal((m, arch.hidden))
        lin_k, lin_v = _cache(arch, rng, pos + m)
        ring_k = np.full((ring, arch.num_kv_heads, arch.head_dim), np.nan, np.float16)
        ring_v = ring_k.copy()
        for t in range(max(0, pos - ring), pos):
            ring_k[t % ring], ring_v[t % ring] = lin_k[t], lin_v[t]
        a = O.block_chunk(arch, False, w_qkv, w_g, w_o, x, _seq(ring_k, ring_v, ring, pos), m)
        b = O.block_chunk(arch, False, w_qkv, w_g, w_o, x, _seq(lin_k, lin_v, 0, pos), m)
        assert np.array_equal(a.out, b.out), pos
        assert a.slots == [(pos + t) % ring for t in range(m)] and b.slots == list(range(pos, pos + m))


# ----------------------------------------------------------------------------
# stack harness
# ----------------------------------------------------------------------------

def pin_rms_norm_closed_form(O):
    for c in (0.5, -3.0, 1e-4):
        h = np.full((1, 32), c)
        w = _bf16(np.full(32, 2.0, np.float32))
        got = O.rms_norm(h, w, 1e-6)
        assert np.allclose(got, 2.0 * c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    h = np.array([[3.0, 4.0]])
    got = O.rms_norm(h, _bf16(np.ones(2, np.float32)), 0.0)
    assert np.allclose(got, h / math.sqrt(12.5), rtol=1e-15)


def pin_stack_is_residual_sum(O):
    """Two layers whose o_proj is zero leave h unchanged; with o_proj live the
    returned h is h0 plus the per-layer outputs."""
    arch = tiny_arch()
    rng = _rng(19)
    h0 = rng.standard_normal((1, arch.hidden))
    layers = []
    for li in range(2):
        w_qkv, w_g, w_o = _tiny_weights(arch, rng)
        k, v = _cache(arch, rng, 4)
        layers.append(SimpleNamespace(is_full=bool(li % 2), w_norm=_bf16(np.ones(arch.hidden, np.float32)),
                                      w_qkv=w_qkv, w_g=w_g, w_o=np.zeros_like(w_o),
                                      cache=_seq(k, v, 0, 3)))
    r = O.stack_decode(arch, h0, layers)
    assert np.array_equal(r.h, h0)
    for li in range(2):
        layers[li].w_o = _tiny_weights(arch, rng)[2]
    r = O.stack_decode(arch, h0, layers)
    assert np.allclose(r.h, h0 + r.block_outs[0] + r.block_outs[1], rtol=1e-14)
    assert np.allclose(r.normed[0], h0 / np.sqrt(np.mean(h0 ** 2) + 1e-6), rtol=1e-13)




# ----------------------------------------------------------------------------
# the rest of the decoder layer: erf GELU, gated MLP, whole-layer stack
# ----------------------------------------------------------------------------

def pin_gelu_erf_closed_forms(O):
    """GELU(x) = x * Phi(x) with the standard normal CDF Phi (textbook values to
    10 digits), GELU(0) = 0, and GELU(x) - GELU(-x) = x (erf is odd).  The tanh
    form differs from these by ~1e-4."""
    phi = {1.0: 0.8413447461, 2.0: 0.9772498681, 0.5: 0.6914624613, 3.0: 0.9986501020}
    for x, p in phi.items():
        assert abs(float(O.gelu_erf(np.array([x]))[0]) - x * p) < 1e-9 * max(1.0, x)
        assert abs(float(O.gelu_erf(np.array([-x]))[0]) + x * (1.0 - p)) < 1e-9 * max(1.0, x)
    assert float(O.gelu_erf(np.array([0.0]))[0]) == 0.0
    x = np.linspace(-6.0, 6.0, 49)
    assert np.max(np.abs(O.gelu_erf(x) - O.gelu_erf(-x) - x)) < 1e-14


def _tiny_mlp(rng, hidden=8, inter=12):
    return (_bf16(1.0 + 0.1 * rng.standard_normal(hidden).astype(np.float32)),
            _bf16(0.5 * rng.standard_normal((inter, hidden)).astype(np.float32)),
            _bf16(0.5 * rng.standard_normal((inter, hidden)).astype(np.float32)),
            _bf16(0.5 * rng.standard_normal((hidden, inter)).astype(np.float32)))


def pin_mlp_brute_force(O):
    """The layer's last two lines written out element by element (math.erf)."""
    rng = _rng(41)
    w_post, w_gate, w_up, w_down = _tiny_mlp(rng)
    dec = lambda b: float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])  # noqa: E731
    hid, inter = w_gate.shape[1], w_gate.shape[0]
    for b in range(2):
        h = rng.standard_normal(hid)
        ms = sum(v * v for v in h) / hid
        x = [h[c] / math.sqrt(ms + 1e-6) * dec(w_post[c]) for c in range(hid)]
        act = []
        for i in range(inter):
            g = sum(dec(w_gate[i, c]) * x[c] for c in range(hid))
            u = sum(dec(w_up[i, c]) * x[c] for c in range(hid))
            act.append(0.5 * g * (1.0 + math.erf(g / math.sqrt(2.0))) * u)
        want = [h[r] + sum(dec(w_down[r, i]) * act[i] for i in range(inter)) for r in range(hid)]
        got = O.mlp_decode(h, w_post, w_gate, w_up, w_down, 1e-6).h[0]
        assert np.max(np.abs(got - np.array(want))) < 1e-11 * (1 + np.max(np.abs(want)))


def pin_mlp_zero_gate_adds_nothing(O):
    """gate_proj = 0 makes GELU(0) = 0, so the MLP leaves h exactly as it was."""
    rng = _rng(42)
    w_post, w_gate, w_up, w_down = _tiny_mlp(rng)
    h = rng.standard_normal((3, w_gate.shape[1]))
    r = O.mlp_decode(h, w_post, np.zeros_like(w_gate), w_up, w_down, 1e-6)
    assert np.array_equal(r.h, h) and not r.out.any()


def pin_decoder_stack_order(O):
    """Whole layers: the MLP reads the stream after the attention's add, and the
    stack is h0 plus every layer's contribution."""
    arch = tiny_arch()
    rng = _rng(43)
    layers = []
    for li in range(3):
        w_qkv, w_g, w_o = _tiny_weights(arch, rng)
        k, v = _cache(arch, rng, 8)
        w_post, w_gate, w_up, w_down = _tiny_mlp(rng, hidden=arch.hidden, inter=24)
        layers.append(SimpleNamespace(is_full=li == 2, w_norm=_bf16(1.0 + 0.1 * rng.standard_normal(
            arch.hidden).astype(np.float32)), w_qkv=w_qkv, w_g=w_g, w_o=w_o,
            cache=_seq(k, v, 0, 5), w_post=w_post, w_gate=w_gate, w_up=w_up, w_down=w_down))
    h0 = rng.standard_normal((1, arch.hidden))
    res = O.decoder_stack_decode(arch, h0, layers)
    h = h0.copy()
    for L in layers:
        # attention block on the normed stream, raw add, then the MLP on the new stream
        xn = h / np.sqrt(np.mean(h * h) + 1e-6) * O.bf16_bits_to_f64(L.w_norm)
        a = O.block_decode(arch, L.is_full, L.w_qkv, L.w_g, L.w_o, xn, [L.cache]).out
        h = h + a
        h = O.mlp_decode(h, L.w_post, L.w_gate, L.w_up, L.w_down, 1e-6).h
    assert np.max(np.abs(res.h - h)) < 1e-12 * (1 + np.max(np.abs(h)))
    assert np.max(np.abs(h0 + sum(res.block_outs) - res.h)) < 1e-12 * (1 + np.max(np.abs(h)))


# ----------------------------------------------------------------------------
# the ends of the decode step: raw embedding row, final norm, tied head
# ----------------------------------------------------------------------------

def pin_embed_is_the_raw_row(O):
    """The embedding row is used as stored: no sqrt(hidden) scale, no norm
    (the bf16 value decoded through struct, independently of the oracle)."""
    import struct
    rng = _rng(51)
    e = _bf16(rng.standard_normal((10, 16)).astype(np.float32))
    ids = [3, 0, 9, 3]
    got = O.embed_gather(e, ids)
    for b, t in enumerate(ids):
        want = [struct.unpack("<f", struct.pack("<I", int(v) << 16))[0] for v in e[t]]
        assert np.array_equal(got[b], np.array(want))


def pin_lm_head_one_hot_closed_form(O):
    """h = e_k: mean(h^2) = 1/H, so logits_j = E[j][k] * w_k / sqrt(1/H + eps)."""
    rng = _rng(52)
    hid, vocab, eps = 16, 24, 1e-6
    e = _bf16(rng.standard_normal((vocab, hid)).astype(np.float32))
    w = _bf16(1.0 + 0.1 * rng.standard_normal(hid).astype(np.float32))
    ev, wv = O.bf16_bits_to_f64(e), O.bf16_bits_to_f64(w)
    for k in (0, 5, 15):
        h = np.zeros((1, hid))
        h[0, k] = 1.0
        want = ev[:, k] * wv[k] / math.sqrt(1.0 / hid + eps)
        assert np.max(np.abs(O.lm_head(h, w, e, eps)[0] - want)) < 1e-12


def pin_lm_head_brute_force(O):
    rng = _rng(53)
    hid, vocab = 8, 11
    e = _bf16(rng.standard_normal((vocab, hid)).astype(np.float32))
    w = _bf16(1.0 + 0.1 * rng.standard_normal(hid).astype(np.float32))
    dec = lambda b: float(np.array([int(b) << 16], np.uint32).view(np.float32)[0])  # noqa: E731
    h = rng.standard_normal((2, hid))
    got = O.lm_head(h, w, e, 1e-6)
    for b in range(2):
        r = math.sqrt(sum(v * v for v in h[b]) / hid + 1e-6)
        for j in range(vocab):
            want = sum(dec(e[j, c]) * h[b, c] / r * dec(w[c]) for c in range(hid))
            assert abs(got[b, j] - want) < 1e-12 * (1 + abs(want))


# ----------------------------------------------------------------------------
# attention sinks (reading O23: one more logit per head, no value row)
# ----------------------------------------------------------------------------

def pin_sink_closed_form(O):
    """Zero keys make every score 0, so with n rows and sink sigma each row
    weighs 1 / (n + e^sigma): sigma = ln 3 over 5 rows gives 1/8, ln 11 gives
    1/16, -inf gives the plain mean 1/5, whatever the scale and the query."""
    rng = _rng(40)
    hq, hk, d, n = 4, 2, 8, 5
    k = np.zeros((n, hk, d), np.float16)
    v = rng.standard_normal((n, hk, d)).astype(np.float16)
    q = rng.standard_normal((hq, d))
    sinks = np.array([math.log(3.0), math.log(11.0), -np.inf, 0.0])
    got = O.attention_decode(q, k, v, n, 0, 0, 0.37, sinks)
    for h, den in zip(range(hq), (8.0, 16.0, 5.0, 6.0)):
        want = v[:, h // 2].astype(np.float64).sum(axis=0) / den
        assert np.allclose(got[h], want, rtol=1e-13, atol=1e-15), h


def pin_sink_is_a_valueless_extra_key(O):
    """Against scipy's softmax over the window's scores with sigma_h appended
    as one more entry, whose value row is zero; through a ring window."""
    from scipy.special import softmax
    rng = _rng(41)
    hq, hk, d, ring, pos, window = 8, 2, 16, 12, 30, 9
    k = rng.standard_normal((ring, hk, d)).astype(np.float16)
    v = rng.standard_normal((ring, hk, d)).astype(np.float16)
    q = 2.0 * rng.standard_normal((hq, d))
    sinks = rng.standard_normal(hq) * 3.0
    sl, ks, ar = O.kv_window(False, pos, window, ring)
    got = O.attention_decode(q, k, v, sl, ks, ar, 0.3, sinks)
    rows = [t % ring for t in range(pos - window + 1, pos + 1)]
    for h in range(hq):
        kk = k[rows, h // 4].astype(np.float64)
        vv = v[rows, h // 4].astype(np.float64)
        p = softmax(np.append(0.3 * (kk @ q[h]), sinks[h]))
        want = p[:-1] @ vv
        assert np.allclose(got[h], want, rtol=1e-12, atol=1e-14), h


def pin_sink_scales_the_plain_attention(O):
    """With S = sum_t e^{s_t}, the sink multiplies the plain attention by
    S / (S + e^sigma): checked per head with S summed by brute force."""
    rng = _rng(42)
    hq, hk, d, n = 4, 1, 8, 7
    k = rng.standard_normal((n, hk, d)).astype(np.float16)
    v = rng.standard_normal((n, hk, d)).astype(np.float16)
    q = rng.standard_normal((hq, d))
    sinks = np.array([-2.0, 0.5, 3.0, 40.0])
    plain = O.attention_decode(q, k, v, n, 0, 0, 0.5)
    got = O.attention_decode(q, k, v, n, 0, 0, 0.5, sinks)
    for h in range(hq):
        S = sum(math.exp(0.5 * float(np.dot(k[t, 0].astype(np.float64), q[h]))) for t in range(n))
        f = S / (S + math.exp(sinks[h]))
        assert np.allclose(got[h], f * plain[h], rtol=1e-12, atol=1e-300), h


def pin_block_and_chunk_pass_sinks_on(O):
    """The block and the several-token path hand the sinks to the attention:
    sinks of -inf change nothing (bit for bit), sinks of +1e4 make every
    attention weight underflow to 0, so gated attention and output are 0."""
    arch = tiny_arch()
    rng = _rng(43)
    w_qkv, w_g, w_o = _tiny_weights(arch, rng)
    x = rng.standard_normal((3, arch.hidden))
    k, v = _cache(arch, rng, 16)
    seq = _seq(k, v, 0, 6)
    plain = O.block_decode(arch, True, w_qkv, w_g, w_o, x[:1], [seq])
    minus = O.block_decode(arch, True, w_qkv, w_g, w_o, x[:1], [seq],
                           np.full(arch.num_heads, -np.inf))
    assert np.array_equal(plain.out, minus.out) and np.array_equal(plain.gated, minus.gated)
    big = O.block_decode(arch, True, w_qkv, w_g, w_o, x[:1], [seq], np.full(arch.num_heads, 1e4))
    assert not np.any(big.gated) and not np.any(big.out)
    assert np.array_equal(big.k_caches[0], plain.k_caches[0])
    c_plain = O.block_chunk(arch, False, w_qkv, w_g, w_o, x, seq, 3)
    c_big = O.block_chunk(arch, False, w_qkv, w_g, w_o, x, seq, 3, np.full(arch.num_heads, 1e4))
    assert not np.any(c_big.out)
    assert np.array_equal(c_big.k_cache, c_plain.k_cache)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
