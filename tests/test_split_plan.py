"""The split-K plan on the host (no GPU): over random batches, context
lengths, KV-head counts and ring settings, every plan the attention launches
would use keeps the invariants the kernels rely on.

  * rows per chunk are a positive multiple of 64 (whole 16-row tiles for
    every wave of a workgroup);
  * the chunks of each sequence cover its window exactly once:
    ceil(n / chunk) chunks, the last one holding the remainder;
  * no launch group writes more chunk partials than gqa_workspace_size
    provisions (max_group_chunks <= chunk_bound, and the block's workspace
    layout for that many chunks fits in gqa_workspace_size's bytes);
  * a chunk of a ring sequence spans at most ring_capacity rows, so it wraps
    around the ring at most once (the kernels' row map subtracts the ring
    size once);
  * the one-chunk direct form is taken only for windows of at most 128 rows,
    and two-wave workgroups only for several sequences.
"""
from __future__ import annotations

import numpy as np
import pytest

import gqa_attention_block_amd as gqa

KV_ROW_QUANTUM = 64


def _round_up(x, a):
    return (x + a - 1) // a * a


SYNC_BYTES = 32768   # the one-launch block's flag words at the start of every workspace


def _layout_bytes(arch, batch, chunks):
    """The block's workspace: the synchronisation words, q, gate logits, gated
    attention, partial O and partial (m, l), each rounded up to 256 bytes."""
    q = SYNC_BYTES + _round_up(batch * arch.q_dim * 4, 256)
    g = _round_up(batch * arch.num_heads * 4, 256)
    a = _round_up(batch * arch.q_dim * 4, 256)
    po = _round_up(chunks * arch.num_heads * arch.head_dim * 4, 256)
    pm = _round_up(chunks * arch.num_heads * 2 * 4, 256)
    return q + g + a + po + pm


def _check_plan(arch, is_full, positions, ring):
    plan = gqa.split_plan(arch, is_full, positions, ring_capacity=ring)
    plan_p = gqa.split_plan(arch, is_full, positions, ring_capacity=ring, allow_direct=False)
    windows = [gqa.kv_window(is_full, p, arch.sliding_window, ring) for p in positions]
    ns = [sl - ks for sl, ks, _ in windows]
    for pl, direct_ok in ((plan, True), (plan_p, False)):
        c = pl.chunk_rows
        assert c >= KV_ROW_QUANTUM and c % KV_ROW_QUANTUM == 0, pl
        assert pl.waves in (2, 4), pl
        if pl.waves == 2:
            assert len(positions) >= 2 and not pl.direct, pl
        if pl.direct:
            assert direct_ok and max(ns) <= 128 and c >= max(ns), (pl, max(ns))
        # groups of at most 32 sequences, chunk counts per group
        per_group = [sum(-(-n // c) for n in ns[i:i + 32]) for i in range(0, len(ns), 32)]
        assert pl.groups == len(per_group), pl
        assert pl.max_group_chunks == max(per_group), (pl, per_group)
        assert pl.max_group_chunks <= pl.chunk_bound, pl
        for n in ns:
            k = -(-n // c)
            assert (k - 1) * c < n <= k * c            # exact cover, last chunk non-empty
        for (sl, ks, ar), n in zip(windows, ns):
            if ar:
                assert min(c, n) <= ar                 # a ring chunk wraps at most once
    ws = gqa.workspace_size(arch, len(positions), max(positions) + 1)
    assert _layout_bytes(arch, len(positions), plan.max_group_chunks) <= ws
    return plan


@pytest.mark.parametrize("num_kv_heads", [1, 2, 4, 8])
def test_random_plans_keep_their_invariants(num_kv_heads):
    rng = np.random.default_rng([7, num_kv_heads])
    arch = gqa.Arch(hidden=1024, num_heads=4 * num_kv_heads, num_kv_heads=num_kv_heads)
    for trial in range(300):
        batch = int(rng.choice([1, 1, 2, 3, 5, 8, 12, 16, 31, 32, 33, 47, 64, 80]))
        hi = int(rng.choice([64, 130, 600, 5000, 20000, 70000]))
        positions = [int(p) for p in rng.integers(0, hi, size=batch)]
        kind = int(rng.integers(0, 3))
        if kind == 0:
            _check_plan(arch, True, positions, 0)
        else:
            ring = int(rng.choice([512, 513, 1024, 4096]))
            _check_plan(arch, False, positions, ring)


@pytest.mark.parametrize("n,chunk", [(32768, 512), (4096, 128), (100, 128)])
def test_known_one_sequence_plans(n, chunk):
    """One full-layer sequence: 32K rows in 64 chunks of 512 (256 workgroups
    over the 4 KV heads), 4096 rows in 32 chunks of 128 (a short launch aims
    for half the workgroups: 128), 100 rows in one direct chunk."""
    arch = gqa.Arch(hidden=2560)
    plan = gqa.split_plan(arch, True, [n - 1])
    assert plan.chunk_rows == chunk, plan
    assert plan.direct == (n <= 128)
    assert plan.waves == 4
