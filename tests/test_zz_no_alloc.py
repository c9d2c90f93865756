"""gqa_attention_block_decode_noalloc: the block with its workspace in the
library's static per-GPU scratch.  Two calls in a row through the C ABI --
a batch of three full-layer sequences, then one shorter sequence on a smaller
layer -- each against gqa_attention_block_decode with a caller workspace on
the same inputs (same bar as every block test, and the same cache rows), and
the size limit refused with a clear status before anything is launched."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gqa_attention_block_amd as gqa
import synth
from tests.gpu_util import DevBlock, assert_parity, say

WS_SMALL = 3

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a CPU host only with -m gpu
    pytest.skip("needs a GPU", allow_module_level=True)


def _both(case):
    ref_dev = DevBlock(case)
    out_ref = ref_dev.run_block()
    dev = DevBlock(case)
    out = torch.empty((case.batch, dev.arch.hidden), dtype=torch.float32, device="cuda")
    gqa.attention_block_decode_noalloc(dev.arch, dev.w_qkv, dev.w_g, dev.w_o, case.is_full, dev.seqs(),
                                       dev.x, out)
    torch.cuda.synchronize()
    for i in range(case.batch):
        assert torch.equal(dev.k[i], ref_dev.k[i]) and torch.equal(dev.v[i], ref_dev.v[i]), "cache rows differ"
    return out.cpu().numpy(), out_ref


def test_noalloc_matches_the_workspace_block_on_two_calls():
    first = synth.block_case("noalloc_full_h2560_b3", 2560, True, [5000, 700, 9000], seed=0, case_id=80)
    say(f"noalloc call 1: {first.name}")
    got, ref = _both(first)
    assert_parity(got, ref, "noalloc call 1 against the workspace block")
    second = synth.block_case("noalloc_ring_h1024_b1", 1024, False, [1000], ring_capacity=512, seed=0,
                              case_id=81)
    say(f"noalloc call 2: {second.name}")
    got, ref = _both(second)
    assert_parity(got, ref, "noalloc call 2 against the workspace block")


def test_noalloc_refuses_sequences_beyond_its_scratch():
    """300 long sequences need more than the 8 MiB scratch: refused with
    GQA_ERR_WORKSPACE_TOO_SMALL, nothing launched, out untouched."""
    a = gqa.Arch(hidden=1024)
    w = torch.zeros(a.qkv_rows * a.hidden, dtype=torch.int16, device="cuda")
    wg = torch.zeros(a.num_heads * a.hidden, dtype=torch.int16, device="cuda")
    wo = torch.zeros(a.hidden * a.q_dim, dtype=torch.int16, device="cuda")
    k = torch.zeros((16, a.num_kv_heads, a.head_dim), dtype=torch.float16, device="cuda")
    seqs = [gqa.KvSeq(k=k, v=k, position=15) for _ in range(300)]
    assert gqa.workspace_size(a, 300, 16) > 8 << 20
    x = torch.zeros((300, a.hidden), dtype=torch.float32, device="cuda")
    out = torch.full((300, a.hidden), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(gqa.GqaError) as e:
        gqa.attention_block_decode_noalloc(a, w, wg, wo, True, seqs, x, out)
    assert e.value.status == WS_SMALL and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
