"""Helpers for the GPU tests: device copies of synthetic cases, the parity bar,
and the fp16-ulp comparison of cache rows.

The parity bar on floating point is the one the block is built to: relative
L2 error <= 1e-3 and max abs error <= 5e-3 * max|ref| against the fp64 oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import gqa_attention_block_amd as gqa
import synth

REL_L2_TOL = 1e-3
MAX_ABS_FRAC = 5e-3


def say(msg: str):
    """Name the case before a GPU step, so a failing run says which one."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def arch_of(case_arch: synth.Arch) -> gqa.Arch:
    return gqa.Arch(hidden=case_arch.hidden, num_heads=case_arch.num_heads,
                    num_kv_heads=case_arch.num_kv_heads, head_dim=case_arch.head_dim,
                    full_rotary_dim=case_arch.full_rotary_dim,
                    sliding_window=case_arch.sliding_window,
                    full_rope_theta=case_arch.full_rope_theta, rope_theta=case_arch.rope_theta,
                    attention_scale=case_arch.attention_scale, rms_eps=case_arch.rms_eps)


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def f32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def f16_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def assert_parity(got, ref, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    lim = MAX_ABS_FRAC * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert r <= REL_L2_TOL, f"{what}: rel-L2 {r:.3e} > {REL_L2_TOL}"
    assert m <= lim, f"{what}: max-abs {m:.3e} > {lim:.3e}"
    return r, m


def assert_fp16_within_one_ulp(got16: np.ndarray, ref16: np.ndarray, what: str,
                               row_scale: float = 0.0):
    """Both fp16: equal or one rounding apart.  A value produced by
    cancellation (k_i cos - k_j sin near 0) may differ by more, up to the fp32
    evaluation error of its inputs: 2^-18 * row_scale (the row's max |value|)
    on top of one ulp."""
    g = np.asarray(got16, np.float16)
    r = np.asarray(ref16, np.float16)
    assert g.shape == r.shape, what
    gi = g.view(np.int16).astype(np.int32)
    ri = r.view(np.int16).astype(np.int32)
    # map sign-magnitude bit patterns to an ordered integer line
    go = np.where(gi < 0, -(gi & 0x7FFF), gi)
    ro = np.where(ri < 0, -(ri & 0x7FFF), ri)
    d = np.abs(go - ro)
    far = d > 1
    if far.any():
        ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
        diff = np.abs(g.astype(np.float64) - r.astype(np.float64))
        ok = diff <= ulp + 2.0 ** -18 * row_scale
        assert np.all(ok | ~far), (f"{what}: {int((far & ~ok).sum())} values beyond one ulp "
                                   f"+ 2^-18*{row_scale:.3g}")
    assert far.sum() <= max(2, 0.01 * far.size), f"{what}: {int(far.sum())} values more than 1 ulp apart"


class DevBlock:
    """Device copies of a synthetic single-layer case (caches cloned fresh)."""

    def __init__(self, case: synth.BlockCase):
        self.case = case
        self.arch = arch_of(case.arch)
        self.w_qkv = bits_to_dev(case.w_qkv)
        self.w_g = bits_to_dev(case.w_g)
        self.w_o = bits_to_dev(case.w_o)
        self.x = f32_to_dev(case.x)
        self.k = [f16_to_dev(s.k) for s in case.seqs]
        self.v = [f16_to_dev(s.v) for s in case.seqs]
        max_len = max(s.position + 1 for s in case.seqs)
        self.ws = torch.empty(gqa.workspace_size(self.arch, len(case.seqs), max_len),
                              dtype=torch.uint8, device="cuda")

    def seqs(self):
        return [gqa.KvSeq(k=self.k[i], v=self.v[i], position=s.position,
                          ring_capacity=s.ring_capacity)
                for i, s in enumerate(self.case.seqs)]

    def run_block(self, sinks=None) -> np.ndarray:
        out = torch.empty((self.case.batch, self.arch.hidden), dtype=torch.float32, device="cuda")
        gqa.attention_block_decode(self.arch, self.w_qkv, self.w_g, self.w_o, self.case.is_full,
                                   self.seqs(), self.x, out, self.ws,
                                   sinks=None if sinks is None else f32_to_dev(sinks))
        torch.cuda.synchronize()
        return out.cpu().numpy()


def check_caches(case: synth.BlockCase, k_dev, v_dev, k16_ref, v16_ref, slots, what: str,
                 exact_v: bool = False):
    """Only the slot row changes; it holds this token's k (within one fp16
    ulp of the oracle's) and v (likewise, or bitwise when exact_v)."""
    for i, s in enumerate(case.seqs):
        kg = k_dev[i].cpu().numpy()
        vg = v_dev[i].cpu().numpy()
        slot = slots[i]
        mask = np.ones(s.capacity, bool)
        mask[slot] = False
        assert np.array_equal(kg[mask].view(np.int16), s.k[mask].view(np.int16)), \
            f"{what}[{i}]: K rows other than slot {slot} changed"
        assert np.array_equal(vg[mask].view(np.int16), s.v[mask].view(np.int16)), \
            f"{what}[{i}]: V rows other than slot {slot} changed"
        kscale = float(np.max(np.abs(np.asarray(k16_ref[i], np.float64))))
        assert_fp16_within_one_ulp(kg[slot], k16_ref[i], f"{what}[{i}] K slot row", kscale)
        if exact_v:
            assert np.array_equal(vg[slot].view(np.int16), np.asarray(v16_ref[i]).view(np.int16)), \
                f"{what}[{i}] V slot row not bitwise equal"
        else:
            vscale = float(np.max(np.abs(np.asarray(v16_ref[i], np.float64))))
            assert_fp16_within_one_ulp(vg[slot], v16_ref[i], f"{what}[{i}] V slot row", vscale)
