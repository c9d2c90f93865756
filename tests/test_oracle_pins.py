"""The oracle against its pins, and planted mistakes against the pins.

``test_pin`` runs every pin on the real oracle.  ``test_planted_mistake_is_caught``
rebuilds the oracle from its own source with one plausible mistake planted
(a wrong sign, index, divisor, operand or missing term) and requires at least
one pin to fail on it, so the pins are shown to be able to see such mistakes.
"""
from __future__ import annotations

import os
import sys
import types

import pytest

import oracle
from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "block.py")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# (name, text in oracle/block.py, replacement)
MUTANTS = [
    ("rope_sign", "x[:, :half] = lo * c - hi * s", "x[:, :half] = lo * c + hi * s"),
    ("rope_divisor_is_head_dim", "-2.0 * i / rotary_dim", "-2.0 * i / x.shape[1]"),
    ("rope_width_swapped", "return int(full_rotary_dim), float(full_theta)",
     "return int(head_dim), float(full_theta)"),
    ("rope_theta_swapped", "return int(head_dim), float(sliding_theta)",
     "return int(head_dim), float(full_theta)"),
    ("rope_pairs_adjacent", "lo = x[:, :half].copy()\n    hi = x[:, half:rotary_dim].copy()",
     "lo = x[:, 0:rotary_dim:2].copy()\n    hi = x[:, 1:rotary_dim:2].copy()"),
    ("window_off_by_one", "kv_start = max(seq_len - sliding_window, 0)",
     "kv_start = max(seq_len - sliding_window + 1, 0)"),
    ("full_layer_windowed", "if is_full:\n        return seq_len, 0, 0",
     "if is_full:\n        return seq_len, max(seq_len - sliding_window, 0), 0"),
    ("ring_active_too_early", "seq_len > ring_capacity", "seq_len >= ring_capacity"),
    ("slot_shifted", "return position % ring_capacity if", "return (position + 1) % ring_capacity if"),
    ("gqa_modulo_map", "g = h // group", "g = h % num_kv"),
    ("softmax_unnormalised", "p /= p.sum()", "p = p"),
    ("scale_dropped", "s = scale * (kk @", "s = (kk @"),
    ("gate_sign", "return attn * sigmoid(gate_logits)[:, None]",
     "return attn * sigmoid(-gate_logits)[:, None]"),
    ("gate_dropped", 'res["gated"].append(head_gate(a, gl[b]).reshape(hq * d))',
     'res["gated"].append(a.reshape(hq * d))'),
    ("split_k_reads_v", "k = qkv_row[q_dim:q_dim + kv_dim]",
     "k = qkv_row[q_dim + kv_dim:q_dim + 2 * kv_dim]"),
    ("k_not_rotated", "k_r = rope_neox(k, pos, rotary_dim, theta)", "k_r = k.copy()"),
    ("q_not_rotated", "q_r = rope_neox(q, pos, rotary_dim, theta)", "q_r = q.copy()"),
    ("v_rotated", "k16, v16 = to_fp16(k_r), to_fp16(v)",
     "k16, v16 = to_fp16(k_r), to_fp16(rope_neox(v, pos, rotary_dim, theta))"),
    ("k_not_written", "kc[slot] = k16", "kc[slot] = kc[slot]"),
    ("rms_one_plus_w", "keepdims=True) + eps) * w", "keepdims=True) + eps) * (1.0 + w)"),
    ("rms_no_eps", "keepdims=True) + eps)", "keepdims=True))"),
    ("no_residual", "h = h + r.out", "h = r.out"),
    ("fp16_double_rounding", "return np.asarray(a, dtype=np.float64).astype(np.float16)",
     "return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float16)"),
    ("bf16_shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("gemv_transposed", "return x @ w.T", "return x @ w"),
    ("chunk_reuses_first_input", "x[t:t + 1], [cur], sinks)", "x[0:1], [cur], sinks)"),
    ("chunk_cache_not_threaded", "        k, v = r.k_caches[0], r.v_caches[0]\n        outs.append",
     "        outs.append"),
    ("chunk_positions_frozen", "position=int(seq.position) + t)", "position=int(seq.position))"),
    ("gelu_tanh_form", "0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))",
     "0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))"),
    ("gelu_on_up", "act = gelu_erf(gate) * up", "act = gelu_erf(up) * gate"),
    ("mlp_no_residual", "return MlpResult(h=h + out,", "return MlpResult(h=out,"),
    ("mlp_norm_skipped", "x = rms_norm(h, w_post_bits, eps)", "x = h"),
    ("mlp_reads_stream_before_attention_add", "m = mlp_decode(h_mid,", "m = mlp_decode(h,"),
    ("embedding_scaled", "return bf16_bits_to_f64(np.asarray(e_bits)[np.asarray(ids, dtype=np.int64)])",
     "return bf16_bits_to_f64(np.asarray(e_bits)[np.asarray(ids, dtype=np.int64)]) * np.sqrt(np.asarray(e_bits).shape[1])"),
    ("sink_ignored", "sig = float(sinks[h])", "sig = -np.inf"),
    ("sink_scaled_like_a_score", "sig = float(sinks[h])", "sig = scale * float(sinks[h])"),
    ("sink_base_2", "p = p / (p.sum() + np.exp(sig - ref))", "p = p / (p.sum() + np.exp2(sig - ref))"),
    ("sink_renormalised_away", "p = p / (p.sum() + np.exp(sig - ref))", "p = p / p.sum()"),
    ("block_drops_sinks", "st = attention_step(arch, is_full, qkv, gl, seqs, sinks)",
     "st = attention_step(arch, is_full, qkv, gl, seqs)"),
    ("head_without_final_norm", "x = rms_norm(h, w_final_bits, eps)\n    return gemv",
     "x = np.atleast_2d(np.asarray(h, dtype=np.float64))\n    return gemv"),
]


def _mutated_oracle(name, old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutant {name}: anchor not unique/absent"
    src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = ORACLE_SRC
    sys.modules[mod.__name__] = mod      # dataclasses look the module up
    try:
        exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    except Exception:
        sys.modules.pop(mod.__name__, None)
        raise
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutated_oracle(name, old, new)
    failed = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mod)
            except Exception:            # assertion or a crash both count
                failed.append(pin.__name__)
    finally:
        sys.modules.pop(mod.__name__, None)
    assert failed, f"no pin detects the planted mistake '{name}'"
