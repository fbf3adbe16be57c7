"""Planted mistakes in the oracle (on the CPU only): each must be caught by a pin.

These tests monkeypatch a plausible error into the oracle and check that the
corresponding independent check (brute force, torch SDPA, closed form) sees a
difference.  They show the pins are sharp enough, not just self-consistent.
"""
import math

import numpy as np
import pytest

import oracle
import importlib

oatt = importlib.import_module("oracle.attention")
from synth_inputs import rng_normal
from test_oracle_pins import brute_attention


def _ragged_case():
    return rng_normal(41, (4, 5, 8), (2, 9, 8), (2, 9, 8))


def _differs_from_brute(causal=True, window=0, ops=()):
    q, k, v = _ragged_case()
    o_ref, _ = brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, window, 1 / math.sqrt(8), 2, ops)
    o, _ = oracle.attention(q, k, v, causal=causal, window=window, epilogue=ops)
    return not np.allclose(o, o_ref, atol=1e-13, rtol=0)


def test_top_left_causal_alignment_is_caught(monkeypatch):
    def top_left(s_q, s_k, causal, window=0):
        i = np.arange(s_q)[:, None]
        j = np.arange(s_k)[None, :]
        vis = np.ones((s_q, s_k), bool)
        if causal:
            vis &= j <= i
        if window:
            vis &= j > i - window
        return vis
    assert not _differs_from_brute()
    monkeypatch.setattr(oatt, "visible_mask", top_left)
    assert _differs_from_brute()


def test_window_off_by_one_is_caught(monkeypatch):
    orig = oatt.visible_mask

    def wider(s_q, s_k, causal, window=0):
        return orig(s_q, s_k, causal, window + 1 if window else 0)
    assert not _differs_from_brute(window=3)
    monkeypatch.setattr(oatt, "visible_mask", wider)
    assert _differs_from_brute(window=3)


def test_interleaved_gqa_mapping_is_caught(monkeypatch):
    q, k, v = _ragged_case()
    o_ref, _ = brute_attention(q.tolist(), k.tolist(), v.tolist(), True, 0, 1 / math.sqrt(8), 2)
    # plant: query head h uses KV head h % bh_kv instead of h // G
    o_bad, _ = oracle.attention(q[[0, 2, 1, 3]], k, v, causal=True)
    o_bad = o_bad[[0, 2, 1, 3]]
    assert not np.allclose(o_bad, o_ref, atol=1e-13)


def test_epilogue_order_swap_is_caught(monkeypatch):
    orig = oatt.apply_epilogue
    ops = [("mul", 2.0), ("add", 0.5)]
    assert not _differs_from_brute(ops=ops)
    monkeypatch.setattr(oatt, "apply_epilogue", lambda x, o: orig(x, list(o)[::-1]))
    assert _differs_from_brute(ops=ops)


def test_missing_scale_in_dequantize_is_caught(monkeypatch):
    q, k, v = _ragged_case()
    kq, ks = oracle.quantize_per_token(k)
    vq, vs = oracle.quantize_per_token(v)
    o_ref, _ = brute_attention(q.tolist(), kq.tolist(), vq.tolist(), True, 0, 1 / math.sqrt(8), 2,
                               (), ks.tolist(), vs.tolist())
    monkeypatch.setattr(oatt, "dequantize", lambda a, s: a.astype(np.float64))
    o, _ = oracle.attention(q, kq, vq, causal=True, k_scale=ks, v_scale=vs)
    assert not np.allclose(o, o_ref, atol=1e-13)


def _quantizer_variant(rounding, divisor=127.0):
    def q(x):
        x = np.asarray(x, np.float32)
        a = np.max(np.abs(x), axis=-1)
        s = (a / np.float32(divisor)).astype(np.float32)
        safe = np.where(s > 0, s, np.float32(1))
        r = np.clip(rounding(x / safe[..., None]), -127, 127)
        return np.where((s > 0)[..., None], r, 0).astype(np.int8), s
    return q


def test_half_up_rounding_is_caught(monkeypatch):
    from test_oracle_pins import test_quantizer_hand_vector as pin
    pin()
    monkeypatch.setattr(oracle, "quantize_per_token", _quantizer_variant(lambda t: np.floor(t + 0.5)))
    with pytest.raises(AssertionError):
        pin()


def test_wrong_scale_divisor_is_caught(monkeypatch):
    from test_oracle_pins import test_quantizer_scale_and_codes_follow_ieee_fp32_decisions as pin
    pin()
    monkeypatch.setattr(oracle, "quantize_per_token", _quantizer_variant(np.rint, 128.0))
    with pytest.raises(AssertionError):
        pin()


def test_truncating_quantizer_is_caught(monkeypatch):
    from test_oracle_pins import test_quantizer_bounds_and_extremes as pin
    from test_oracle_pins import test_quantizer_scale_and_codes_follow_ieee_fp32_decisions as pin2
    monkeypatch.setattr(oracle, "quantize_per_token", _quantizer_variant(np.trunc))
    with pytest.raises(AssertionError):
        pin2()


def test_append_position_off_by_one_is_caught(monkeypatch):
    from test_oracle_pins import test_append_kv_hand_placement as pin
    pin()
    oq = importlib.import_module("oracle.quantize")
    orig = oq.append_kv
    monkeypatch.setattr(oracle, "append_kv",
                        lambda kc, vc, ks, vs, kn, vn, pos: orig(kc, vc, ks, vs, kn, vn, np.asarray(pos) + 1))
    with pytest.raises(AssertionError):
        pin()


def test_append_writing_past_the_cache_end_is_caught(monkeypatch):
    """A cache write that wraps a row past the end around to row 0 instead of skipping it."""
    from test_oracle_pins import test_append_kv_hand_placement as pin
    oq = importlib.import_module("oracle.quantize")

    def wrapping(kc, vc, ks, vs, kn, vn, pos):
        kc, vc, ks, vs = (np.array(a, copy=True) for a in (kc, vc, ks, vs))
        cap = kc.shape[1]
        for b in range(kn.shape[0]):
            for j in range(kn.shape[1]):
                p = (int(pos[b]) + j) % cap
                for new, codes, scales in ((kn, kc, ks), (vn, vc, vs)):
                    codes[b, p], scales[b, p] = oq.quantize_per_token(new[b, j])
        return kc, vc, ks, vs
    monkeypatch.setattr(oracle, "append_kv", wrapping)
    with pytest.raises(AssertionError):
        pin()


def test_merge_without_mass_weights_is_caught(monkeypatch):
    """Averaging the chunk outputs (ignoring each chunk's share of the softmax mass)."""
    from test_oracle_pins import test_merge_of_key_chunks_equals_attention_over_all_keys as pin
    pin()
    orig = oatt.merge_lse

    def plain_mean(o_parts, lse_parts, epilogue=()):
        o, l = orig(o_parts, lse_parts, epilogue)
        live = ~np.isneginf(np.asarray(lse_parts))
        mean = (np.asarray(o_parts) * live[..., None]).sum(0) / np.maximum(live.sum(0), 1)[..., None]
        return oatt.apply_epilogue(mean, epilogue), l
    monkeypatch.setattr(oracle, "merge_lse", plain_mean)
    with pytest.raises(AssertionError):
        pin()


def test_merge_with_max_instead_of_logsumexp_is_caught(monkeypatch):
    from test_oracle_pins import test_merge_special_cases as pin
    orig = oatt.merge_lse

    def max_lse(o_parts, lse_parts, epilogue=()):
        o, _ = orig(o_parts, lse_parts, epilogue)
        return o, np.asarray(lse_parts, np.float64).max(axis=0)
    monkeypatch.setattr(oracle, "merge_lse", max_lse)
    with pytest.raises(AssertionError):
        pin()


def test_relu_as_abs_or_bias_reversed_is_caught(monkeypatch):
    from test_oracle_pins import test_bias_relu_chain_matches_brute_force as pin
    pin()
    orig = oatt.apply_epilogue

    monkeypatch.setattr(oatt, "apply_epilogue", lambda x, ops: _abs_variant(orig, x, ops))
    with pytest.raises(AssertionError):
        pin()
    monkeypatch.setattr(oatt, "apply_epilogue",
                        lambda x, ops: orig(x, [(k, v[::-1]) if k == "bias" else (k, v) for k, v in ops]))
    with pytest.raises(AssertionError):
        pin()


def test_score_ops_after_the_softmax_scale_are_caught(monkeypatch):
    """Plant: the score-scope ops act on sigma x instead of x (the oracle then multiplies by sigma
    again, so the planted form equals f(sigma x))."""
    from test_oracle_pins import test_score_ops_match_brute_force as pin
    from test_oracle_pins import TINY
    case = TINY[3]
    sig = 1.0 / math.sqrt(case[4])
    pin(case, 4)
    orig = oatt.apply_epilogue

    def after_scale(x, ops):
        if ops and np.ndim(x) == 2 and x.shape[-1] == case[3] and any(kd == "add" for kd, _ in ops):
            return orig(np.asarray(x) * sig, ops) / sig
        return orig(x, ops)
    monkeypatch.setattr(oatt, "apply_epilogue", after_scale)
    with pytest.raises(AssertionError):
        pin(case, 4)


def test_score_bias_reversed_is_caught(monkeypatch):
    from test_oracle_pins import test_score_ops_match_brute_force as pin
    from test_oracle_pins import TINY
    pin(TINY[2], 3)
    orig = oatt.apply_epilogue
    monkeypatch.setattr(oatt, "apply_epilogue",
                        lambda x, ops: orig(x, [(k, v[::-1]) if k == "bias" else (k, v) for k, v in ops]))
    with pytest.raises(AssertionError):
        pin(TINY[2], 3)


def _abs_variant(orig, x, ops):
    """The epilogue with relu planted as abs."""
    y = np.array(x, dtype=np.float64)
    for k, v in ops:
        y = np.abs(y) if k == "relu" else orig(y, [(k, v)])
    return y


def test_rope_with_the_sine_sign_flipped_is_caught_by_the_hand_fixture():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_rotate_half_hand.json")))
    x = np.array(g["x"], np.float32)
    wrong = oracle.rope_rotate_half(x, g["cos"], [-v for v in g["sin"]])   # rotation the other way
    assert wrong.tolist() != g["out"]
    swapped = oracle.rope_rotate_half(x[[2, 3, 0, 1]], g["cos"], g["sin"])[[2, 3, 0, 1]]   # halves swapped
    assert swapped.tolist() != g["out"]
