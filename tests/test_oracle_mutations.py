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
