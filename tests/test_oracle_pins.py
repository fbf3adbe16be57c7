"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force in pure Python (math.exp / math.fsum) on tiny inputs,
* torch's scaled_dot_product_attention in float64 on the CPU with an explicit mask,
* invariants of softmax attention and closed forms,
* the values the pages print (tests/golden/printed_values.json),
* exact-arithmetic checks of the quantizer's IEEE fp32 decisions.

None of these tests needs a GPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth_inputs import rng_normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- brute force
def _score_op(x, kind, val, j):
    """One score-scope op on the raw score x of key j."""
    if kind == "mul":
        return x * val
    if kind == "add":
        return x + val
    if kind == "bias":
        return x + float(val[j])
    return x if x > 0 else 0.0


def brute_attention(q, k, v, causal, window, scale, group, ops=(), ks=None, vs=None, sops=()):
    """Pure-Python loops; exact sums via math.fsum.  Independent of numpy linear algebra.
    sops: score-scope ops, applied one key at a time to the raw dot product before the scale."""
    bh_q, s_q, d = len(q), len(q[0]), len(q[0][0])
    s_k = len(k[0])
    out = [[[0.0] * d for _ in range(s_q)] for _ in range(bh_q)]
    lse = [[0.0] * s_q for _ in range(bh_q)]
    for h in range(bh_q):
        g = h // group
        kk = [[float(k[g][j][c]) * (float(ks[g][j]) if ks is not None else 1.0) for c in range(d)]
              for j in range(s_k)]
        vv = [[float(v[g][j][c]) * (float(vs[g][j]) if vs is not None else 1.0) for c in range(d)]
              for j in range(s_k)]
        for i in range(s_q):
            ia = i + s_k - s_q
            keys = [j for j in range(s_k)
                    if (not causal or j <= ia) and (window == 0 or j > ia - window)]
            if not keys:
                out[h][i] = [0.0] * d
                lse[h][i] = -math.inf
                continue
            sc = {}
            for j in keys:
                x = math.fsum(float(q[h][i][c]) * kk[j][c] for c in range(d))
                for kind, val in sops:
                    x = _score_op(x, kind, val, j)
                sc[j] = scale * x
            m = max(sc.values())
            w = {j: math.exp(sc[j] - m) for j in keys}
            z = math.fsum(w.values())
            row = [math.fsum(w[j] * vv[j][c] for j in keys) / z for c in range(d)]
            for kind, val in ops:
                if kind == "mul":
                    row = [x * val for x in row]
                elif kind == "add":
                    row = [x + val for x in row]
                elif kind == "bias":
                    row = [x + float(val[c]) for c, x in enumerate(row)]
                else:
                    row = [x if x > 0 else 0.0 for x in row]
            out[h][i] = row
            lse[h][i] = m + math.log(z)
    return np.array(out), np.array(lse)


TINY = [
    # bh_q, bh_kv, s_q, s_k, d, causal, window
    (1, 1, 1, 1, 1, False, 0),
    (2, 2, 3, 5, 2, False, 0),
    (2, 2, 4, 4, 4, True, 0),
    (3, 1, 2, 6, 4, True, 0),       # GQA + ragged causal
    (4, 2, 5, 6, 2, True, 2),       # window
    (2, 1, 6, 6, 32, True, 3),
    (2, 2, 3, 6, 1, True, 1),
]


@pytest.mark.parametrize("case", TINY)
@pytest.mark.parametrize("seed", [11, 12, 13])
def test_oracle_matches_brute_force(case, seed):
    bh_q, bh_kv, s_q, s_k, d, causal, window = case
    q, k, v = rng_normal(seed, (bh_q, s_q, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    scale = 1.0 / math.sqrt(d)
    ops = [("mul", 2.0), ("add", 0.5)] if seed == 12 else []
    o_ref, l_ref = brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, window, scale,
                                   bh_q // bh_kv, ops)
    o, l = oracle.attention(q, k, v, causal=causal, window=window, epilogue=ops)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", [21, 22])
def test_oracle_int8_matches_brute_force(seed):
    bh_q, bh_kv, s_q, s_k, d = 4, 2, 3, 7, 4
    q, k, v = rng_normal(seed, (bh_q, s_q, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    g = np.random.default_rng(seed)
    kq = g.integers(-127, 128, size=(bh_kv, s_k, d)).astype(np.int8)
    vq = g.integers(-127, 128, size=(bh_kv, s_k, d)).astype(np.int8)
    ks = (np.abs(k[..., 0]) / 127).astype(np.float32)
    vs = (np.abs(v[..., 0]) / 127).astype(np.float32)
    o_ref, l_ref = brute_attention(q.tolist(), kq.tolist(), vq.tolist(), True, 0, 0.5,
                                   bh_q // bh_kv, (), ks.tolist(), vs.tolist())
    o, l = oracle.attention(q, kq, vq, causal=True, scale=0.5, k_scale=ks, v_scale=vs)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-13)


def test_empty_rows_give_zero_and_neg_inf_lse():
    # causal with s_q > s_k leaves the first s_q - s_k rows without a visible key
    q, k, v = rng_normal(5, (1, 5, 4), (1, 3, 4), (1, 3, 4))
    o, l = oracle.attention(q, k, v, causal=True)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), True, 0, 0.5, 1)
    assert np.all(o[0, :2] == 0) and np.all(np.isneginf(l[0, :2]))
    np.testing.assert_allclose(o, ob, atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("case", [
    (4, 4, 33, 127, 32, False, 0),
    (8, 2, 64, 64, 64, True, 0),
    (4, 1, 40, 100, 128, True, 0),
    (2, 2, 50, 90, 64, True, 17),
])
def test_oracle_matches_torch_sdpa_fp64(case):
    torch = pytest.importorskip("torch")
    bh_q, bh_kv, s_q, s_k, d, causal, window = case
    q, k, v = rng_normal(7, (bh_q, s_q, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    o, l = oracle.attention(q, k, v, causal=causal, window=window)
    G = bh_q // bh_kv
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(G, dim=0)
    qt = torch.from_numpy(q.astype(np.float64))
    # explicit boolean mask built here (bottom-right alignment), not torch's top-left is_causal
    i = torch.arange(s_q)[:, None] + (s_k - s_q)
    j = torch.arange(s_k)[None, :]
    m = torch.ones(s_q, s_k, dtype=torch.bool)
    if causal:
        m &= j <= i
    if window:
        m &= j > i - window
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    sc = torch.einsum("hid,hjd->hij", qt, kt) / math.sqrt(d)
    sc = sc.masked_fill(~m, -math.inf)
    np.testing.assert_allclose(l, torch.logsumexp(sc, dim=-1).numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- invariants
def test_softmax_rows_sum_to_one_and_nonnegative():
    # with V = identity the output rows are the softmax rows themselves
    s_q, s_k = 9, 13
    q, k = rng_normal(3, (2, s_q, 8), (2, s_k, 8))
    v = np.broadcast_to(np.eye(s_k), (2, s_k, s_k)).copy()
    qq = np.concatenate([q, np.zeros((2, s_q, s_k - 8))], axis=2)
    kk = np.concatenate([k, np.zeros((2, s_k, s_k - 8))], axis=2)
    for causal, window in [(False, 0), (True, 0), (True, 4)]:
        p, _ = oracle.attention(qq, kk, v, causal=causal, window=window, scale=0.3)
        assert np.all(p >= 0)
        np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
        vis = oracle.visible_mask(s_q, s_k, causal, window)
        assert np.all(p[:, ~vis] == 0)


def test_causal_rows_ignore_future_keys_bitwise():
    s = 24
    q, k, v = rng_normal(4, (3, s, 16), (3, s, 16), (3, s, 16))
    o1, l1 = oracle.attention(q, k, v, causal=True)
    k2, v2 = k.copy(), v.copy()
    cut = 10
    k2[:, cut + 1:] = rng_normal(99, k2[:, cut + 1:].shape)[0]
    v2[:, cut + 1:] = 1e3
    o2, l2 = oracle.attention(q, k2, v2, causal=True)
    assert np.array_equal(o1[:, :cut + 1], o2[:, :cut + 1])
    assert np.array_equal(l1[:, :cut + 1], l2[:, :cut + 1])
    assert not np.allclose(o1[:, cut + 1:], o2[:, cut + 1:])


def test_output_is_convex_combination_of_visible_values():
    s_q, s_k, d = 12, 20, 8
    q, k, v = rng_normal(6, (2, s_q, d), (2, s_k, d), (2, s_k, d))
    o, _ = oracle.attention(q, k, v, causal=True, window=5)
    vis = oracle.visible_mask(s_q, s_k, True, 5)
    for h in range(2):
        for i in range(s_q):
            vv = v[h][vis[i]]
            assert np.all(o[h, i] >= vv.min(0) - 1e-12) and np.all(o[h, i] <= vv.max(0) + 1e-12)


def test_noncausal_key_permutation_invariance():
    q, k, v = rng_normal(8, (2, 7, 16), (2, 31, 16), (2, 31, 16))
    perm = np.random.default_rng(0).permutation(31)
    o1, l1 = oracle.attention(q, k, v, causal=False)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-13, rtol=0)


def test_gqa_equals_mha_on_repeated_kv():
    G = 4
    q, k, v = rng_normal(9, (8, 10, 16), (2, 10, 16), (2, 10, 16))
    o1, _ = oracle.attention(q, k, v, causal=True)
    o2, _ = oracle.attention(q, np.repeat(k, G, 0), np.repeat(v, G, 0), causal=True)
    assert np.array_equal(o1, o2)
    # and a wrong head grouping (interleaved) would differ
    o3, _ = oracle.attention(q, np.tile(k, (G, 1, 1)), np.tile(v, (G, 1, 1)), causal=True)
    assert not np.allclose(o1, o3)


def test_window_at_least_sk_equals_causal():
    q, k, v = rng_normal(10, (2, 9, 8), (2, 15, 8), (2, 15, 8))
    oc, _ = oracle.attention(q, k, v, causal=True)
    for w in (15, 16, 100):
        ow, _ = oracle.attention(q, k, v, causal=True, window=w)
        assert np.array_equal(oc, ow)


def test_window_one_selects_the_diagonal_value():
    s_q, s_k = 6, 11
    q, k, v = rng_normal(12, (2, s_q, 8), (2, s_k, 8), (2, s_k, 8))
    o, l = oracle.attention(q, k, v, causal=True, window=1)
    for i in range(s_q):
        np.testing.assert_allclose(o[:, i], v[:, i + s_k - s_q], atol=1e-15, rtol=0)
        np.testing.assert_allclose(l[:, i], (q[:, i].astype(np.float64) * k[:, i + s_k - s_q]).sum(-1)
                                   / math.sqrt(8), atol=1e-12, rtol=0)


def test_single_key_returns_v0():
    q, k, v = rng_normal(13, (3, 4, 8), (3, 1, 8), (3, 1, 8))
    o, _ = oracle.attention(q, k, v, causal=False)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-15, rtol=0)


def test_zero_query_gives_mean_of_visible_values():
    s_q, s_k = 5, 9
    _, k, v = rng_normal(14, (1,), (2, s_k, 8), (2, s_k, 8))
    q = np.zeros((2, s_q, 8), np.float32)
    o, l = oracle.attention(q, k, v, causal=True, window=3)
    vis = oracle.visible_mask(s_q, s_k, True, 3)
    for i in range(s_q):
        np.testing.assert_allclose(o[:, i], v[:, vis[i]].astype(np.float64).mean(1), atol=1e-14, rtol=0)
        np.testing.assert_allclose(l[:, i], math.log(vis[i].sum()), atol=1e-14, rtol=0)


def test_two_keys_closed_form():
    # out = v0 + (v1 - v0) * sigmoid(s1 - s0)
    q, k, v = rng_normal(15, (1, 1, 4), (1, 2, 4), (1, 2, 4))
    o, _ = oracle.attention(q, k, v, causal=False, scale=0.7)
    s = [0.7 * sum(float(q[0, 0, c]) * float(k[0, j, c]) for c in range(4)) for j in range(2)]
    sig = 1.0 / (1.0 + math.exp(-(s[1] - s[0])))
    ref = v[0, 0].astype(np.float64) + (v[0, 1].astype(np.float64) - v[0, 0]) * sig
    np.testing.assert_allclose(o[0, 0], ref, atol=1e-14, rtol=0)


def test_decode_equals_last_row_of_causal_prefill():
    s = 40
    q, k, v = rng_normal(16, (4, s, 16), (2, s, 16), (2, s, 16))
    o, l = oracle.attention(q, k, v, causal=True)
    od, ld = oracle.decode(q[:, -1:], k, v)
    # equal up to BLAS blocking of a one-row vs a many-row product
    np.testing.assert_allclose(od[:, 0], o[:, -1], atol=1e-14, rtol=0)
    np.testing.assert_allclose(ld[:, 0], l[:, -1], atol=1e-14, rtol=0)
    ow, _ = oracle.attention(q, k, v, causal=True, window=7)
    odw, _ = oracle.decode(q[:, -1:], k, v, window=7)
    np.testing.assert_allclose(odw[:, 0], ow[:, -1], atol=1e-14, rtol=0)


def test_row_and_head_subsets_match_full_computation():
    q, k, v = rng_normal(17, (4, 300, 8), (2, 300, 8), (2, 300, 8))
    o, l = oracle.attention(q, k, v, causal=True)
    rows = [0, 7, 255, 256, 299]
    os_, ls_ = oracle.attention(q, k, v, causal=True, heads=[1, 3], rows=rows)
    np.testing.assert_allclose(os_[[1, 3]][:, rows], o[[1, 3]][:, rows], atol=1e-14, rtol=0)
    np.testing.assert_allclose(ls_[[1, 3]][:, rows], l[[1, 3]][:, rows], atol=1e-14, rtol=0)
    assert np.isnan(os_[0]).all()


def test_epilogue_order_and_values():
    x = np.array([[-1.0, 0.25, 3.0]])
    np.testing.assert_array_equal(oracle.apply_epilogue(x, [("mul", 2.0), ("add", 0.5)]), 2 * x + 0.5)
    np.testing.assert_array_equal(oracle.apply_epilogue(x, [("add", 0.5), ("mul", 2.0)]), 2 * x + 1.0)
    np.testing.assert_array_equal(oracle.apply_epilogue(x, []), x)
    with pytest.raises(ValueError):
        oracle.apply_epilogue(x, [("gelu", 0.0)])
    # per-channel bias and relu, worked by hand
    b = [10.0, -1.0, 0.5]
    np.testing.assert_array_equal(oracle.apply_epilogue(x, [("bias", b)]), [[9.0, -0.75, 3.5]])
    np.testing.assert_array_equal(oracle.apply_epilogue(x, [("relu", None)]), [[0.0, 0.25, 3.0]])
    np.testing.assert_array_equal(oracle.apply_epilogue(x, [("bias", b), ("relu", None), ("mul", -2.0)]),
                                  [[-18.0, 0.0, -7.0]])
    with pytest.raises(ValueError):
        oracle.apply_epilogue(x, [("bias", [1.0, 2.0])])


def test_window_without_causal_rejected():
    with pytest.raises(ValueError):
        oracle.visible_mask(3, 3, False, 2)


# ----------------------------------------------------------------------------- dequantize
def test_dequantize_is_exact_product():
    g = np.random.default_rng(1)
    qv = g.integers(-127, 128, size=(3, 5, 7)).astype(np.int8)
    s = g.random((3, 5)).astype(np.float32)
    dq = oracle.dequantize(qv, s)
    for idx in np.ndindex(qv.shape):
        exact = Fraction(int(qv[idx])) * Fraction(float(s[idx[:2]]))
        assert Fraction(float(dq[idx])) == exact


# ----------------------------------------------------------------------------- quantizer
def _nearest_f32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even), by exhaustive neighbourhood."""
    approx = np.float32(float(fr))
    cands = [np.nextafter(approx, np.float32(-np.inf)), approx, np.nextafter(approx, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                      int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_quantizer_hand_vector():
    hv = json.load(open(os.path.join(GOLDEN, "quantizer_hand_vector.json")))
    x = np.array(hv["x"], np.float32)[None]
    q, s = oracle.quantize_per_token(x)
    assert s[0] == np.float32(hv["scale"])
    assert q[0].tolist() == hv["codes"]


def test_quantizer_scale_and_codes_follow_ieee_fp32_decisions():
    x = rng_normal(31, (64, 48))[0] * np.float32(3.0)
    q, s = oracle.quantize_per_token(x)
    for r in range(x.shape[0]):
        a = max(abs(Fraction(float(t))) for t in x[r])
        s_ref = _nearest_f32(a / 127)
        assert s[r] == s_ref
        for c in range(0, x.shape[1], 5):
            quot = _nearest_f32(Fraction(float(x[r, c])) / Fraction(float(s_ref)))
            code = max(-127, min(127, round(Fraction(float(quot)))))   # round(): half to even
            assert int(q[r, c]) == code


def test_quantizer_bounds_and_extremes():
    x = rng_normal(32, (200, 128))[0]
    x[3] = 0.0
    x[4, :] = 1e-30
    x[5, 7] = -50.0
    q, s = oracle.quantize_per_token(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(int)) <= 127)
    assert s[3] == 0 and np.all(q[3] == 0)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))
    amax = np.argmax(np.abs(x), axis=1)
    nz = s > 0
    assert np.all(np.abs(q[np.arange(200), amax].astype(int))[nz] == 127)
    assert q[5, 7] == -127


def test_compression_ratio_matches_printed_value():
    gv = json.load(open(os.path.join(GOLDEN, "printed_values.json")))
    c = gv["compression_ratio_d64"]
    r = oracle.compression_ratio(c["head_dim"])
    assert round(r, c["digits"]) == c["printed"] and r > c["threshold"]
    assert abs(r - 64 * 4 / 68) < 1e-15
    big = oracle.compression_ratio(1 << 20)
    assert abs(big - gv["capacity_limit"]["printed"]) < 1e-4


def test_quantization_error_is_bounded_like_the_pages_claim():
    # fkl PR, Summary: int8 KV for a bounded error of order 1e-3 on the attention output
    w = 256
    q, k, v = rng_normal(33, (4, 1, 64), (4, w, 64), (4, w, 64))
    kq, ks = oracle.quantize_per_token(k)
    vq, vs = oracle.quantize_per_token(v)
    o_ref, _ = oracle.decode(q, k, v)
    o_q, _ = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
    err = np.abs(o_ref - o_q).max()
    assert 1e-4 < err < 1e-2


def test_append_kv_hand_placement():
    """Placement of new tokens at device-held positions, against a hand-worked fixture."""
    g = json.load(open(os.path.join(GOLDEN, "append_placement.json")))
    kn = np.array(g["k_new"], np.float32)
    bh, cap, d = kn.shape[0], g["capacity"], kn.shape[2]
    kc = np.full((bh, cap, d), g["cache_before_fill"], np.int8)
    ks = np.full((bh, cap), g["scale_before_fill"], np.float32)
    kc2, vc2, ks2, vs2 = oracle.append_kv(kc, kc, ks, ks, kn, -kn, np.array(g["pos"]))
    assert kc2.tolist() == g["expected_codes"]
    want_s = np.array(g["expected_scales_times_127"], np.float64) / 127
    assert np.all(np.abs(ks2.astype(np.float64) - want_s) <= 1e-7 * np.maximum(want_s, 1e-30))
    # V carries the negated tokens: codes negate, scales agree
    assert np.array_equal(vc2[ks2 != ks], -kc2[ks2 != ks]) and np.array_equal(vs2, ks2)
    # the inputs were not modified in place
    assert np.all(kc == g["cache_before_fill"])


def test_append_kv_token_by_token_equals_whole_sequence_quantization():
    """Writing a sequence one token per step, at advancing positions, gives exactly the codes and
    scales of quantizing the whole sequence at once (each token is quantized on its own)."""
    k, v = rng_normal(35, (3, 9, 32), (3, 9, 32))
    kc = np.zeros((3, 12, 32), np.int8)
    vc = np.zeros_like(kc)
    ks = np.zeros((3, 12), np.float32)
    vs = np.zeros_like(ks)
    start = np.array([0, 2, 3])
    for j in range(9):
        kc, vc, ks, vs = oracle.append_kv(kc, vc, ks, vs, k[:, j:j + 1], v[:, j:j + 1], start + j)
    kq, ksq = oracle.quantize_per_token(k)
    vq, vsq = oracle.quantize_per_token(v)
    for b in range(3):
        n = min(9, 12 - start[b])
        assert np.array_equal(kc[b, start[b]:start[b] + n], kq[b, :n])
        assert np.array_equal(vs[b, start[b]:start[b] + n], vsq[b, :n])
        assert np.all(kc[b, :start[b]] == 0) and np.all(ks[b, :start[b]] == 0)


def _key_chunks_causal(q, k, v, bounds):
    """Per-chunk oracle results of a causal prefill with query and key chunks aligned: the block
    (query chunk r, key chunk c) is full for c < r, causal for c == r, empty for c > r."""
    outs, lses = [], []
    for r, (r0, r1) in enumerate(bounds):
        oo, ll = [], []
        for c, (c0, c1) in enumerate(bounds):
            if c > r:
                oo.append(np.zeros((q.shape[0], r1 - r0, q.shape[2])))
                ll.append(np.full((q.shape[0], r1 - r0), -np.inf))
                continue
            o, l = oracle.attention(q[:, r0:r1], k[:, c0:c1], v[:, c0:c1], causal=(c == r),
                                    scale=1 / np.sqrt(q.shape[2]))
            oo.append(o)
            ll.append(l)
        outs.append(np.stack(oo))
        lses.append(np.stack(ll))
    return outs, lses


def test_merge_of_key_chunks_equals_attention_over_all_keys():
    """Exact attention is a mass-weighted mix of attention over any partition of its keys: the
    merge of per-chunk results equals the one-shot oracle (an identity of the softmax, checked
    here against the unsplit computation, causal with aligned query/key chunks, GQA)."""
    q, k, v = rng_normal(37, (4, 96, 32), (2, 96, 32), (2, 96, 32))
    bounds = [(0, 17), (17, 40), (40, 41), (41, 96)]
    full, lfull = oracle.attention(q, k, v, causal=True)
    outs, lses = _key_chunks_causal(q, k, v, bounds)
    for (r0, r1), o_p, l_p in zip(bounds, outs, lses):
        o, l = oracle.merge_lse(o_p, l_p)
        assert np.abs(o - full[:, r0:r1]).max() < 1e-12
        assert np.abs(l - lfull[:, r0:r1]).max() < 1e-12
    # non-causal, keys split in two: the same identity
    o1, l1 = oracle.attention(q, k[:, :50], v[:, :50], causal=False)
    o2, l2 = oracle.attention(q, k[:, 50:], v[:, 50:], causal=False)
    om, lm = oracle.merge_lse(np.stack([o1, o2]), np.stack([l1, l2]), epilogue=[("mul", 2.0), ("add", 0.5)])
    ref, lref = oracle.attention(q, k, v, causal=False, epilogue=[("mul", 2.0), ("add", 0.5)])
    assert np.abs(om - ref).max() < 1e-12 and np.abs(lm - lref).max() < 1e-12


def test_merge_special_cases():
    o = rng_normal(38, (3, 5, 8))[0].astype(np.float64)
    lse = np.array([[0.5, -np.inf, 2.0, 1.0, -np.inf],
                    [0.5, -np.inf, -np.inf, 1.0, 3.0],
                    [-np.inf, -np.inf, -np.inf, 1.0, -np.inf]])
    o[np.isneginf(lse)] = 0.0
    out, l = oracle.merge_lse(o, lse)
    # equal masses average; a lone part passes through; no part -> 0 and -inf
    assert np.allclose(out[0], (o[0, 0] + o[1, 0]) / 2, atol=1e-15) and np.isclose(l[0], 0.5 + np.log(2))
    assert np.isneginf(l[1]) and np.all(out[1] == 0)
    assert np.allclose(out[2], o[0, 2], atol=1e-15) and l[2] == 2.0
    assert np.allclose(out[3], o.mean(axis=0)[3], atol=1e-15) and np.isclose(l[3], 1.0 + np.log(3))
    assert np.allclose(out[4], o[1, 4], atol=1e-15) and l[4] == 3.0   # parts 0 and 2 empty


def test_bias_relu_chain_matches_brute_force():
    """A chain with a per-channel bias and a relu, through the whole attention, against the
    pure-Python loops (which apply the ops element by element)."""
    q, k, v = rng_normal(39, (3, 4, 8), (1, 6, 8), (1, 6, 8))
    bias = rng_normal(40, (8,))[0]
    ops = [("mul", 3.0), ("bias", bias.tolist()), ("relu", None), ("add", -0.25)]
    o_ref, _ = brute_attention(q.tolist(), k.tolist(), v.tolist(), True, 0, 1 / math.sqrt(8), 3, ops)
    o, _ = oracle.attention(q, k, v, causal=True, epilogue=ops)
    assert np.abs(o - o_ref).max() < 1e-13
    assert (o_ref == -0.25).any() and (o_ref > -0.25).any()     # the relu both clipped and passed


# ---- score-scope ops (kernbench2 commit page: tl.composite() ops with a k_tile scope run on each
# K tile right after its GEMM; here, on the raw scores q.k before the softmax scale)

SCORE_CHAINS = [
    [("mul", 0.5)],
    [("add", 1.25)],
    [("relu", None)],
    [("bias", "vec")],
    [("mul", 2.0), ("bias", "vec"), ("relu", None), ("add", -0.75)],
    [("relu", None), ("mul", -1.5)],
]


def _chain(chain, s_k, seed):
    vec = rng_normal(seed, (s_k,))[0] * 2.0
    return [(kd, vec.tolist() if vl == "vec" else vl) for kd, vl in chain]


@pytest.mark.parametrize("case", TINY[1:6])
@pytest.mark.parametrize("ci", range(len(SCORE_CHAINS)))
def test_score_ops_match_brute_force(case, ci):
    bh_q, bh_kv, s_q, s_k, d, causal, window = case
    q, k, v = rng_normal(60 + ci, (bh_q, s_q, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    sops = _chain(SCORE_CHAINS[ci], s_k, 70 + ci)
    out_ops = [("mul", 2.0)] if ci % 2 else []
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, window, scale,
                                   bh_q // bh_kv, out_ops, sops=sops)
    o, l = oracle.attention(q, k, v, causal=causal, window=window, epilogue=out_ops, score_epilogue=sops)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-13)


def test_score_ops_on_int8_keys_act_on_the_dequantized_score():
    bh_q, bh_kv, s_q, s_k, d = 4, 2, 3, 7, 4
    g = np.random.default_rng(77)
    q = rng_normal(77, (bh_q, s_q, d))[0]
    kq = g.integers(-127, 128, size=(bh_kv, s_k, d)).astype(np.int8)
    vq = g.integers(-127, 128, size=(bh_kv, s_k, d)).astype(np.int8)
    ks = g.uniform(0.001, 0.02, size=(bh_kv, s_k)).astype(np.float32)
    vs = g.uniform(0.001, 0.02, size=(bh_kv, s_k)).astype(np.float32)
    sops = _chain(SCORE_CHAINS[4], s_k, 78)
    o_ref, l_ref = brute_attention(q.tolist(), kq.tolist(), vq.tolist(), True, 0, 0.5, bh_q // bh_kv,
                                   (), ks.tolist(), vs.tolist(), sops=sops)
    o, l = oracle.attention(q, kq, vq, causal=True, scale=0.5, k_scale=ks, v_scale=vs, score_epilogue=sops)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-13)


def test_score_mul_is_a_softmax_temperature_and_add_shifts_only_the_lse():
    """Closed forms: sigma * (c x) is the softmax at scale sigma c; sigma (x + c) leaves every
    probability unchanged and raises the log-sum-exp by sigma c."""
    q, k, v = rng_normal(81, (4, 9, 16), (2, 13, 16), (2, 13, 16))
    sig = 0.3
    o1, l1 = oracle.attention(q, k, v, causal=True, window=5, scale=sig, score_epilogue=[("mul", 1.7)])
    o2, l2 = oracle.attention(q, k, v, causal=True, window=5, scale=sig * 1.7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    o3, l3 = oracle.attention(q, k, v, causal=True, window=5, scale=sig, score_epilogue=[("add", -2.5)])
    o4, l4 = oracle.attention(q, k, v, causal=True, window=5, scale=sig)
    np.testing.assert_allclose(o3, o4, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, l4 - 2.5 * sig, rtol=0, atol=1e-12)


def test_score_relu_over_negative_scores_averages_the_visible_values():
    """With every q.k < 0 a relu makes all scores 0: the output is the plain mean of the visible
    V rows and the log-sum-exp is log(number of visible keys)."""
    g = np.random.default_rng(83)
    q = g.uniform(0.1, 1.0, size=(2, 5, 8))
    k = -g.uniform(0.1, 1.0, size=(1, 7, 8))
    v = g.standard_normal((1, 7, 8))
    o, l = oracle.attention(q, k, v, causal=True, window=3, score_epilogue=[("relu", None)])
    for i in range(5):
        ia = i + 2
        keys = [j for j in range(7) if ia - 3 < j <= ia]
        for h in range(2):
            np.testing.assert_allclose(o[h, i], v[0, keys].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(l[h, i] - math.log(len(keys))) < 1e-14


def test_score_bias_of_minus_infinity_size_removes_keys():
    """A bias far below every score takes its keys out of the softmax exactly (exp underflows to
    0 in fp64): the result equals attention over the other keys alone."""
    q, k, v = rng_normal(85, (3, 4, 8), (3, 10, 8), (3, 10, 8))
    drop = np.array([0, 3, 4, 9])
    keep = np.setdiff1d(np.arange(10), drop)
    bias = np.zeros(10)
    bias[drop] = -1e6
    o1, l1 = oracle.attention(q, k, v, causal=False, score_epilogue=[("bias", bias)])
    o2, l2 = oracle.attention(q, k[:, keep], v[:, keep], causal=False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


# ---- rotate-half RoPE in the cache write (FlashRT QKV Cache RoPE: the decode K write)

def _angles(n_pos, d, base=10000.0):
    inv = base ** (-np.arange(0, d // 2, dtype=np.float64) * 2.0 / d)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_rope_hand_worked_fixture():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rope_rotate_half_hand.json")))
    out = oracle.rope_rotate_half(np.array(g["x"], np.float32), g["cos"], g["sin"])
    assert out.tolist() == g["out"]


def test_rope_identity_norms_and_relative_positions():
    rng = np.random.Generator(np.random.PCG64(41))
    d = 64
    cos, sin = _angles(300, d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    # position 0: cos 1, sin 0 leaves every value unchanged, bit for bit
    assert np.array_equal(oracle.rope_rotate_half(x, cos[0], sin[0]), x)
    # a rotation in each (i, i + d/2) plane keeps the norm (up to fp32 rounding)
    y = oracle.rope_rotate_half(x, cos[123], sin[123])
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-6)
    # <R_m q, R_n k> depends on m - n only
    q, k = x[0], x[1]
    a = float(np.dot(oracle.rope_rotate_half(q, cos[200], sin[200]), oracle.rope_rotate_half(k, cos[150], sin[150])))
    b = float(np.dot(oracle.rope_rotate_half(q, cos[50], sin[50]), oracle.rope_rotate_half(k, cos[0], sin[0])))
    assert abs(a - b) < 1e-4 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_append_with_rope_rotates_k_only_and_equals_quantizing_the_rotated_rows():
    rng = np.random.Generator(np.random.PCG64(42))
    bh, cap, d, n_new = 2, 10, 32, 3
    cos, sin = _angles(cap, d)
    k_new = rng.standard_normal((bh, n_new, d)).astype(np.float32)
    v_new = rng.standard_normal((bh, n_new, d)).astype(np.float32)
    z8, z = np.zeros((bh, cap, d), np.int8), np.zeros((bh, cap), np.float32)
    pos = np.array([4, 8])
    kc, vc, ks, vs = oracle.append_kv(z8, z8, z, z, k_new, v_new, pos, rope_cos=cos, rope_sin=sin)
    kc0, vc0, ks0, vs0 = oracle.append_kv(z8, z8, z, z, k_new, v_new, pos)
    assert np.array_equal(vc, vc0) and np.array_equal(vs, vs0)
    for b in range(bh):
        for j in range(n_new):
            p = pos[b] + j
            if p >= cap:
                continue                      # past the end: skipped (row 9 holds token 1 of head 1)
            q, s = oracle.quantize_per_token(oracle.rope_rotate_half(k_new[b, j], cos[p], sin[p]))
            assert np.array_equal(kc[b, p], q) and ks[b, p] == s
            assert not np.array_equal(kc[b, p], kc0[b, p])   # the rotation changed the codes
    assert not kc[1, :8].any() and not kc[0, 7:].any()
