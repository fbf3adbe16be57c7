"""Pins of the TurboQuant codec oracle (CPU): the Hadamard matrix against scipy's, the Lloyd-Max
codebook against its optimality conditions evaluated by an independent quadrature, a hand-worked
encode/decode of a basis vector, packing round trips, the printed K4/V2 size ratio, and the
quality magnitudes the page quotes."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, linalg, stats

import oracle
from synth_inputs import random_signs, rng_normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_is_sylvester_and_orthogonal(d):
    h = oracle.hadamard(d)
    assert np.array_equal(h, linalg.hadamard(d))
    assert np.array_equal(h @ h.T, d * np.eye(d))
    with pytest.raises(ValueError):
        oracle.hadamard(96)


@pytest.mark.parametrize("d,bits", [(64, 2), (64, 4), (128, 2), (128, 4), (32, 3)])
def test_codebook_satisfies_lloyd_max_conditions_by_quadrature(d, bits):
    c, t = oracle.beta_codebook(d, bits)
    a = d / 2
    pdf = lambda u: 0.5 * stats.beta.pdf((u + 1) / 2, a, a)   # noqa: E731
    edges = np.concatenate([[-1.0], t, [1.0]])
    assert len(c) == 1 << bits and np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], atol=1e-14)                            # symmetric law, symmetric codebook
    assert np.allclose(t, (c[:-1] + c[1:]) / 2, atol=0)                    # nearest-neighbour cells
    for k in range(len(c)):                                                # each centroid is its cell's mean
        m0 = integrate.quad(pdf, edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda u: u * pdf(u), edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9 * max(1.0, abs(c[k]))


def test_codebook_distortion_falls_with_bits_like_the_gaussian_limit():
    d = 128
    a = d / 2
    pdf = lambda u: 0.5 * stats.beta.pdf((u + 1) / 2, a, a)   # noqa: E731
    mse = []
    for bits in (1, 2, 3, 4):
        c, t = oracle.beta_codebook(d, bits)
        e = np.concatenate([[-1.0], t, [1.0]])
        mse.append(sum(integrate.quad(lambda u, ck=ck: (u - ck) ** 2 * pdf(u), e[k], e[k + 1])[0]
                       for k, ck in enumerate(c)))
    var = 1.0 / (d + 1)                        # variance of 2B - 1 for B ~ Beta(d/2, d/2)
    rel = np.array(mse) / var
    # the Gaussian Lloyd-Max relative distortions are 0.3634, 0.1175, 0.03454, 0.009497
    assert np.allclose(rel, [0.3634, 0.1175, 0.03454, 0.009497], rtol=0.02)
    assert np.all(np.diff(mse) < 0)


def test_basis_vector_encodes_to_one_repeated_code_by_hand():
    """x = 3 e_j: the rotation spreads it to s_j/sqrt(d) * (+-1 pattern of column j of H); every
    coordinate has magnitude 1/sqrt(d), so every code is the cell of +-1/sqrt(d), and the decode
    returns 3 * c_k * sqrt(d) on e_j with zeros elsewhere."""
    d, bits, j = 64, 4, 5
    s = random_signs(7, d)
    x = np.zeros(d)
    x[j] = 3.0
    codes, n = oracle.tq_encode(x, s, bits)
    c, t = oracle.beta_codebook(d, bits)
    col = oracle.hadamard(d)[:, j] * s[j]
    k_pos = np.searchsorted(t, 1 / math.sqrt(d), side="right")
    k_neg = np.searchsorted(t, -1 / math.sqrt(d), side="right")
    assert n == np.float32(3.0)
    assert np.array_equal(codes, np.where(col > 0, k_pos, k_neg))
    xr = oracle.tq_decode(codes, n, s, bits)
    want = np.zeros(d)
    want[j] = 3.0 * c[k_pos] * math.sqrt(d)     # c[k_neg] = -c[k_pos]
    assert np.allclose(xr, want, atol=1e-12)


def test_zero_vector_and_packing_round_trip():
    d = 128
    s = random_signs(8, d)
    for bits in (2, 3, 4):
        codes, n = oracle.tq_encode(np.zeros((3, d)), s, bits)
        assert np.all(n == 0) and np.all(oracle.tq_decode(codes, n, s, bits) == 0)
        g = np.random.Generator(np.random.PCG64(bits))
        cc = g.integers(0, 1 << bits, (5, d)).astype(np.uint8)
        pk = oracle.tq_pack(cc, bits)
        assert pk.shape == (5, d * bits // 8)
        assert np.array_equal(oracle.tq_unpack(pk, bits, d), cc)
    # bit layout by hand: codes 1, 2, 3, 0 at 2 bits -> 0b00111001; 0xA, 0x5 at 4 bits -> 0x5A
    assert oracle.tq_pack(np.array([[1, 2, 3, 0]], np.uint8), 2)[0, 0] == 0b00111001
    assert oracle.tq_pack(np.array([[0xA, 0x5]], np.uint8), 4)[0, 0] == 0x5A


def test_three_bit_packing_against_a_hand_packed_stream():
    """3-bit codes straddle bytes: the packed stream of a hand-worked example, and the same rule
    checked bit by bit against a plain loop over the stream positions."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tq_pack3_hand.json")))
    pk = oracle.tq_pack(np.array([g["codes"]], np.uint8), g["bits"])
    assert pk[0].tolist() == g["bytes"]
    assert oracle.tq_unpack(pk, 3, 8)[0].tolist() == g["codes"]
    rng = np.random.Generator(np.random.PCG64(33))
    cc = rng.integers(0, 8, (4, 64)).astype(np.uint8)
    pk = oracle.tq_pack(cc, 3)
    for r in range(4):
        for i in range(64):
            got = 0
            for b in range(3):
                k = 3 * i + b
                got |= ((int(pk[r, k // 8]) >> (k % 8)) & 1) << b
            assert got == cc[r, i]


def test_k4v2_size_ratio_matches_printed_value():
    gv = json.load(open(os.path.join(GOLDEN, "printed_values.json")))["turboquant_k4v2_ratio"]
    r = oracle.tq_compression_ratio(64, gv["k_bits"], gv["v_bits"])
    assert round(r, gv["digits"]) == gv["printed"]
    assert abs(r - 512 / 56) < 1e-12


def test_attention_quality_magnitudes_like_the_page():
    """Attention-output cosine against unquantized attention on synthetic N(0,1) K/V: the page
    quotes about 0.94 for K4/V2 and 0.99 for K4/V4 without shapes or data (magnitudes only)."""
    gv = json.load(open(os.path.join(GOLDEN, "printed_values.json")))["turboquant_cosine"]
    d, s_k, heads = 128, 512, 8
    q, k, v = rng_normal(61, (heads, 1, d), (heads, s_k, d), (heads, s_k, d))
    sk, sv = random_signs(62, d), random_signs(63, d)
    ref, _ = oracle.decode(q, k, v)

    def cos(kb, vb):
        kc, kn = oracle.tq_encode(k, sk, kb)
        vc, vn = oracle.tq_encode(v, sv, vb)
        out, _ = oracle.decode(q, oracle.tq_decode(kc, kn, sk, kb), oracle.tq_decode(vc, vn, sv, vb))
        num = np.sum(out * ref, axis=-1)
        return float(np.mean(num / (np.linalg.norm(out, axis=-1) * np.linalg.norm(ref, axis=-1))))
    c42, c44 = cos(4, 2), cos(4, 4)
    assert abs(c42 - gv["k4v2_synthetic"]) < 0.03, c42
    assert c44 > gv["k4v4"] - 0.01 and c44 > c42, c44


def test_attention_over_codes_by_brute_force():
    """Decode attention over TurboQuant codes, pinned by pure-Python loops that rebuild every key
    and value from its codes by the page's steps (centroid times norm, Hadamard entries
    (-1)^popcount(i & j), signs, 1/sqrt(d)) and take the softmax with math.exp / math.fsum."""
    import math
    d, s_k, G = 8, 5, 2
    rng = np.random.Generator(np.random.PCG64(77))
    q = rng.standard_normal((2 * G, 1, d))
    k = rng.standard_normal((2, s_k, d))
    v = rng.standard_normal((2, s_k, d)) + 0.5
    sk = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    sv = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    for kb, vb in ((4, 2), (3, 4)):
        kc, kn = oracle.tq_encode(k, sk, kb)
        vc, vn = oracle.tq_encode(v, sv, vb)
        ccb_k, _ = oracle.beta_codebook(d, kb)
        ccb_v, _ = oracle.beta_codebook(d, vb)
        out, lse = oracle.tq_attention_decode(q, oracle.tq_pack(kc, kb), kn, sk, kb, oracle.tq_pack(vc, vb), vn,
                                              sv, vb, window=4)

        def rebuild(codes, norm, signs, cb):
            y = [float(norm) * float(cb[c]) for c in codes]
            return [signs[i] * math.fsum((-1) ** bin(i & j).count("1") * y[j] for j in range(d)) / math.sqrt(d)
                    for i in range(d)]
        for h in range(2 * G):
            b = h // G
            keys = range(s_k - 4, s_k)                     # window 4 keeps the last four keys
            kk = {j: rebuild(kc[b, j], kn[b, j], sk, ccb_k) for j in keys}
            vv = {j: rebuild(vc[b, j], vn[b, j], sv, ccb_v) for j in keys}
            sc = {j: math.fsum(q[h, 0, i] * kk[j][i] for i in range(d)) / math.sqrt(d) for j in keys}
            m = max(sc.values())
            w = {j: math.exp(sc[j] - m) for j in keys}
            tot = math.fsum(w.values())
            for i in range(d):
                ref = math.fsum(w[j] * vv[j][i] for j in keys) / tot
                assert abs(out[h, 0, i] - ref) < 1e-12
            assert abs(lse[h, 0] - (m + math.log(tot))) < 1e-12
