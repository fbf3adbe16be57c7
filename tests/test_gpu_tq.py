"""GPU parity of the TurboQuant codec (2, 3 and 4 bits) against the oracle: codes equal except where the exact
rotated coordinate lies on a decision threshold (there either neighbouring code is correct),
norms and decoded vectors to fp32 rounding, and attention over a K4/V2 and a K4/V4 cache with the
quality the page quotes."""
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import random_signs, rng_normal, round_bf16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _encode(x, xdt, bits, signs):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    cb = fa.tq_codebook(x.shape[-1], bits)
    sd = torch.from_numpy(signs).cuda()
    codes, norms = fa.tq_encode(to_dev(x, xdt), sd, bits, cb)
    return codes, norms, sd, cb


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_encode_matches_oracle_up_to_threshold_ties(d, bits, xdt):
    torch_gpu()
    n = 3000
    say(f"tq encode d={d} bits={bits} {xdt}")
    x = rng_normal(1000 + d + bits, (n, d))[0] * np.float32(2.0)
    x[5] = 0.0
    if xdt == "bf16":
        x = round_bf16(x)
    s = random_signs(1100 + d, d)
    codes, norms, _, _ = _encode(x, xdt, bits, s)
    got = oracle.tq_unpack(to_np(codes), bits, d)
    want, want_n = oracle.tq_encode(x, s, bits)
    # the exact rotated, normalised coordinates and their distance to the nearest threshold
    c, t = oracle.beta_codebook(d, bits)
    y = (x.astype(np.float64) * s) @ oracle.hadamard(d).T
    u = y / np.maximum(np.linalg.norm(y, axis=-1, keepdims=True), 1e-300)
    gap = np.min(np.abs(u[..., None] - t), axis=-1)
    diff = got != want
    diff[5] = False                  # the all-zero vector decodes to 0 whatever its codes
    say(f"  codes differing: {int(diff.sum())} of {diff.size}, nearest-threshold gap there "
        f"{float(gap[diff].max()) if diff.any() else 0.0:.2e}")
    assert np.all(np.abs(got.astype(int) - want.astype(int))[diff] == 1)
    assert np.all(gap[diff] < 2e-6)
    assert diff.sum() <= 1e-4 * diff.size + 2
    check_close(to_np(norms) / np.maximum(want_n, 1e-30), np.where(want_n > 0, 1.0, 0.0), 2e-6,
                "norms (relative)")


@pytest.mark.parametrize("which", ["close", "tiny"])
def test_encode_with_codebooks_outside_the_decision_table(which):
    """4-bit encode decides through a table of float-bit buckets when the codebook fits it and by a
    search otherwise; antisymmetric codebooks with two thresholds in one bucket ("close") or a
    threshold below 2^-7 ("tiny") take the search and still match the oracle's codes."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    d = 128
    pos = {"close": [0.01, 0.03, 0.05, 0.0504, 0.0508, 0.1, 0.2, 0.3],
           "tiny": [0.001, 0.003, 0.01, 0.03, 0.06, 0.1, 0.2, 0.3]}[which]
    cb = np.array([-x for x in pos[::-1]] + pos, np.float32)
    x = rng_normal(1500, (3000, d))[0]
    s = random_signs(1501, d)
    codes, norms = fa.tq_encode(to_dev(x, "f32"), torch.from_numpy(s).cuda(), 4, cb)
    assert fa.last_kernel() == "tq_encode_search"
    got = oracle.tq_unpack(to_np(codes), 4, d)
    t = (np.float32(0.5) * (cb[1:] + cb[:-1])).astype(np.float64)   # the fp32 midpoints the library uses
    want, _ = oracle.tq_encode(x, s, 4, codebook=(cb.astype(np.float64), t))
    y = (x.astype(np.float64) * s) @ oracle.hadamard(d).T
    u = y / np.linalg.norm(y, axis=-1, keepdims=True)
    gap = np.min(np.abs(u[..., None] - t), axis=-1)
    diff = got != want
    say(f"  {which}: codes differing {int(diff.sum())} of {diff.size}")
    assert np.all(gap[diff] < 2e-6)
    assert diff.sum() <= 1e-4 * diff.size + 2
    # the Beta codebook takes the table
    fa.tq_encode(to_dev(x, "f32"), torch.from_numpy(s).cuda(), 4, fa.tq_codebook(d, 4))
    assert fa.last_kernel() == "tq_encode"


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 4), (256, 4), (32, 2), (32, 3), (64, 3), (128, 3), (256, 3)])
def test_decode_matches_oracle_on_the_same_codes(d, bits):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"tq decode d={d} bits={bits}")
    x = rng_normal(1200 + d, (2000, d))[0]
    x[0] = 0.0
    s = random_signs(1300 + d, d)
    codes, norms, sd, cb = _encode(x, "f32", bits, s)
    out = fa.tq_decode(codes, norms, sd, bits, cb)
    outb = fa.tq_decode(codes, norms, sd, bits, cb, out_dtype=torch.bfloat16)
    ref = oracle.tq_decode(oracle.tq_unpack(to_np(codes), bits, d), to_np(norms), s, bits)
    scale = np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-30)
    check_close(to_np(out) / scale, ref / scale, 2e-6, "decoded (relative to the norm)")
    assert np.all(to_np(out)[0] == 0)
    assert torch.equal(outb, out.to(torch.bfloat16))


@pytest.mark.parametrize("k_bits,v_bits", [(4, 2), (4, 4)])
def test_attention_over_a_turboquant_cache(k_bits, v_bits):
    """Decode attention over K/V stored as TurboQuant codes (decoded to fp32 by the codec, then
    attended by the fp32 kernel), against the oracle on the same codes, and its quality against
    unquantized attention (the page: cosine about 0.94 for K4/V2, 0.99 for K4/V4)."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    d, s_k, heads = 128, 512, 8
    q, k, v = rng_normal(61, (heads, 1, d), (heads, s_k, d), (heads, s_k, d))
    sk, sv = random_signs(62, d), random_signs(63, d)
    kc, kn, skd, kcb = _encode(k, "f32", k_bits, sk)
    vc, vn, svd, vcb = _encode(v, "f32", v_bits, sv)
    kh = fa.tq_decode(kc, kn, skd, k_bits, kcb)
    vh = fa.tq_decode(vc, vn, svd, v_bits, vcb)
    out = fa.flash_attention(to_dev(q, "f32"), kh, vh, causal=False)
    kref = oracle.tq_decode(oracle.tq_unpack(to_np(kc), k_bits, d), to_np(kn), sk, k_bits)
    vref = oracle.tq_decode(oracle.tq_unpack(to_np(vc), v_bits, d), to_np(vn), sv, v_bits)
    ref, _ = oracle.attention(q, kref, vref, causal=False)
    check_close(to_np(out), ref, TOL_F32, f"K{k_bits}/V{v_bits} attention vs oracle")
    full, _ = oracle.attention(q, k, v, causal=False)
    o = to_np(out)[:, 0]
    cos = float(np.mean(np.sum(o * full[:, 0], -1) / (np.linalg.norm(o, axis=-1) * np.linalg.norm(full[:, 0], axis=-1))))
    gv = json.load(open(os.path.join(GOLDEN, "printed_values.json")))["turboquant_cosine"]
    say(f"  K{k_bits}/V{v_bits} attention-output cosine vs unquantized: {cos:.4f}")
    if v_bits == 2:
        assert abs(cos - gv["k4v2_synthetic"]) < 0.03
    else:
        assert cos > gv["k4v4"] - 0.01
