"""GPU parity of fa_compress_kv against the oracle quantizer: codes and scales bit for bit."""
import numpy as np
import pytest

import oracle
from gpu_util import say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu

DIMS = [32, 64, 96, 128, 160, 192, 224, 256]


def _edge_rows(d):
    rows = [np.zeros(d, np.float32)]                                  # all-zero token
    r = np.zeros(d, np.float32); r[d // 2] = -3.0; rows.append(r)      # single nonzero
    r = np.full(d, 0.5, np.float32); r[0] = 127.0; rows.append(r)     # s = 1: ties at .5
    r = np.arange(d, dtype=np.float32) - d / 2 + 0.5; r[1] = 127.0; rows.append(r)
    r = np.full(d, 1e-30, np.float32); rows.append(r)                  # tiny values
    r = np.linspace(-1e4, 1e4, d).astype(np.float32); rows.append(r)   # large values
    return np.stack(rows)


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_compress_bit_exact(d, dt):
    import int8_compressed_kv_amd as fa
    torch_gpu()
    say(f"compress d={d} dtype={dt}")
    x = rng_normal(100 + d, (2, 517, d))[0] * np.float32(2.0)
    x[0, :6] = _edge_rows(d)
    if dt == "bf16":
        x = round_bf16(x)
    codes, scales = fa.compress_kv(to_dev(x, dt))
    q_ref, s_ref = oracle.quantize_per_token(x)
    c, s = to_np(codes), to_np(scales)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    assert np.array_equal(c, q_ref), f"{int((c != q_ref).sum())} codes differ"
    assert fa.last_kernel().startswith("compress")


def test_compress_empty_and_single_token():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    x = torch.zeros(0, 64, device="cuda")
    c, s = fa.compress_kv(x)
    assert c.shape == (0, 64) and s.shape == (0,)
    x1 = rng_normal(5, (1, 128))[0]
    c, s = fa.compress_kv(to_dev(x1, "f32"))
    q_ref, s_ref = oracle.quantize_per_token(x1)
    assert np.array_equal(to_np(c), q_ref) and np.array_equal(to_np(s), s_ref)


def test_compress_ratio_of_the_stored_cache():
    """Bytes of the compressed cache (codes + scales) against fp32, at d = 64 (3.76x)."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    x = torch.randn(4, 256, 64, device="cuda")
    c, s = fa.compress_kv(x)
    ratio = (x.numel() * 4) / (c.numel() * c.element_size() + s.numel() * s.element_size())
    assert abs(ratio - oracle.compression_ratio(64)) < 1e-12 and round(ratio, 2) == 3.76


def _tie_rows(seed, n_rows, d):
    """Rows whose quotients x / s sit on and one ulp either side of half-integers, where the
    rounding of the quotient decides the code.  Built from the scale the quantizer will compute
    (s = fp32(a / 127) for the row's absmax a), so the cases are exact, not statistical."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = np.empty((n_rows, d), np.float32)
    for i in range(n_rows):
        # absmax across many binades, including scales below 2^-64 and near the fp32 limits
        e = int(g.integers(-100, 100)) if i % 8 else int(g.integers(-140, -80))
        a = np.float32(np.ldexp(1.0 + g.random(), e))
        s = np.float32(a) / np.float32(127)
        k = g.integers(-126, 126, size=d).astype(np.float64)
        x = ((k + 0.5) * np.float64(s)).astype(np.float32)
        sel = g.integers(0, 4, size=d)
        x = np.where(sel == 1, np.nextafter(x, np.float32(np.inf)), x)
        x = np.where(sel == 2, np.nextafter(x, np.float32(-np.inf)), x)
        x = np.where(sel == 3, (k * np.float64(s)).astype(np.float32), x)
        x = np.clip(x, -a, a)
        x[int(g.integers(0, d))] = a if g.random() < 0.5 else -a
        rows[i] = x
    return rows


@pytest.mark.parametrize("d", [32, 128, 256])
def test_compress_bit_exact_at_rounding_ties(d):
    import int8_compressed_kv_amd as fa
    torch_gpu()
    say(f"compress ties d={d}")
    x = _tie_rows(700 + d, 4096, d)
    q_ref, s_ref = oracle.quantize_per_token(x)
    codes, scales = fa.compress_kv(to_dev(x, "f32"))
    c, s = to_np(codes), to_np(scales)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    bad = int((c != q_ref).sum())
    assert bad == 0, f"{bad} codes differ"
    # the rows exercise the tie cases: many quotients are exact half-integers
    qf = x.astype(np.float64) / s_ref.astype(np.float64)[:, None]
    assert np.sum(np.abs(qf - np.round(qf)) == 0.5) > 1000
