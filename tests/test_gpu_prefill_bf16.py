"""GPU parity of the bf16 forward (bf16 Q with bf16 K/V, or with the int8 cache) against the
fp64 oracle, plus invariants checked on the kernel's own outputs."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_BF16, TOL_E2E, check_bf16_output, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu


def _inputs(seed, bh_q, bh_kv, s_q, s_k, d):
    q, k, v = rng_normal(seed, (bh_q, s_q, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    return round_bf16(q), round_bf16(k), round_bf16(v)


def _bf16(q, k, v, **kw):
    import int8_compressed_kv_amd as fa
    return fa.flash_attention(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), **kw)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 100), (False, 0)])
def test_gqa_prefill_bf16_reduced_c5(causal, window):
    """The long-context GQA workload's structure (G = 8, d = 128) at 1024 tokens."""
    torch = torch_gpu()
    say(f"bf16 gqa causal={causal} window={window}")
    q, k, v = _inputs(51, 16, 2, 1024, 1024, 128)
    out, lse = _bf16(q, k, v, causal=causal, window=window, return_lse=True)
    ref, lref = oracle.attention(q, k, v, causal=causal, window=window)
    check_bf16_output(to_np(out), ref, "bf16 out")
    check_close(to_np(lse), lref, 1e-4, "lse")   # l is the fp32 sum of the fp32 exponentials
    o32 = _bf16(q, k, v, causal=causal, window=window, out_dtype=torch.float32)
    check_close(to_np(o32), ref, TOL_BF16, "fp32 output of the bf16 path")
    assert torch.equal(o32.to(torch.bfloat16), out), "bf16 store is not the RNE of the fp32 result"


@pytest.mark.parametrize("d", [32, 64, 96, 128, 160, 192, 224, 256])
def test_head_dims_ragged(d):
    torch = torch_gpu()
    say(f"bf16 d={d}")
    q, k, v = _inputs(300 + d, 4, 2, 300, 459, d)
    for causal, window in [(False, 0), (True, 0), (True, 37)]:
        out = _bf16(q, k, v, causal=causal, window=window, out_dtype=torch.float32)
        ref, _ = oracle.attention(q, k, v, causal=causal, window=window)
        check_close(to_np(out), ref, TOL_BF16, f"d={d} causal={causal} window={window}")


def test_tiny_and_single_key():
    torch = torch_gpu()
    q, k, v = _inputs(61, 2, 1, 3, 1, 64)
    out = _bf16(q, k, v, causal=False, out_dtype=torch.float32)
    check_close(to_np(out), np.broadcast_to(v[0, 0], (2, 3, 64)).astype(np.float64), 1e-6, "s_k = 1")
    q, k, v = _inputs(62, 1, 1, 1, 1, 32)
    out = _bf16(q, k, v, causal=True, out_dtype=torch.float32)
    check_close(to_np(out), v.astype(np.float64), 1e-6, "1x1")


def test_causal_rows_ignore_future_bitwise_and_determinism():
    torch = torch_gpu()
    q, k, v = _inputs(63, 8, 2, 700, 700, 128)
    o1 = _bf16(q, k, v, causal=True)
    o1b = _bf16(q, k, v, causal=True)
    assert torch.equal(o1, o1b), "run-to-run results differ"
    k2, v2 = k.copy(), v.copy()
    cut = 333
    k2[:, cut + 1:] = round_bf16(rng_normal(64, k2[:, cut + 1:].shape)[0])
    v2[:, cut + 1:] = 100.0
    o2 = _bf16(q, k2, v2, causal=True)
    assert torch.equal(o1[:, :cut + 1], o2[:, :cut + 1])


def test_gqa_equals_mha_on_repeated_kv_bitwise():
    torch = torch_gpu()
    q, k, v = _inputs(65, 8, 2, 300, 300, 64)
    o_gqa = _bf16(q, k, v, causal=True)
    o_mha = _bf16(q, np.repeat(k, 4, 0), np.repeat(v, 4, 0), causal=True)
    assert torch.equal(o_gqa, o_mha)


def test_epilogue_fused_equals_host_applied_bf16_path():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    q, k, v = _inputs(66, 4, 4, 200, 200, 128)
    o0 = _bf16(q, k, v, causal=True, out_dtype=torch.float32)
    name = fa.last_kernel()
    o1 = _bf16(q, k, v, causal=True, out_dtype=torch.float32, epilogue=[fa.Mul(2.0), fa.Add(0.5)])
    host = (o0.cpu() * 2.0) + 0.5
    assert torch.equal(o1.cpu(), host)
    assert fa.last_kernel() == name


# ----------------------------------------------------------------------------- int8 K/V, bf16 Q
def _int8(q, k, v, **kw):
    import int8_compressed_kv_amd as fa
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    out = fa.flash_attention(to_dev(q, "bf16"), kc, vc, k_scale=ks, v_scale=vs, **kw)
    return out, (to_np(kc).astype(np.int8), to_np(ks), to_np(vc).astype(np.int8), to_np(vs))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_int8_kv_bf16_reduced_c3(d):
    """int8-KV causal prefill (the compressed-cache workload's structure) at 2048 tokens:
    against the dequantized oracle (bf16 bar) and end to end on rows with >= 1024 keys."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"int8 bf16 d={d}")
    s = 2048 if d == 128 else 700
    q, k, v = rng_normal(70 + d, (4, s, d), (4, s, d), (4, s, d))
    q = round_bf16(q)
    out, (kq, ks, vq, vs) = _int8(q, k, v, causal=True)
    assert fa.last_kernel() == "prefill_bf16_i8kv"
    ref, _ = oracle.attention(q, kq, vq, causal=True, k_scale=ks, v_scale=vs)
    check_bf16_output(to_np(out), ref, "int8 vs dequantized")
    out32, _ = _int8(q, k, v, causal=True, out_dtype=torch.float32)
    check_close(to_np(out32), ref, TOL_BF16, "int8 fp32-out vs dequantized")
    if s >= 2048:
        e2e, _ = oracle.attention(q, k, v, causal=True, rows=range(1023, s))
        err = np.abs(to_np(out32)[:, 1023:] - e2e[:, 1023:])
        say(f"  end-to-end rows >= 1024 keys: max {err.max():.3e}")
        assert err.max() <= TOL_E2E


def test_int8_kv_window_and_ragged():
    torch = torch_gpu()
    q, k, v = rng_normal(77, (6, 190, 128), (3, 333, 128), (3, 333, 128))
    q = round_bf16(q)
    for causal, window in [(True, 50), (False, 0)]:
        out, (kq, ks, vq, vs) = _int8(q, k, v, causal=causal, window=window, out_dtype=torch.float32)
        ref, _ = oracle.attention(q, kq, vq, causal=causal, window=window, k_scale=ks, v_scale=vs)
        check_close(to_np(out), ref, TOL_BF16, f"int8 causal={causal} window={window}")


def test_int8_kv_small_and_large_value_scales():
    """fp16 range of P * v_s: values of very different magnitude per KV head."""
    torch = torch_gpu()
    q, k, v = rng_normal(78, (2, 128, 64), (2, 300, 64), (2, 300, 64))
    q = round_bf16(q)
    v[0] *= np.float32(1e-4)
    v[1] *= np.float32(3e4)
    out, (kq, ks, vq, vs) = _int8(q, k, v, causal=True, out_dtype=torch.float32)
    ref, _ = oracle.attention(q, kq, vq, causal=True, k_scale=ks, v_scale=vs)
    o = to_np(out)
    check_close(o[0] / 1e-4, ref[0] / 1e-4, TOL_BF16, "small V (relative)")
    check_close(o[1] / 3e4, ref[1] / 3e4, TOL_BF16, "large V (relative)")


@pytest.mark.parametrize("d", [64, 96, 128])
def test_int8_kv_query_and_key_magnitudes(d):
    """The int8 path computes Q K^T in fp16 with a power-of-two scale per query row and per block
    of key scales.  Key scales of 1e-4 and 3e4 (offset by the queries, so that the scores stay of
    unit size), rows of magnitude 1/2, 1 and 2, and the whole of Q multiplied by 2^20 or 2^-20
    with the softmax scale divided by the same power: all give the oracle's unscaled result."""
    import math
    torch = torch_gpu()
    say(f"int8 magnitudes d={d}")
    s = 333
    q, k, v = rng_normal(79 + d, (4, s, d), (2, s, d), (2, s, d))
    q = q * (np.float32(2.0) ** ((np.arange(s) % 3) - 1).astype(np.float32))[None, :, None]
    k[0] *= np.float32(1e-4)
    k[1] *= np.float32(3e4)
    q[:2] *= np.float32(1e4)      # query heads 0, 1 read KV head 0 (group of 2)
    q[2:] /= np.float32(3e4)      # query heads 2, 3 read KV head 1
    q = round_bf16(q)
    sigma = 1.0 / math.sqrt(d)
    for qf in (1.0, 2.0 ** 20, 2.0 ** -20):
        qq = (q * np.float32(qf)).astype(np.float32)   # exact: a power of two times bf16 values
        for causal in (True, False):
            out, (kq, ks, vq, vs) = _int8(qq, k, v, causal=causal, scale=sigma / qf, out_dtype=torch.float32)
            ref, _ = oracle.attention(q, kq, vq, causal=causal, k_scale=ks, v_scale=vs)
            check_close(to_np(out), ref, TOL_BF16, f"d={d} q x {qf:g} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_int8_kv_masked_keys_with_large_scales(d):
    """Keys that a block loads but masks (the window's lower edge) may have far larger scales than
    the visible ones: the block's fp16 normalisers cover every loaded key, so nothing overflows
    into the masked zeros of P (0 * inf), and the visible keys keep the oracle's result."""
    torch = torch_gpu()
    q, k, v = rng_normal(88 + d, (2, 600, d), (2, 600, d), (2, 600, d))
    q = round_bf16(q)
    v[:, 192:247] *= np.float32(1e5)   # loaded by the second block of 256 rows, visible to none of them
    k[:, 192:247] *= np.float32(1e3)
    out, (kq, ks, vq, vs) = _int8(q, k, v, causal=True, window=10, out_dtype=torch.float32)
    o = to_np(out)
    assert np.all(np.isfinite(o))
    ref, _ = oracle.attention(q, kq, vq, causal=True, window=10, k_scale=ks, v_scale=vs, rows=range(256, 600))
    check_close(o[:, 256:], ref[:, 256:], TOL_BF16, "rows of the second and third blocks")


@pytest.mark.parametrize("d", [64, 128])
def test_tile_and_pair_boundaries(d):
    """Key lengths around the 64-key tile and the two-tile copy / barrier grouping (odd and even
    tile counts, tails of 1 and 63 keys), causal and windowed, with s_q both equal to and below
    s_k (bottom-right alignment)."""
    torch = torch_gpu()
    say(f"bf16 tile/pair boundaries d={d}")
    cases = [(1, 1), (63, 63), (64, 64), (65, 65), (128, 128), (129, 129), (191, 191), (192, 192),
             (257, 257), (70, 200), (5, 321)]
    for i, (s_q, s_k) in enumerate(cases):
        q, k, v = _inputs(900 + 7 * d + i, 4, 2, s_q, s_k, d)
        for causal, window in [(True, 0), (False, 0), (True, 65), (True, 130)]:
            out = _bf16(q, k, v, causal=causal, window=window, out_dtype=torch.float32)
            ref, _ = oracle.attention(q, k, v, causal=causal, window=window)
            check_close(to_np(out), ref, TOL_BF16, f"s_q={s_q} s_k={s_k} causal={causal} window={window}")


@pytest.mark.parametrize("d", [64, 128])
def test_int8_kv_tile_and_pipeline_boundaries(d):
    """The int8 cache's staging pipeline (copies of tile t + 3 in flight, conversion one tile
    ahead) at 1 to 5 tiles, full and partial last tiles, causal, windowed and bottom-right aligned
    shapes, against the dequantized oracle."""
    torch = torch_gpu()
    say(f"int8 tile/pipeline boundaries d={d}")
    cases = [(1, 1), (63, 63), (64, 64), (65, 65), (128, 128), (129, 129), (191, 191), (192, 192),
             (257, 257), (70, 200), (5, 321)]
    for i, (s_q, s_k) in enumerate(cases):
        q, k, v = rng_normal(1900 + 7 * d + i, (4, s_q, d), (2, s_k, d), (2, s_k, d))
        q = round_bf16(q)
        for causal, window in [(True, 0), (False, 0), (True, 65)]:
            out, (kq, ks, vq, vs) = _int8(q, k, v, causal=causal, window=window, out_dtype=torch.float32)
            ref, _ = oracle.attention(q, kq, vq, causal=causal, window=window, k_scale=ks, v_scale=vs)
            check_close(to_np(out), ref, TOL_BF16, f"s_q={s_q} s_k={s_k} causal={causal} window={window}")
