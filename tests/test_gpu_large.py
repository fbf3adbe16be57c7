"""Maximum-size GPU cases: tensors past 2^31 elements, so every offset into them needs 64 bits.
Inputs are drawn on the device (seeded torch generators) and checked on sampled rows / heads
against the oracle: the compress of 2^24 + 3 tokens (bit-exact), the decode over an int8 cache of
more than 2^31 bytes per matrix, and bf16 and int8 prefills whose K/V hold more than 2^31
elements."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_BF16, TOL_F32, check_bf16_output, check_close, say, to_np, torch_gpu

pytestmark = pytest.mark.gpu


def _gen(torch, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def test_compress_past_2_31_elements():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    n, d = (1 << 24) + 3, 128
    say(f"compress {n} x {d} fp32 ({n * d} elements)")
    x = torch.randn((n, d), generator=_gen(torch, 1), device="cuda", dtype=torch.float32)
    codes, scales = fa.compress_kv(x)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(2))
    rows = np.unique(np.concatenate([[0, 1, n // 2, n - 3, n - 2, n - 1], g.integers(0, n, 200)]))
    idx = torch.from_numpy(rows).cuda()
    xs = to_np(x[idx])
    q, s = oracle.quantize_per_token(xs)
    assert np.array_equal(to_np(codes[idx]).astype(np.int8), q)
    assert np.array_equal(to_np(scales[idx]), s)


def _int8_cache(torch, bh_kv, s_k, d, seed):
    g = _gen(torch, seed)
    kc = torch.randint(-127, 128, (bh_kv, s_k, d), generator=g, device="cuda", dtype=torch.int8)
    vc = torch.randint(-127, 128, (bh_kv, s_k, d), generator=g, device="cuda", dtype=torch.int8)
    ks = torch.rand((bh_kv, s_k), generator=g, device="cuda") * 0.02 + 1e-3
    vs = torch.rand((bh_kv, s_k), generator=g, device="cuda") * 0.02 + 1e-3
    return kc, vc, ks, vs


def test_decode_over_a_cache_past_2_31_bytes():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh_kv, group, s_k, d = 8, 4, (1 << 21) + 77, 128
    say(f"decode over {bh_kv} x {s_k} x {d} int8 ({bh_kv * s_k * d} bytes per matrix)")
    kc, vc, ks, vs = _int8_cache(torch, bh_kv, s_k, d, 3)
    q = torch.randn((bh_kv * group, 1, d), generator=_gen(torch, 4), device="cuda").to(torch.bfloat16)
    out = fa.decode(q, kc, vc, ks, vs)
    for kvh in (bh_kv - 1, 0):
        sl = slice(kvh * group, (kvh + 1) * group)
        ref, _ = oracle.decode(to_np(q[sl]), to_np(kc[kvh:kvh + 1]).astype(np.int8),
                               to_np(vc[kvh:kvh + 1]).astype(np.int8), k_scale=to_np(ks[kvh:kvh + 1]),
                               v_scale=to_np(vs[kvh:kvh + 1]))
        check_close(to_np(out[sl]), ref, TOL_F32, f"KV head {kvh}")
    # the int8 prefill kernel over the same cache: a block of queries at the end of the sequence
    qp = torch.randn((bh_kv * group, 64, d), generator=_gen(torch, 5), device="cuda").to(torch.bfloat16)
    o8 = fa.flash_attention(qp, kc, vc, k_scale=ks, v_scale=vs, causal=True, out_dtype=torch.float32)
    kvh = bh_kv - 1
    h = kvh * group + group - 1
    rows = [0, 31, 63]
    ref, _ = oracle.attention(to_np(qp[h:h + 1]), to_np(kc[kvh:kvh + 1]).astype(np.int8),
                              to_np(vc[kvh:kvh + 1]).astype(np.int8), causal=True,
                              k_scale=to_np(ks[kvh:kvh + 1]), v_scale=to_np(vs[kvh:kvh + 1]), rows=rows)
    check_close(to_np(o8[h:h + 1])[:, rows], ref[:, rows], TOL_BF16, "int8 prefill, last query head")


def test_bf16_prefill_with_kv_past_2_31_elements():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh_kv, group, s_q, s_k, d = 8, 2, 64, (1 << 21) + 100, 128
    say(f"bf16 prefill, K/V {bh_kv} x {s_k} x {d} ({bh_kv * s_k * d} elements each)")
    g = _gen(torch, 6)
    k = torch.randn((bh_kv, s_k, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((bh_kv, s_k, d), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((bh_kv * group, s_q, d), generator=g, device="cuda").to(torch.bfloat16)
    out = fa.flash_attention(q, k, v, causal=True, out_dtype=torch.bfloat16)
    kvh = bh_kv - 1
    rows = [0, 40, 63]
    for h in (kvh * group, kvh * group + 1):
        ref, _ = oracle.attention(to_np(q[h:h + 1]), to_np(k[kvh:kvh + 1]), to_np(v[kvh:kvh + 1]),
                                  causal=True, rows=rows)
        check_bf16_output(to_np(out[h:h + 1])[:, rows], ref[:, rows], f"query head {h}")
