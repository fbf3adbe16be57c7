"""GPU checks of the richer epilogue (per-channel Bias and ReLU beside Mul and Add) on every
kernel family: the fused chain equals the same fp32 ops applied on the host to the kernel's own
plain output, bit for bit; it matches the oracle; and it never changes the kernel instantiation."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_BF16, TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu


def _chain(fa, torch, d, seed):
    bias = rng_normal(seed, (d,))[0]
    dev = torch.from_numpy(bias).cuda()
    ops = [fa.Mul(1.5), fa.Bias(dev), fa.ReLU(), fa.Add(-0.125)]
    ref_ops = [("mul", 1.5), ("bias", bias), ("relu", None), ("add", -0.125)]

    def host(o):   # the same fp32 ops, one rounding each, on the device
        y = o.float() * 1.5
        y = y + dev
        y = torch.where(y > 0, y, torch.zeros_like(y))
        return y + (-0.125)
    return ops, ref_ops, host


@pytest.mark.parametrize("d", [64, 128, 96, 256])
def test_bias_relu_chain_bf16_and_int8_prefill(d):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"epilogue chain prefill d={d}")
    q, k, v = rng_normal(900 + d, (4, 130, d), (2, 200, d), (2, 200, d))
    qb, kb, vb = round_bf16(q), round_bf16(k), round_bf16(v)
    ops, ref_ops, host = _chain(fa, torch, d, 950 + d)
    args = (to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"))
    o0 = fa.flash_attention(*args, causal=True, out_dtype=torch.float32)
    name = fa.last_kernel()
    o1 = fa.flash_attention(*args, causal=True, out_dtype=torch.float32, epilogue=ops)
    assert fa.last_kernel() == name
    assert torch.equal(o1, host(o0)), "bf16 path: fused chain differs from host-applied"
    ref, _ = oracle.attention(qb, kb, vb, causal=True, epilogue=ref_ops)
    check_close(to_np(o1), ref, TOL_BF16, "bf16 path vs oracle")
    # int8 cache
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    i0 = fa.flash_attention(args[0], kc, vc, k_scale=ks, v_scale=vs, causal=True, out_dtype=torch.float32)
    i1 = fa.flash_attention(args[0], kc, vc, k_scale=ks, v_scale=vs, causal=True, out_dtype=torch.float32,
                            epilogue=ops)
    assert torch.equal(i1, host(i0)), "int8 path: fused chain differs from host-applied"


def test_bias_relu_chain_fp32_prefill_and_decode():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    d = 64
    q, k, v = rng_normal(960, (8, 33, d), (2, 127, d), (2, 127, d))
    ops, ref_ops, host = _chain(fa, torch, d, 961)
    o0 = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=False)
    o1 = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=False, epilogue=ops)
    assert torch.equal(o1, host(o0)), "fp32 path: fused chain differs from host-applied"
    ref, _ = oracle.attention(q, k, v, causal=False, epilogue=ref_ops)
    check_close(to_np(o1), ref, TOL_F32, "fp32 path vs oracle")
    # decode: the merge kernel applies the chain (d = 96 has lanes past the head dim)
    for dd in (128, 96):
        say(f"epilogue chain decode d={dd}")
        q1, k1, v1 = rng_normal(962 + dd, (8, 1, dd), (2, 3000, dd), (2, 3000, dd))
        q1 = round_bf16(q1)
        kc, ks = fa.compress_kv(to_dev(k1, "f32"))
        vc, vs = fa.compress_kv(to_dev(v1, "f32"))
        ops, ref_ops, host = _chain(fa, torch, dd, 963 + dd)
        d0 = fa.decode(to_dev(q1, "bf16"), kc, vc, ks, vs, num_splits=5)
        d1 = fa.decode(to_dev(q1, "bf16"), kc, vc, ks, vs, num_splits=5, epilogue=ops)
        assert torch.equal(d1, host(d0)), "decode: fused chain differs from host-applied"
        kq, ksn = to_np(kc).astype(np.int8), to_np(ks)
        vq, vsn = to_np(vc).astype(np.int8), to_np(vs)
        ref, _ = oracle.decode(q1, kq, vq, k_scale=ksn, v_scale=vsn, epilogue=ref_ops)
        check_close(to_np(d1), ref, TOL_F32, f"decode d={dd} vs oracle")


def test_bias_relu_chain_merge():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    d = 128
    o = rng_normal(970, (3, 500, d))[0]
    lse = rng_normal(971, (3, 500))[0] * 3
    ops, ref_ops, host = _chain(fa, torch, d, 972)
    m0 = fa.merge_lse(to_dev(o, "f32"), to_dev(lse, "f32"))
    m1 = fa.merge_lse(to_dev(o, "f32"), to_dev(lse, "f32"), epilogue=ops)
    assert torch.equal(m1, host(m0)), "merge: fused chain differs from host-applied"
    ref, _ = oracle.merge_lse(o, lse, epilogue=ref_ops)
    check_close(to_np(m1), ref, TOL_F32, "merge vs oracle")
