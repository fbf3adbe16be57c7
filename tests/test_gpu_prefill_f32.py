"""GPU parity of the fp32 forward (fp32 Q with fp32 or int8 K/V) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import WORKLOADS, draw_qkv, rng_normal

pytestmark = pytest.mark.gpu


def _run(q, k, v, **kw):
    import int8_compressed_kv_amd as fa
    out, lse = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), return_lse=True, **kw)
    return to_np(out), to_np(lse)


def test_c1_causal_fp32():
    w = WORKLOADS["c1"]
    say(f"c1 {w.name}")
    q, k, v = draw_qkv(w)
    out, lse = _run(q, k, v, causal=True)
    ref, lref = oracle.attention(q, k, v, causal=True)
    check_close(out, ref, TOL_F32, "c1 out")
    check_close(lse, lref, TOL_F32, "c1 lse")


def test_c2_ragged_fp32_with_epilogue():
    import int8_compressed_kv_amd as fa
    w = WORKLOADS["c2"]
    say(f"c2 {w.name}")
    q, k, v = draw_qkv(w)
    out0, _ = _run(q, k, v, causal=False)
    ref0, _ = oracle.attention(q, k, v, causal=False)
    check_close(out0, ref0, TOL_F32, "c2 plain")
    k_plain = fa.last_kernel()
    ops = [fa.Mul(2.0), fa.Add(0.5)]
    out1, _ = _run(q, k, v, causal=False, epilogue=ops)
    ref1, _ = oracle.attention(q, k, v, causal=False, epilogue=[("mul", 2.0), ("add", 0.5)])
    check_close(out1, ref1, TOL_F32, "c2 epilogue")
    # fused == host-applied, bit for bit: the same fp32 ops applied to the kernel's own output
    host = (out0.astype(np.float32) * np.float32(2.0)).astype(np.float32) + np.float32(0.5)
    assert np.array_equal(out1.view(np.uint32), host.astype(np.float32).view(np.uint32))
    # values and chain length are kernel arguments: the same instantiation runs
    assert fa.last_kernel() == k_plain
    _run(q, k, v, causal=False, epilogue=[fa.Mul(-3.25), fa.Add(1e-3), fa.Mul(0.5)])
    assert fa.last_kernel() == k_plain


@pytest.mark.parametrize("d", [32, 64, 96, 128, 160, 192, 224, 256])
def test_head_dims_gqa_window_ragged(d):
    say(f"f32 d={d}")
    q, k, v = rng_normal(200 + d, (6, 45, d), (2, 77, d), (2, 77, d))
    for causal, window in [(False, 0), (True, 0), (True, 9)]:
        out, lse = _run(q, k, v, causal=causal, window=window)
        ref, lref = oracle.attention(q, k, v, causal=causal, window=window)
        check_close(out, ref, TOL_F32, f"d={d} causal={causal} window={window}")
        check_close(lse, lref, TOL_F32, "lse")


def test_empty_rows_and_empty_keys():
    torch = torch_gpu()
    import int8_compressed_kv_amd as fa
    q, k, v = rng_normal(7, (2, 40, 64), (2, 25, 64), (2, 25, 64))
    out, lse = _run(q, k, v, causal=True)   # rows 0..14 see no key
    ref, lref = oracle.attention(q, k, v, causal=True)
    assert np.all(out[:, :15] == 0) and np.all(np.isneginf(lse[:, :15]))
    check_close(out, ref, TOL_F32, "empty-row causal")
    o0 = fa.flash_attention(to_dev(q, "f32"), torch.zeros(2, 0, 64, device="cuda"),
                            torch.zeros(2, 0, 64, device="cuda"))
    assert torch.count_nonzero(o0).item() == 0


@pytest.mark.parametrize("case", ["c1", "c2"])
def test_int8_kv_fp32_parity_mode(case):
    """int8 K/V compressed on the GPU, attention in fp32: within 1e-5 of the oracle fed the
    dequantized cache (the page's int8-KV exact check)."""
    import int8_compressed_kv_amd as fa
    w = WORKLOADS[case]
    say(f"int8 fp32 mode {case}")
    q, k, v = draw_qkv(w)
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    kq, ksr = oracle.quantize_per_token(k)
    vq, vsr = oracle.quantize_per_token(v)
    assert np.array_equal(to_np(kc), kq) and np.array_equal(to_np(vs), vsr)
    out, lse = fa.flash_attention(to_dev(q, "f32"), kc, vc, k_scale=ks, v_scale=vs, causal=w.causal,
                                  return_lse=True)
    ref, lref = oracle.attention(q, kq, vq, causal=w.causal, k_scale=ksr, v_scale=vsr)
    check_close(to_np(out), ref, TOL_F32, f"{case} int8 vs dequantized")
    check_close(to_np(lse), lref, TOL_F32, f"{case} int8 lse")
    assert fa.last_kernel() == "prefill_f32_i8kv"
    e2e, _ = oracle.attention(q, k, v, causal=w.causal)
    say(f"  {case} int8 end-to-end max err {np.abs(to_np(out) - e2e).max():.3e} (context only at this length)")


def test_bf16_output_is_rounded_fp32_output():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    q, k, v = rng_normal(9, (4, 70, 64), (4, 70, 64), (4, 70, 64))
    o32 = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=True)
    o16 = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=True,
                             out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
