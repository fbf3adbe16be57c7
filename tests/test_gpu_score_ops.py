"""GPU parity of the score-scope (K-tile) ops: Mul, Add, Bias by key position and ReLU applied to
every raw score q.k before the mask and the softmax scale, on every kernel family that forms
scores (fp32 and int8-KV fp32 prefill, bf16 prefill, bf16 prefill over the int8 cache, int8
decode with 4 and 8 heads per workgroup, the no-allocation decode, attention over TurboQuant
codes), against the oracle with the same ops, over ragged shapes, GQA, causal and window masks."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_BF16, TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import random_signs, rng_normal, round_bf16

pytestmark = pytest.mark.gpu

CHAINS = {
    "temperature": [("mul", 0.5)],
    "bias": [("bias", None)],
    "relu": [("relu", None)],
    "chain": [("mul", 2.0), ("bias", None), ("relu", None), ("add", -0.75)],
}


def _ops(fa, torch, name, s_k, seed):
    """(device ops, oracle ops) for chain `name`; a bias holds s_k values drawn N(0, 2^2)."""
    vec = (rng_normal(seed, (s_k,))[0] * 2.0).astype(np.float32)
    dev_vec = torch.from_numpy(vec).cuda()
    dev, ref = [], []
    for kind, val in CHAINS[name]:
        if kind == "mul":
            dev.append(fa.Mul(val))
        elif kind == "add":
            dev.append(fa.Add(val))
        elif kind == "bias":
            dev.append(fa.Bias(dev_vec))
            val = vec
        else:
            dev.append(fa.ReLU())
        ref.append((kind, val))
    return dev, ref


@pytest.mark.parametrize("chain", list(CHAINS))
def test_fp32_prefill_score_ops(chain):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"score ops fp32 prefill {chain}")
    d, s_q, s_k = 64, 70, 203
    q, k, v = rng_normal(3000, (6, s_q, d), (2, s_k, d), (2, s_k, d))
    ops, ref_ops = _ops(fa, torch, chain, s_k, 3001)
    for causal, window in ((False, 0), (True, 0), (True, 37)):
        out, lse = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=causal,
                                      window=window, score_ops=ops, return_lse=True)
        assert fa.last_kernel() == "prefill_f32_sops"
        ref, lref = oracle.attention(q, k, v, causal=causal, window=window, score_epilogue=ref_ops)
        check_close(to_np(out), ref, TOL_F32, f"fp32 {chain} causal={causal} window={window}")
        check_close(to_np(lse), lref, TOL_F32 * 10, "lse")
    # int8 K/V through the fp32 kernel: the ops see the dequantized score
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    out = fa.flash_attention(to_dev(q, "f32"), kc, vc, k_scale=ks, v_scale=vs, causal=True, score_ops=ops)
    assert fa.last_kernel() == "prefill_f32_i8kv_sops"
    ref, _ = oracle.attention(q, to_np(kc), to_np(vc), causal=True, k_scale=to_np(ks), v_scale=to_np(vs),
                              score_epilogue=ref_ops)
    check_close(to_np(out), ref, TOL_F32, f"fp32 int8-KV {chain}")


@pytest.mark.parametrize("d", [64, 128, 96])
@pytest.mark.parametrize("chain", ["bias", "chain"])
def test_bf16_prefill_score_ops(d, chain):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"score ops bf16 prefill d={d} {chain}")
    s_q, s_k = 300, 333
    q, k, v = rng_normal(3100 + d, (4, s_q, d), (2, s_k, d), (2, s_k, d))
    qb, kb, vb = round_bf16(q), round_bf16(k), round_bf16(v)
    ops, ref_ops = _ops(fa, torch, chain, s_k, 3101 + d)
    args = (to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"))
    for causal, window in ((False, 0), (True, 0), (True, 90)):
        out, lse = fa.flash_attention(*args, causal=causal, window=window, out_dtype=torch.float32,
                                      score_ops=ops, return_lse=True)
        assert fa.last_kernel() == "prefill_bf16_sops"
        ref, lref = oracle.attention(qb, kb, vb, causal=causal, window=window, score_epilogue=ref_ops)
        check_close(to_np(out), ref, TOL_BF16, f"bf16 d={d} {chain} causal={causal} window={window}")
        check_close(to_np(lse), lref, 1e-4, "lse")
    # the same kernel without score ops is the plain one
    fa.flash_attention(*args, causal=True)
    assert fa.last_kernel() == "prefill_bf16"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chain", ["temperature", "chain"])
def test_int8_cache_prefill_score_ops(d, chain):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"score ops int8-cache prefill d={d} {chain}")
    s_q, s_k = 260, 390
    q, k, v = rng_normal(3200 + d, (8, s_q, d), (2, s_k, d), (2, s_k, d))
    qb = round_bf16(q)
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    ops, ref_ops = _ops(fa, torch, chain, s_k, 3201 + d)
    kq, ksn, vq, vsn = to_np(kc), to_np(ks), to_np(vc), to_np(vs)
    for causal, window in ((False, 0), (True, 0), (True, 100)):
        out = fa.flash_attention(to_dev(qb, "bf16"), kc, vc, k_scale=ks, v_scale=vs, causal=causal, window=window,
                                 out_dtype=torch.float32, score_ops=ops)
        assert fa.last_kernel() == "prefill_bf16_i8kv_sops"
        ref, _ = oracle.attention(qb, kq, vq, causal=causal, window=window, k_scale=ksn, v_scale=vsn,
                                  score_epilogue=ref_ops)
        check_close(to_np(out), ref, TOL_BF16, f"int8-cache d={d} {chain} causal={causal} window={window}")


@pytest.mark.parametrize("d,group", [(128, 4), (128, 8), (64, 8), (96, 2), (256, 4)])
@pytest.mark.parametrize("chain", list(CHAINS))
def test_decode_score_ops(d, group, chain):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say(f"score ops decode d={d} G={group} {chain}")
    bh_kv, s_k = 2, 2100
    q, k, v = rng_normal(3300 + d + group, (bh_kv * group, 1, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    v += np.float32(0.5)
    q = round_bf16(q)
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    kq, ksn, vq, vsn = to_np(kc), to_np(ks), to_np(vc), to_np(vs)
    ops, ref_ops = _ops(fa, torch, chain, s_k, 3301 + d)
    want = ("decode_int8_h8" if group > 4 and d <= 128 else "decode_int8") + "_sops"
    for window, splits in ((0, 0), (0, 7), (333, 3)):
        out, lse = fa.decode(to_dev(q, "bf16"), kc, vc, ks, vs, window=window, num_splits=splits, score_ops=ops,
                             return_lse=True)
        assert fa.last_kernel() == want
        ref, lref = oracle.decode(q, kq, vq, k_scale=ksn, v_scale=vsn, window=window, score_epilogue=ref_ops)
        check_close(to_np(out), ref, TOL_F32, f"decode d={d} G={group} {chain} window={window} splits={splits}")
        check_close(to_np(lse), lref[:, 0], TOL_F32 * 10, "lse")
    # the allocation-free entry point runs the same kernels: same bits
    out2 = torch.empty_like(out)
    fa.decode_noalloc(to_dev(q, "bf16"), kc, vc, ks, vs, out2, window=333, num_splits=3, score_ops=ops)
    assert torch.equal(out2, out)


@pytest.mark.parametrize("kb,vb", [(4, 2), (2, 4), (3, 3), (3, 4)])
@pytest.mark.parametrize("chain", ["bias", "chain"])
def test_tq_attention_score_ops(kb, vb, chain):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    d, bh_kv, G, s_k = 128, 2, 8 if kb == 3 else 4, 1300   # group 8: two wave groups per block
    say(f"score ops tq attention K{kb}/V{vb} {chain} G={G}")
    q, k, v = rng_normal(3400 + kb, (bh_kv * G, 1, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    q = round_bf16(q)
    sk, sv = random_signs(3401, d), random_signs(3402, d)
    kcb, vcb = fa.tq_codebook(d, kb), fa.tq_codebook(d, vb)
    skd, svd = torch.from_numpy(sk).cuda(), torch.from_numpy(sv).cuda()
    kc, kn = fa.tq_encode(to_dev(k, "f32"), skd, kb, kcb)
    vc, vn = fa.tq_encode(to_dev(v, "f32"), svd, vb, vcb)
    ops, ref_ops = _ops(fa, torch, chain, s_k, 3403)
    for window, splits in ((0, 0), (200, 3)):
        out = fa.tq_attention_decode(to_dev(q, "bf16"), kc, kn, skd, kb, kcb, vc, vn, svd, vb, vcb, window=window,
                                     num_splits=splits, score_ops=ops)
        assert fa.last_kernel() == "tq_attention_decode_sops"
        ref, _ = oracle.tq_attention_decode(q, to_np(kc), to_np(kn), sk, kb, to_np(vc), to_np(vn), sv, vb,
                                            k_codebook=kcb, v_codebook=vcb, window=window, score_epilogue=ref_ops)
        check_close(to_np(out), ref, TOL_F32, f"tq K{kb}/V{vb} {chain} window={window}")


def test_score_and_output_ops_together_and_merge_refuses_score_ops():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    say("score + output ops; merge refusal")
    d, s_k = 64, 150
    q, k, v = rng_normal(3500, (2, 40, d), (2, s_k, d), (2, s_k, d))
    sops, sref = _ops(fa, torch, "chain", s_k, 3501)
    out = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=True,
                             epilogue=[fa.Mul(3.0), fa.Add(0.25)], score_ops=sops)
    ref, _ = oracle.attention(q, k, v, causal=True, epilogue=[("mul", 3.0), ("add", 0.25)], score_epilogue=sref)
    check_close(to_np(out), ref, 3 * TOL_F32, "score + output ops")
    # a -1e30 bias on a set of keys takes them out of the softmax: equal to attention without them
    drop = np.zeros(s_k, np.float32)
    drop[::3] = -1e30
    keep = np.nonzero(drop == 0)[0]
    out = fa.flash_attention(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), causal=False,
                             score_ops=[fa.Bias(torch.from_numpy(drop).cuda())])
    ref, _ = oracle.attention(q, k[:, keep], v[:, keep], causal=False)
    check_close(to_np(out), ref, TOL_F32, "keys dropped by a -1e30 bias")
    o = to_dev(rng_normal(3502, (2, 10, d))[0], "f32")
    lse = to_dev(rng_normal(3503, (2, 10))[0], "f32")
    with pytest.raises(fa.FAError):
        fa._check(fa.lib().fa_merge_lse(fa._dev(o, "o"), fa._dev(lse, "l"), 2, 10, d, fa._dev(o, "o"), 0, None,
                                         *fa._epilogue([], d, [fa.Mul(2.0)], 10), None))
