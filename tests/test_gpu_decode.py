"""GPU parity of the split-KV int8 decode against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_E2E, TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu


def _cache(k, v):
    import int8_compressed_kv_amd as fa
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    host = (to_np(kc).astype(np.int8), to_np(ks), to_np(vc).astype(np.int8), to_np(vs))
    return (kc, vc, ks, vs), host


@pytest.mark.parametrize("group", [1, 2, 4, 8, 6])
def test_decode_groups_ragged(group):
    import int8_compressed_kv_amd as fa
    torch_gpu()
    say(f"decode group={group}")
    bh_kv, s_k, d = 3, 5000, 128
    q, k, v = rng_normal(400 + group, (bh_kv * group, 1, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
    q = round_bf16(q)
    dev, (kq, ks, vq, vs) = _cache(k, v)
    ref, lref = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
    for splits in (0, 1, 7):
        out, lse = fa.decode(to_dev(q, "bf16"), *dev, num_splits=splits, return_lse=True)
        check_close(to_np(out), ref, TOL_F32, f"G={group} splits={splits}")
        check_close(to_np(lse), lref[:, 0], TOL_F32, "lse")
    e2e, _ = oracle.decode(q, k, v)
    check_close(to_np(out), e2e, TOL_E2E, "end to end vs unquantized")


@pytest.mark.parametrize("d", [32, 64, 96, 160, 192, 224, 256])
def test_decode_head_dims(d):
    import int8_compressed_kv_amd as fa
    torch_gpu()
    say(f"decode d={d}")
    q, k, v = rng_normal(500 + d, (8, 1, d), (2, 1111, d), (2, 1111, d))
    dev, (kq, ks, vq, vs) = _cache(k, v)
    for qdt in ("bf16", "f32"):
        qq = round_bf16(q) if qdt == "bf16" else q
        out = fa.decode(to_dev(qq, qdt), *dev, num_splits=3)
        ref, _ = oracle.decode(qq, kq, vq, k_scale=ks, v_scale=vs)
        check_close(to_np(out), ref, TOL_F32, f"d={d} q={qdt}")


def test_decode_window_short_cache_and_epilogue():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    q, k, v = rng_normal(600, (8, 1, 128), (2, 3000, 128), (2, 3000, 128))
    q = round_bf16(q)
    dev, (kq, ks, vq, vs) = _cache(k, v)
    out = fa.decode(to_dev(q, "bf16"), *dev, window=777, num_splits=4)
    ref, _ = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs, window=777)
    check_close(to_np(out), ref, TOL_F32, "window 777")
    # more splits than tiles: empty splits merge to nothing
    q2, k2, v2 = rng_normal(601, (4, 1, 64), (1, 70, 64), (1, 70, 64))
    dev2, (kq2, ks2, vq2, vs2) = _cache(k2, v2)
    out2 = fa.decode(to_dev(round_bf16(q2), "bf16"), *dev2, num_splits=16)
    ref2, _ = oracle.decode(round_bf16(q2), kq2, vq2, k_scale=ks2, v_scale=vs2)
    check_close(to_np(out2), ref2, TOL_F32, "splits > tiles")
    # epilogue: fused equals host-applied on the same kernel output
    o0 = fa.decode(to_dev(q, "bf16"), *dev, num_splits=4)
    o1 = fa.decode(to_dev(q, "bf16"), *dev, num_splits=4, epilogue=[fa.Mul(2.0), fa.Add(0.5)])
    assert torch.equal(o1.cpu(), o0.cpu() * 2.0 + 0.5)
    ob = fa.decode(to_dev(q, "bf16"), *dev, num_splits=4, out_dtype=torch.bfloat16)
    assert torch.equal(ob, o0.to(torch.bfloat16))


def test_decode_equals_last_row_of_fp32_prefill_on_the_same_cache():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    q, k, v = rng_normal(602, (8, 1, 128), (2, 2000, 128), (2, 2000, 128))
    q = round_bf16(q)
    dev, _ = _cache(k, v)
    od = fa.decode(to_dev(q, "bf16"), *dev)
    kc, vc, ks, vs = dev
    op = fa.flash_attention(to_dev(q, "f32"), kc, vc, k_scale=ks, v_scale=vs, causal=True)
    check_close(to_np(od), to_np(op).astype(np.float64), 2e-6, "decode vs s_q = 1 prefill")


def test_decode_split_count_independence_and_determinism():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    q, k, v = rng_normal(603, (16, 1, 128), (4, 9000, 128), (4, 9000, 128))
    q = round_bf16(q)
    dev, _ = _cache(k, v)
    outs = [to_np(fa.decode(to_dev(q, "bf16"), *dev, num_splits=s)) for s in (1, 2, 5, 13, 32)]
    for o in outs[1:]:
        check_close(o, outs[0].astype(np.float64), 2e-6, "split independence")
    a = fa.decode(to_dev(q, "bf16"), *dev, num_splits=5)
    b = fa.decode(to_dev(q, "bf16"), *dev, num_splits=5)
    assert torch.equal(a, b)


def test_decode_extreme_scales():
    """Per-token scales spanning many octaves within one head (outlier tokens).  The outputs reach
    about 1e3, where fp32 itself resolves only about 1e-4, so the bar is applied relative to the
    largest output; the absolute bar is exercised at unit scale by the other decode tests."""
    import int8_compressed_kv_amd as fa
    torch_gpu()
    q, k, v = rng_normal(604, (4, 1, 128), (1, 4000, 128), (1, 4000, 128))
    q = round_bf16(q)
    v[0, ::7] *= np.float32(1e3)
    v[0, 1::11] *= np.float32(1e-3)
    k[0, ::13] *= np.float32(5.0)
    dev, (kq, ks, vq, vs) = _cache(k, v)
    out = fa.decode(to_dev(q, "bf16"), *dev, num_splits=3)
    ref, _ = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
    scale = np.abs(ref).max()
    check_close(to_np(out) / scale, ref / scale, TOL_F32, "relative to max |out|")


@pytest.mark.parametrize("kind", ["sink12", "sink16", "rising", "step"])
@pytest.mark.parametrize("group", [4, 8])
def test_decode_long_cache_score_profiles_absolute(kind, group):
    """32768 keys with a non-zero-mean V (channel mean 0.5) and the score profiles that stress
    the P~ V digit scale: an attention sink 12 / 16 nats above the rest, scores rising 0 -> 30
    nats over the cache, and a 7-octave step (below the lazy-raise threshold) followed by a
    20-nat step (a raise).  Checked at an absolute 1e-5 against the dequantized oracle, in the
    split count the long-cache workload uses (2 per KV head at 128 KV heads) and the automatic one."""
    import int8_compressed_kv_amd as fa
    from synth_inputs import decode_profile_inputs
    torch_gpu()
    bh_kv, s_k, d = 4, 32768, 128
    say(f"decode profile={kind} G={group} s_k={s_k}")
    q, k, v = decode_profile_inputs(700 + group, bh_kv, group, s_k, d, kind)
    dev, (kq, ks, vq, vs) = _cache(k, v)
    ref, lref = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
    for splits in (2, 0):
        out, lse = fa.decode(to_dev(q, "bf16"), *dev, num_splits=splits, return_lse=True)
        check_close(to_np(out), ref, TOL_F32, f"{kind} G={group} splits={splits}")
        check_close(to_np(lse), lref[:, 0], TOL_F32 * max(1.0, float(np.abs(lref).max())), "lse")
    assert fa.last_kernel() == ("decode_int8_h8" if group == 8 else "decode_int8")


def test_decode_group8_reads_the_cache_with_one_workgroup_set():
    """G = 8 at head_dim 128: one workgroup serves all 8 query heads of its KV head (grid z = 1),
    and the split count matches G = 4 for the same number of KV heads."""
    import int8_compressed_kv_amd as fa
    torch_gpu()
    assert fa.decode_num_splits(8 * 128, 128, 32768, 128) == fa.decode_num_splits(4 * 128, 128, 32768, 128)
    q, k, v = rng_normal(710, (16, 1, 128), (2, 3000, 128), (2, 3000, 128))
    q = round_bf16(q)
    dev, (kq, ks, vq, vs) = _cache(k, v)
    ref, _ = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
    for splits in (0, 1, 5):
        out = fa.decode(to_dev(q, "bf16"), *dev, num_splits=splits)
        check_close(to_np(out), ref, TOL_F32, f"G=8 splits={splits}")
        assert fa.last_kernel() == "decode_int8_h8"


@pytest.mark.parametrize("d", [32, 96, 128])
@pytest.mark.parametrize("group", [4, 8])
def test_decode_tiny_caches_end_at_the_allocation(d, group):
    """Caches of 1 to 33 keys, so the only (or last) tile runs past the last key of the last KV
    head, which is the end of the cache allocation: rows past it must read as zeros and be
    masked.  At head_dim 32 and 96 some lanes' K chunks lie past the row (their Q digits are
    zero); the last row's overhang is past the allocation too."""
    import int8_compressed_kv_amd as fa
    torch_gpu()
    for s_k in (1, 7, 31, 32, 33):
        say(f"decode tiny d={d} G={group} s_k={s_k}")
        q, k, v = rng_normal(720 + s_k + d, (2 * group, 1, d), (2, s_k, d), (2, s_k, d))
        q = round_bf16(q)
        dev, (kq, ks, vq, vs) = _cache(k, v)
        ref, lref = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
        for splits in (0, 1, 3):
            out, lse = fa.decode(to_dev(q, "bf16"), *dev, num_splits=splits, return_lse=True)
            check_close(to_np(out), ref, TOL_F32, f"d={d} G={group} s_k={s_k} splits={splits}")
            check_close(to_np(lse), lref[:, 0], TOL_F32, "lse")
