"""fa_decode_noalloc: the decode with its partial states in the library's fixed device scratch
array instead of a caller workspace.  Its output must equal fa_decode's on the same inputs and
split count bit for bit (same kernels), and the oracle's to the int8-vs-dequantized bar, on two
calls in a row where the second is smaller (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16


def _cache(fa, k, v):
    kc, ks = fa.compress_kv(to_dev(k, "f32"))
    vc, vs = fa.compress_kv(to_dev(v, "f32"))
    host = (to_np(kc).astype(np.int8), to_np(ks), to_np(vc).astype(np.int8), to_np(vs))
    return (kc, vc, ks, vs), host


@pytest.mark.gpu
def test_decode_noalloc_equals_decode_on_two_calls():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    cases = [  # (seed, bh_kv, group, s_k, d, splits): the second call is smaller
        (810, 8, 4, 20000, 128, 0),
        (811, 2, 8, 3001, 64, 3),
    ]
    for seed, bh_kv, group, s_k, d, splits in cases:
        say(f"decode_noalloc seed={seed} bh_kv={bh_kv} G={group} s_k={s_k} d={d} splits={splits}")
        q, k, v = rng_normal(seed, (bh_kv * group, 1, d), (bh_kv, s_k, d), (bh_kv, s_k, d))
        q = round_bf16(q)
        dev, (kq, ks, vq, vs) = _cache(fa, k, v)
        qd = to_dev(q, "bf16")
        ref_out, ref_lse = fa.decode(qd, *dev, num_splits=splits, return_lse=True)
        out = torch.full((bh_kv * group, 1, d), float("nan"), device="cuda")
        lse = torch.full((bh_kv * group,), float("nan"), device="cuda")
        fa.decode_noalloc(qd, *dev, out, lse=lse, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "fa_decode_noalloc differs from fa_decode"
        assert torch.equal(lse, ref_lse)
        ref, _ = oracle.decode(q, kq, vq, k_scale=ks, v_scale=vs)
        check_close(to_np(out), ref, TOL_F32, "noalloc vs oracle")


@pytest.mark.gpu
def test_decode_noalloc_rejects_states_beyond_the_scratch():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    cap = int(fa.lib().fa_decode_noalloc_max_bytes())
    bh_kv, group, s_k, d = 16, 8, 4096, 256
    per = (d + 2) * 4 * bh_kv * group
    splits = cap // per + 1            # one split more than fits
    q = torch.zeros((bh_kv * group, 1, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((bh_kv, s_k, d), dtype=torch.int8, device="cuda")
    s = torch.zeros((bh_kv, s_k), dtype=torch.float32, device="cuda")
    out = torch.zeros((bh_kv * group, 1, d), device="cuda")
    with pytest.raises(fa.FAError, match="scratch"):
        fa.decode_noalloc(q, k, k, s, s, out, num_splits=splits)


def test_decode_noalloc_size_limit_is_checked_on_the_host():
    """Sizes past the fixed scratch are refused before any HIP call (runs without a GPU)."""
    import ctypes
    import int8_compressed_kv_amd as fa
    L = fa.lib()
    cap = int(L.fa_decode_noalloc_max_bytes())
    assert cap == 4 << 20
    bh_q, bh_kv, s_k, d = 128, 16, 4096, 256
    splits = cap // ((d + 2) * 4 * bh_q) + 1
    vp = ctypes.c_void_p
    p = vp(1 << 20)
    rc = L.fa_decode_noalloc(p, 1, p, p, p, p, p, 0, None, bh_q, bh_kv, s_k, d, 0.0, 0, splits, None, 0, None)
    assert rc == -3 and "scratch" in fa.last_error()
    assert L.fa_decode_noalloc(p, 1, p, p, p, p, p, 0, None, bh_q, bh_kv, s_k, 48, 0.0, 0, 1, None, 0, None) == -2
