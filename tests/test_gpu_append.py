"""GPU parity of the decode-time cache write (fa_append_kv): codes and scales bit-exact against
the oracle's cache write, including positions outside the cache, and one whole decode step
(append the new token, then attend) against the oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_E2E, TOL_F32, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu


def _random_cache(seed, bh, cap, d):
    g = np.random.Generator(np.random.PCG64(seed))
    kc = g.integers(-127, 128, (bh, cap, d)).astype(np.int8)
    vc = g.integers(-127, 128, (bh, cap, d)).astype(np.int8)
    ks = g.random((bh, cap)).astype(np.float32)
    vs = g.random((bh, cap)).astype(np.float32)
    return kc, vc, ks, vs


def _append(kn, vn, xdt, pos, cache):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    dev = [to_dev(c, "i8") if c.dtype == np.int8 else to_dev(c, "f32") for c in cache]
    fa.append_kv(to_dev(kn, xdt), to_dev(vn, xdt), torch.from_numpy(pos.astype(np.int32)).cuda(), *dev)
    torch.cuda.synchronize()
    return [to_np(t) for t in dev]


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_append_bit_exact(d, xdt):
    torch_gpu()
    for bh, n_new, cap in [(1, 1, 5), (5, 3, 40), (128, 1, 64), (7, 17, 20)]:
        say(f"append d={d} {xdt} bh={bh} n_new={n_new} cap={cap}")
        kn, vn = rng_normal(700 + d + n_new, (bh, n_new, d), (bh, n_new, d))
        kn[0, 0] = 0.0                     # an all-zero token
        if xdt == "bf16":
            kn, vn = round_bf16(kn), round_bf16(vn)
        g = np.random.Generator(np.random.PCG64(bh * 1000 + n_new))
        # positions inside, straddling the end, before the start and far past the end
        pos = g.integers(-n_new - 2, cap + 3, bh)
        pos[0] = 0
        if bh > 2:
            pos[1] = cap - n_new
            pos[2] = cap - 1
        cache = _random_cache(d + bh, bh, cap, d)
        got = _append(kn, vn, xdt, pos, cache)
        want = oracle.append_kv(*cache, kn, vn, pos)
        for name, a, b in zip(("k codes", "v codes", "k scales", "v scales"), got, want):
            assert np.array_equal(a.astype(b.dtype), b), f"{name} differ: {np.argwhere(a.astype(b.dtype) != b)[:5]}"


def test_append_equals_compress_of_the_same_rows():
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh, n, d = 16, 33, 128
    k, v = rng_normal(760, (bh, n, d), (bh, n, d))
    kc_all, ks_all = fa.compress_kv(to_dev(k, "f32"))
    cache = [np.zeros((bh, n, d), np.int8), np.zeros((bh, n, d), np.int8),
             np.zeros((bh, n), np.float32), np.zeros((bh, n), np.float32)]
    got = _append(k, v, "f32", np.zeros(bh, np.int64), cache)
    assert np.array_equal(got[0].astype(np.int8), to_np(kc_all).astype(np.int8))
    assert np.array_equal(got[2], to_np(ks_all))
    assert torch.cuda.is_available()


def test_decode_step_append_then_attend():
    """One serving decode step on a GQA cache with sequences at different lengths: the new
    token's K/V are appended at each head's length, then the split-KV decode attends over the
    cache including it.  Compared with the oracle on the oracle-quantized sequences."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh_kv, group, d, cap = 8, 4, 128, 3000
    lens = np.array([2999, 1, 1000, 2048, 17, 2500, 64, 1234])   # tokens already cached per head
    q, k, v = rng_normal(770, (bh_kv * group, 1, d), (bh_kv, cap, d), (bh_kv, cap, d))
    q = round_bf16(q)
    kq, ks = oracle.quantize_per_token(k)
    vq, vs = oracle.quantize_per_token(v)
    dev = [to_dev(kq, "i8"), to_dev(vq, "i8"), to_dev(ks, "f32"), to_dev(vs, "f32")]
    # the new token of head b is token lens[b] of its sequence: clear every row from there on
    for b in range(bh_kv):
        for t in dev:
            t[b, lens[b]:] = 0
    kn = np.stack([k[b, lens[b]] for b in range(bh_kv)])[:, None]
    vn = np.stack([v[b, lens[b]] for b in range(bh_kv)])[:, None]
    fa.append_kv(to_dev(kn, "f32"), to_dev(vn, "f32"), torch.from_numpy(lens.astype(np.int32)).cuda(), *dev)
    for b in range(bh_kv):
        say(f"decode step head {b} len {lens[b] + 1}")
        s = int(lens[b]) + 1
        sl = slice(b * group, (b + 1) * group)
        out = fa.decode(to_dev(q[sl], "bf16"), dev[0][b:b + 1, :s].contiguous(), dev[1][b:b + 1, :s].contiguous(),
                        dev[2][b:b + 1, :s].contiguous(), dev[3][b:b + 1, :s].contiguous())
        for t, want in zip(dev, (kq, vq, ks, vs)):
            assert np.array_equal(to_np(t[b, :s]).astype(want.dtype), want[b, :s])
            assert not np.any(to_np(t[b, s:]))
        ref, _ = oracle.decode(q[sl], kq[b:b + 1, :s], vq[b:b + 1, :s], k_scale=ks[b:b + 1, :s],
                               v_scale=vs[b:b + 1, :s])
        check_close(to_np(out), ref, TOL_F32, f"head {b}")
        if s >= 1024:
            e2e, _ = oracle.decode(q[sl], k[b:b + 1, :s], v[b:b + 1, :s])
            check_close(to_np(out), e2e, TOL_E2E, f"head {b} end to end")


def _rope_tables(cap, d, base=10000.0):
    inv = base ** (-np.arange(0, d // 2, dtype=np.float64) * 2.0 / d)
    ang = np.arange(cap, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_append_with_rope_bit_exact(d, xdt):
    """fa_append_kv_rope: K rotated by rotate-half RoPE at its cache position, then quantized;
    codes and scales bit-equal to the oracle's cache write with the same tables (positions inside,
    across and past the end of the cache; V unrotated)."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    for bh, n_new, cap in [(1, 1, 5), (5, 3, 40), (128, 1, 64), (7, 17, 20)]:
        say(f"append rope d={d} {xdt} bh={bh} n_new={n_new} cap={cap}")
        kn, vn = rng_normal(780 + d + n_new, (bh, n_new, d), (bh, n_new, d))
        if xdt == "bf16":
            kn, vn = round_bf16(kn), round_bf16(vn)
        g = np.random.Generator(np.random.PCG64(bh * 1000 + n_new + 7))
        pos = g.integers(-n_new - 2, cap + 3, bh)
        pos[0] = 0
        if bh > 2:
            pos[1] = cap - n_new
            pos[2] = cap - 1
        cos, sin = _rope_tables(cap, d)
        cache = _random_cache(d + bh + 1, bh, cap, d)
        dev = [to_dev(c, "i8") if c.dtype == np.int8 else to_dev(c, "f32") for c in cache]
        fa.append_kv(to_dev(kn, xdt), to_dev(vn, xdt), torch.from_numpy(pos.astype(np.int32)).cuda(), *dev,
                     rope_cos=to_dev(cos, "f32"), rope_sin=to_dev(sin, "f32"))
        torch.cuda.synchronize()
        assert fa.last_kernel() == ("append_rope_bf16" if xdt == "bf16" else "append_rope_f32")
        got = [to_np(t) for t in dev]
        want = oracle.append_kv(*cache, kn, vn, pos, rope_cos=cos, rope_sin=sin)
        for name, a, b in zip(("k codes", "v codes", "k scales", "v scales"), got, want):
            assert np.array_equal(a.astype(b.dtype), b), f"{name} differ: {np.argwhere(a.astype(b.dtype) != b)[:5]}"


def test_rope_append_then_decode_matches_attention_over_rotated_keys():
    """A decode step after a RoPE append: the query rotated at the last position attends over the
    rotated cache; against the oracle's decode over the oracle's cache write."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh_kv, G, cap, d = 4, 4, 300, 128
    k, v = rng_normal(790, (bh_kv, cap, d), (bh_kv, cap, d))
    q = rng_normal(791, (bh_kv * G, 1, d))[0]
    cos, sin = _rope_tables(cap, d)
    qr = round_bf16(oracle.rope_rotate_half(q, cos[cap - 1], sin[cap - 1]))
    z8, z = np.zeros((bh_kv, cap, d), np.int8), np.zeros((bh_kv, cap), np.float32)
    dev = [to_dev(z8, "i8"), to_dev(z8, "i8"), to_dev(z, "f32"), to_dev(z, "f32")]
    pos = torch.zeros(bh_kv, dtype=torch.int32, device="cuda")
    fa.append_kv(to_dev(k, "f32"), to_dev(v, "f32"), pos, *dev, rope_cos=to_dev(cos, "f32"), rope_sin=to_dev(sin, "f32"))
    kc, vc, ks, vs = oracle.append_kv(z8, z8, z, z, k, v, np.zeros(bh_kv, int), rope_cos=cos, rope_sin=sin)
    out = fa.decode(to_dev(qr, "bf16"), dev[0], dev[1], dev[2], dev[3])
    ref, _ = oracle.decode(qr, kc, vc, k_scale=ks, v_scale=vs)
    check_close(to_np(out), ref, TOL_F32, "decode over the RoPE cache")
