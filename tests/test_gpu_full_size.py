"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot finish a whole 32768-token causal prefill in test time, so it checks sampled
outputs: whole query heads at the group boundaries, and within them the first rows, the rows
around the window edge, rows spread through the sequence and the last rows (the ones that see the
most keys).  The decode workload is small enough for the oracle to check every output.
"""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_E2E, TOL_F32, check_bf16_output, check_close, say, to_np, torch_gpu
from synth_inputs import WORKLOADS, draw_qkv

pytestmark = pytest.mark.gpu


def _oracle_rows(q, k, v, heads, rows, group, **kw):
    """Oracle outputs (len(heads), len(rows), d) computed one query head at a time."""
    res = []
    for h in heads:
        kvh = h // group
        sl = slice(kvh, kvh + 1)
        extra = {}
        if "k_scale" in kw:
            extra = {"k_scale": kw["k_scale"][sl], "v_scale": kw["v_scale"][sl]}
        o, _ = oracle.attention(q[h:h + 1], k[sl], v[sl], causal=kw["causal"], window=kw.get("window", 0),
                                rows=rows, **extra)
        res.append(o[0, rows])
    return np.stack(res)


def _sample_rows(s, extra=()):
    rng = np.random.Generator(np.random.PCG64(12345))
    rows = set(range(0, 64)) | set(range(s - 64, s)) | set(int(x) for x in rng.integers(0, s, 64))
    for e in extra:
        rows |= set(range(max(0, e - 4), min(s, e + 4)))
    return sorted(rows)


@pytest.mark.parametrize("leg", ["c5", "c5w"])
def test_full_size_gqa_prefill_bf16(leg):
    torch = torch_gpu()
    import int8_compressed_kv_amd as fa
    w = WORKLOADS[leg]
    say(f"full size {w.name}")
    q, k, v = draw_qkv(w)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    kd = torch.from_numpy(k).cuda().to(torch.bfloat16)
    vd = torch.from_numpy(v).cuda().to(torch.bfloat16)
    out = torch.empty_like(qd)
    fa.flash_attention(qd, kd, vd, causal=True, window=w.window, out=out)
    torch.cuda.synchronize()
    heads = [0, 7, 8, 31, 63]                    # both ends of the first GQA group, the next group, the last head
    rows = _sample_rows(w.s_q, extra=(w.window, w.window + 1000) if w.window else (4096,))
    ref = _oracle_rows(q, k, v, heads, rows, w.group, causal=True, window=w.window)
    got = out[heads][:, rows].float().cpu().numpy()
    check_bf16_output(got, ref, f"{leg} sampled {len(heads)} heads x {len(rows)} rows")


def test_full_size_int8_kv_prefill():
    torch = torch_gpu()
    import int8_compressed_kv_amd as fa
    w = WORKLOADS["c3"]
    say(f"full size {w.name}")
    q, k, v = draw_qkv(w)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    kc, ks = fa.compress_kv(torch.from_numpy(k).cuda())
    vc, vs = fa.compress_kv(torch.from_numpy(v).cuda())
    out = torch.empty_like(qd)
    fa.flash_attention(qd, kc, vc, k_scale=ks, v_scale=vs, causal=True, out=out)
    torch.cuda.synchronize()
    heads = [0, 31, 32, 127]
    rows = _sample_rows(w.s_q, extra=(1024,))
    kq, ksn = to_np(kc).astype(np.int8), to_np(ks)
    vq, vsn = to_np(vc).astype(np.int8), to_np(vs)
    # the cache itself: bit-exact against the oracle quantizer on the sampled heads
    for h in heads:
        qk_ref, sk_ref = oracle.quantize_per_token(k[h])
        assert np.array_equal(kq[h], qk_ref) and np.array_equal(ksn[h], sk_ref), f"K cache head {h}"
    ref = _oracle_rows(q, kq, vq, heads, rows, 1, causal=True, k_scale=ksn, v_scale=vsn)
    got = out[heads][:, rows].float().cpu().numpy()
    check_bf16_output(got, ref, "c3 vs dequantized oracle")
    # end to end against unquantized attention, on rows that see at least 1024 keys
    long_rows = [r for r in rows if r + 1 >= 1024]
    e2e = _oracle_rows(q, k, v, heads, long_rows, 1, causal=True)
    check_close(out[heads][:, long_rows].float().cpu().numpy(), e2e, TOL_E2E,
                "c3 end to end (rows with >= 1024 visible keys)")


def test_full_size_gqa_decode_all_outputs():
    torch = torch_gpu()
    import int8_compressed_kv_amd as fa
    w = WORKLOADS["c4"]
    say(f"full size {w.name}")
    q, k, v = draw_qkv(w)
    qd = torch.from_numpy(q).cuda().to(torch.bfloat16)
    kc, ks = fa.compress_kv(torch.from_numpy(k).cuda())
    vc, vs = fa.compress_kv(torch.from_numpy(v).cuda())
    splits = fa.decode_num_splits(w.bh_q, w.bh_kv, w.s_k, w.d)
    ws = torch.empty(fa.decode_workspace_bytes(w.bh_q, w.bh_kv, w.s_k, w.d, splits), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.bh_q, 1, w.d), dtype=torch.float32, device="cuda")
    fa.decode(qd, kc, vc, ks, vs, num_splits=splits, out=out, workspace=ws)
    torch.cuda.synchronize()
    got = to_np(out)
    G = w.group
    err = e2e_err = 0.0
    for kvh in range(w.bh_kv):          # one KV head at a time keeps the fp64 copies small
        hq = slice(kvh * G, (kvh + 1) * G)
        kq = to_np(kc[kvh:kvh + 1]).astype(np.int8)
        vq = to_np(vc[kvh:kvh + 1]).astype(np.int8)
        ref, _ = oracle.decode(q[hq], kq, vq, k_scale=to_np(ks[kvh:kvh + 1]), v_scale=to_np(vs[kvh:kvh + 1]))
        err = max(err, float(np.abs(got[hq] - ref).max()))
        if kvh % 16 == 0:
            e2e, _ = oracle.decode(q[hq], k[kvh:kvh + 1], v[kvh:kvh + 1])
            e2e_err = max(e2e_err, float(np.abs(got[hq] - e2e).max()))
    say(f"  c4 all {w.bh_q} heads: max abs err {err:.3e} vs dequantized, {e2e_err:.3e} end to end (8 KV heads)")
    assert err <= TOL_F32
    assert e2e_err <= TOL_E2E
