"""GPU parity of the log-sum-exp merge (fa_merge_lse) against the oracle, on random parts with
empty chunks, and a causal prefill split into aligned query/key chunks (the exchange of a ring /
context-parallel prefill, run on one GPU) against the oracle over all keys."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL_BF16, TOL_F32, check_bf16_output, check_close, say, to_dev, to_np, torch_gpu
from synth_inputs import rng_normal, round_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_merge_random_parts(d):
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    for n_parts, rows in [(1, 7), (2, 300), (5, 1000), (8, 129), (9, 64), (17, 65)]:
        say(f"merge d={d} parts={n_parts} rows={rows}")
        o = rng_normal(800 + d + n_parts, (n_parts, rows, d))[0]
        g = np.random.Generator(np.random.PCG64(n_parts * 100 + d))
        lse = (g.standard_normal((n_parts, rows)) * 20).astype(np.float32)
        lse[g.random((n_parts, rows)) < 0.3] = -np.inf       # chunks with no visible key
        lse[:, :2] = -np.inf                                   # rows no chunk covers
        o[np.isneginf(lse)] = 0.0
        ref, lref = oracle.merge_lse(o, lse, epilogue=[("mul", -1.5), ("add", 0.25)])
        out, l = fa.merge_lse(to_dev(o, "f32"), to_dev(lse, "f32"), epilogue=[fa.Mul(-1.5), fa.Add(0.25)],
                              return_lse=True)
        check_close(to_np(out), ref, TOL_F32, "merged output")
        lg = to_np(l)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lref))
        fin = np.isfinite(lref)
        check_close(lg[fin], lref[fin], 1e-5, "merged lse")
        ob = fa.merge_lse(to_dev(o, "f32"), to_dev(lse, "f32"), out_dtype=torch.bfloat16)
        out0 = fa.merge_lse(to_dev(o, "f32"), to_dev(lse, "f32"))
        assert torch.equal(out0.to(torch.bfloat16), ob), "bf16 store is not the RNE of the fp32 result"


@pytest.mark.parametrize("n_chunks", [2, 4])
def test_chunked_causal_prefill_equals_full_attention(n_chunks):
    """Queries and keys cut into the same chunks: block (r, c) is full for c < r, a causal
    diagonal for c == r and empty for c > r; each query chunk merges its blocks."""
    import int8_compressed_kv_amd as fa
    torch = torch_gpu()
    bh_q, bh_kv, s, d = 16, 2, 2048, 128
    q, k, v = rng_normal(820 + n_chunks, (bh_q, s, d), (bh_kv, s, d), (bh_kv, s, d))
    q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    cuts = np.linspace(0, s, n_chunks + 1).astype(int)
    cuts[1] = 700 if n_chunks == 4 else cuts[1]          # unequal chunks
    full_gpu = fa.flash_attention(qd, kd, vd, causal=True, out_dtype=torch.float32)
    ref, lref = oracle.attention(q, k, v, causal=True, rows=range(0, s, 7))
    rows = np.arange(0, s, 7)
    merged = np.empty((bh_q, s, d), np.float32)
    for r in range(n_chunks):
        r0, r1 = cuts[r], cuts[r + 1]
        qc = qd[:, r0:r1].contiguous()
        o_parts, l_parts = [], []
        for c in range(r + 1):
            c0, c1 = cuts[c], cuts[c + 1]
            o, l = fa.flash_attention(qc, kd[:, c0:c1].contiguous(), vd[:, c0:c1].contiguous(), causal=(c == r),
                                      out_dtype=torch.float32, return_lse=True)
            o_parts.append(o)
            l_parts.append(l)
        say(f"chunks={n_chunks} query chunk {r}: {len(o_parts)} parts")
        out = fa.merge_lse(torch.stack(o_parts), torch.stack(l_parts))
        merged[:, r0:r1] = to_np(out)
    check_close(merged[:, rows], ref[:, rows], TOL_BF16, "chunked vs oracle (bf16 inputs)")
    check_close(merged, to_np(full_gpu), TOL_BF16, "chunked vs one-shot kernel")
    mb = fa.merge_lse(torch.stack([full_gpu]), torch.from_numpy(np.zeros((1, bh_q, s), np.float32)).cuda(),
                      out_dtype=torch.bfloat16)
    check_bf16_output(to_np(mb)[:, rows], ref[:, rows], "single part through the merge, bf16 out")
