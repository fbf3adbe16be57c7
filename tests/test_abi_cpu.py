"""C-ABI checks that need no GPU: the library loads, exports every function include/fa.h
declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("int8_compressed_kv_amd")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail(f"{fa.LIB_PATH} not built; run python -m int8_compressed_kv_amd.build")
    return fa.lib()


def test_header_declares_the_three_operations():
    names = _header_functions()
    for n in ("fa_compress_kv", "fa_append_kv", "fa_forward", "fa_merge_lse", "fa_decode", "fa_decode_workspace_bytes",
              "fa_decode_num_splits", "fa_last_error", "fa_last_kernel", "fa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _header_functions():
        assert hasattr(L, n), f"libfa.so does not export {n}"


def test_version(L):
    assert L.fa_version() >= 10000


def _fwd(L, **kw):
    a = dict(q=1 << 20, qd=0, k=1 << 20, v=1 << 20, kvd=0, ks=None, vs=None, out=1 << 20, od=0, lse=None,
             bh_q=2, bh_kv=2, s_q=8, s_k=8, d=64, scale=0.0, causal=1, window=0, epi=None, n_epi=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.fa_forward(vp(a["q"]), a["qd"], vp(a["k"]), vp(a["v"]), a["kvd"], vp(a["ks"]), vp(a["vs"]),
                        vp(a["out"]), a["od"], vp(a["lse"]), a["bh_q"], a["bh_kv"], a["s_q"], a["s_k"], a["d"],
                        a["scale"], a["causal"], a["window"], a["epi"], a["n_epi"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=48), -2), (dict(d=288), -2), (dict(d=0), -1),
    (dict(bh_q=3, bh_kv=2), -1), (dict(bh_q=0), -1),
    (dict(s_q=-1), -1),
    (dict(window=4, causal=0), -1), (dict(window=-1), -1),
    (dict(qd=2), -2), (dict(kvd=7), -2), (dict(od=2), -2),
    (dict(qd=0, kvd=1), -2),                       # fp32 Q with bf16 K/V
    (dict(kvd=2), -1),                             # int8 without scales
    (dict(ks=1 << 20, vs=1 << 20), -1),            # scales with float K/V
    (dict(q=0), -1), (dict(out=0), -1),
    (dict(q=(1 << 20) + 4), -1),                   # misaligned
    (dict(n_epi=9), -2), (dict(n_epi=-1), -1), (dict(n_epi=1, epi=None), -1),
])
def test_forward_rejects_invalid_arguments_on_host(L, kw, code):
    rc = _fwd(L, **kw)
    assert rc == code, (rc, fa.last_error())
    assert fa.last_error() != ""


def test_forward_rejects_unknown_epilogue_kind(L):
    ops = (fa._EpiOp * 1)(fa._EpiOp(7, 1.0))
    assert _fwd(L, epi=ops, n_epi=1) == -1
    assert "kind" in fa.last_error()


def test_forward_empty_query_is_a_noop(L):
    assert _fwd(L, s_q=0, q=0, out=0) == 0


def test_compress_rejects_invalid_arguments(L):
    vp = ctypes.c_void_p
    assert L.fa_compress_kv(vp(1 << 20), 0, 4, 48, vp(1 << 20), vp(1 << 20), None) == -2
    assert L.fa_compress_kv(vp(1 << 20), 2, 4, 64, vp(1 << 20), vp(1 << 20), None) == -2
    assert L.fa_compress_kv(vp(0), 0, 4, 64, vp(1 << 20), vp(1 << 20), None) == -1
    assert L.fa_compress_kv(vp(1 << 20), 0, -1, 64, vp(1 << 20), vp(1 << 20), None) == -1
    assert L.fa_compress_kv(vp(0), 0, 0, 64, vp(0), vp(0), None) == 0


def _dec(L, **kw):
    a = dict(q=1 << 20, qd=1, k=1 << 20, v=1 << 20, ks=1 << 20, vs=1 << 20, out=1 << 20, od=0, lse=None,
             bh_q=8, bh_kv=2, s_k=1000, d=128, scale=0.0, window=0, splits=0, epi=None, n_epi=0,
             ws=1 << 20, ws_bytes=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.fa_decode(vp(a["q"]), a["qd"], vp(a["k"]), vp(a["v"]), vp(a["ks"]), vp(a["vs"]), vp(a["out"]),
                       a["od"], vp(a["lse"]), a["bh_q"], a["bh_kv"], a["s_k"], a["d"], a["scale"], a["window"],
                       a["splits"], a["epi"], a["n_epi"], vp(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), -2), (dict(bh_q=9), -1), (dict(qd=2), -2), (dict(od=2), -2),
    (dict(splits=-1), -1), (dict(splits=5000), -1), (dict(window=-3), -1),
    (dict(ws=0), -3), (dict(ws_bytes=16), -3), (dict(k=0), -1), (dict(ks=0), -1),
])
def test_decode_rejects_invalid_arguments_on_host(L, kw, code):
    rc = _dec(L, **kw)
    assert rc == code, (rc, fa.last_error())


def test_decode_workspace_and_split_sizing(L):
    s = fa.decode_num_splits(512, 128, 32768, 128)
    assert 1 <= s <= 4096
    assert fa.decode_workspace_bytes(512, 128, 32768, 128, 0) == 512 * s * (128 + 2) * 4
    assert fa.decode_workspace_bytes(512, 128, 32768, 128, 7) == 512 * 7 * 130 * 4
    assert fa.decode_num_splits(4, 1, 100, 64) == 1
    # exact workspace passes the size check (argument checks then reach the launch stage only on a GPU)
    need = fa.decode_workspace_bytes(8, 2, 1000, 128, 3)
    assert _dec(L, splits=3, ws_bytes=need - 4) == -3


def test_python_layer_validates_shapes():
    torch = pytest.importorskip("torch")
    q = torch.zeros(2, 4, 64)
    with pytest.raises(ValueError):
        fa.flash_attention(q, torch.zeros(2, 4, 32), torch.zeros(2, 4, 32))
    with pytest.raises(ValueError):
        fa.flash_attention(q, torch.zeros(2, 4, 64), torch.zeros(2, 4, 64))   # CPU tensors
    with pytest.raises(TypeError):
        fa._epilogue([("mul", 2.0)])
    with pytest.raises(ValueError):
        fa._epilogue([fa.Mul(1.0)] * 9)


def _app(L, **kw):
    a = dict(kn=1 << 20, vn=1 << 20, xd=0, bh=4, n=1, d=128, pos=1 << 20, cap=100, kc=1 << 20, vc=1 << 20,
             ks=1 << 20, vs=1 << 20)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.fa_append_kv(vp(a["kn"]), vp(a["vn"]), a["xd"], a["bh"], a["n"], a["d"], vp(a["pos"]), a["cap"],
                          vp(a["kc"]), vp(a["vc"]), vp(a["ks"]), vp(a["vs"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=40), -2), (dict(xd=2), -2), (dict(bh=0), -1), (dict(n=-1), -1), (dict(cap=0), -1),
    (dict(pos=0), -1), (dict(kc=0), -1), (dict(vs=0), -1), (dict(kn=(1 << 20) + 8), -1),
    (dict(ks=(1 << 20) + 2), -1),
])
def test_append_rejects_invalid_arguments_on_host(L, kw, code):
    rc = _app(L, **kw)
    assert rc == code, (rc, fa.last_error())


def test_append_zero_tokens_is_a_noop(L):
    assert _app(L, n=0, kn=0, vn=0, pos=0, kc=0, vc=0, ks=0, vs=0) == 0


def _mrg(L, **kw):
    a = dict(o=1 << 20, l=1 << 20, n=2, rows=10, d=64, out=1 << 20, od=0, lse=None, epi=None, n_epi=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.fa_merge_lse(vp(a["o"]), vp(a["l"]), a["n"], a["rows"], a["d"], vp(a["out"]), a["od"], vp(a["lse"]),
                          a["epi"], a["n_epi"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=50), -2), (dict(n=0), -1), (dict(rows=-1), -1), (dict(od=2), -2), (dict(o=0), -1),
    (dict(out=(1 << 20) + 8), -1), (dict(l=(1 << 20) + 2), -1), (dict(n_epi=9), -2),
])
def test_merge_rejects_invalid_arguments_on_host(L, kw, code):
    rc = _mrg(L, **kw)
    assert rc == code, (rc, fa.last_error())


def test_merge_zero_rows_is_a_noop(L):
    assert _mrg(L, rows=0, o=0, l=0, out=0) == 0


def test_bias_and_relu_ops_are_validated_on_host(L):
    E = fa._EpiOp
    ok = (E * 2)(E(4, 0.0, None), E(3, 0.0, 1 << 20))
    assert _fwd(L, epi=ok, n_epi=2, q=0) == -1 and "null q" in fa.last_error()   # ops accepted; fails later
    no_vec = (E * 1)(E(3, 0.0, None))
    assert _fwd(L, epi=no_vec, n_epi=1) == -1 and "bias" in fa.last_error()
    odd_vec = (E * 1)(E(3, 0.0, (1 << 20) + 2))
    assert _fwd(L, epi=odd_vec, n_epi=1) == -1
    stray_vec = (E * 1)(E(4, 0.0, 1 << 20))
    assert _fwd(L, epi=stray_vec, n_epi=1) == -1 and "NULL" in fa.last_error()
    assert ctypes.sizeof(E) == 24   # int32 kind, float value, pointer vec, int32 scope (+ padding)


def test_epilogue_scopes_are_validated_on_host(L):
    E = fa._EpiOp
    # K-tile (score) ops are accepted by the calls that form scores ...
    both = (E * 3)(E(1, 2.0, None, 0), E(3, 0.0, 1 << 20, 1), E(4, 0.0, None, 1))
    assert _fwd(L, epi=both, n_epi=3, q=0) == -1 and "null q" in fa.last_error()
    assert _dec(L, epi=both, n_epi=3, q=0) == -1 and "null" in fa.last_error()
    # ... and refused by the merge, which forms none
    assert _mrg(L, epi=both, n_epi=3) == -2 and "K-tile" in fa.last_error()
    out_only = (E * 1)(E(1, 2.0, None, 0))
    assert _mrg(L, epi=out_only, n_epi=1, o=0) == -1 and "null" in fa.last_error()
    kernel = (E * 1)(E(1, 2.0, None, 2))
    assert _fwd(L, epi=kernel, n_epi=1) == -2 and "kernel scope" in fa.last_error()
    bad = (E * 1)(E(1, 2.0, None, 5))
    assert _fwd(L, epi=bad, n_epi=1) == -1 and "scope" in fa.last_error()
    nine = (E * 9)(*[E(1, 1.0, None, i % 2) for i in range(9)])
    assert _fwd(L, epi=nine, n_epi=9) == -2


def test_python_epilogue_ops_check_the_bias_vector():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        fa._epilogue([fa.Bias(torch.zeros(64, dtype=torch.float64))], 64)
    with pytest.raises(ValueError):
        fa._epilogue([fa.Bias(torch.zeros(32))], 64)
    arr, n = fa._epilogue([fa.ReLU(), fa.Mul(2.0)], 64)
    assert n == 2 and arr[0].kind == 4 and arr[1].kind == 1
    arr, n = fa._epilogue([fa.Mul(2.0)], 64, [fa.Add(1.0), fa.ReLU()], 1000)
    assert n == 3 and [arr[i].scope for i in range(3)] == [0, 1, 1] and arr[1].kind == 2
    with pytest.raises(ValueError):       # a score bias holds s_k values
        fa._epilogue([], 64, [fa.Bias(torch.zeros(64))], 1000)
    with pytest.raises(ValueError):
        fa._epilogue([fa.Mul(1.0)] * 5, 64, [fa.Mul(1.0)] * 4, 1000)


def test_tq_codebook_on_host_matches_the_oracle_in_fp32(L):
    import numpy as np
    import oracle
    for d in (32, 64, 128, 256):
        for bits in (2, 3, 4):
            cb = fa.tq_codebook(d, bits)
            ref, _ = oracle.beta_codebook(d, bits)
            assert np.abs(cb.astype(np.float64) - ref).max() < 1e-7 * np.abs(ref).max()


@pytest.mark.parametrize("d,bits,code", [(96, 4, -2), (64, 5, -2), (64, 1, -2), (512, 2, -2)])
def test_tq_rejects_unsupported_shapes(L, d, bits, code):
    import numpy as np
    out = np.zeros(16, np.float32)
    assert L.fa_tq_codebook(d, bits, ctypes.c_void_p(out.ctypes.data)) == code
    vp = ctypes.c_void_p
    assert L.fa_tq_encode(vp(1 << 20), 0, 4, d, bits, vp(1 << 20), vp(out.ctypes.data), vp(1 << 20), vp(1 << 20), None) == code


def test_tq_rejects_bad_codebook_and_pointers(L):
    import numpy as np
    vp = ctypes.c_void_p
    bad = np.array([0.0, 0.0, 1.0, 2.0], np.float32)
    good = fa.tq_codebook(64, 2)
    assert L.fa_tq_encode(vp(1 << 20), 0, 4, 64, 2, vp(1 << 20), vp(bad.ctypes.data), vp(1 << 20), vp(1 << 20), None) == -1
    assert L.fa_tq_encode(vp(0), 0, 4, 64, 2, vp(1 << 20), vp(good.ctypes.data), vp(1 << 20), vp(1 << 20), None) == -1
    # encode decides through the codebook's antisymmetry, so a shifted codebook is refused
    shifted = (good + np.float32(0.01)).astype(np.float32)
    assert L.fa_tq_encode(vp(1 << 20), 0, 4, 64, 2, vp(1 << 20), vp(shifted.ctypes.data), vp(1 << 20), vp(1 << 20), None) == -1
    assert "antisymmetric" in fa.last_error()
    for d in (32, 64, 128, 256):
        for bits in (2, 3, 4):
            cb = fa.tq_codebook(d, bits)
            assert np.array_equal(cb, -cb[::-1]), "the host codebook is not exactly antisymmetric"
    assert L.fa_tq_encode(vp(0), 0, 0, 64, 2, vp(0), vp(good.ctypes.data), vp(0), vp(0), None) == 0
    assert L.fa_tq_decode(vp(1 << 20), vp(1 << 20), 4, 64, 2, vp(1 << 20), vp(good.ctypes.data), vp(1 << 20), 2, None) == -2


@pytest.mark.parametrize("case", ["fwd_out_shape", "fwd_scale_dtype", "fwd_scale_shape", "fwd_scale_missing",
                                  "dec_out_shape", "dec_scale_dtype", "tqd_norms_rows", "tqd_out_shape",
                                  "tqe_codes_shape", "tqe_norms_dtype", "tqe_bits", "merge_out_shape"])
def test_python_layer_checks_caller_buffers_before_any_launch(case):
    """Undersized or wrongly typed caller buffers are refused with ValueError by the binding;
    the messages name the offending buffer, so these fire before the device check that CPU
    tensors would otherwise hit."""
    torch = pytest.importorskip("torch")
    z = torch.zeros
    q, k, v = z(4, 8, 64), z(2, 16, 64), z(2, 16, 64)
    k8, v8 = z(2, 16, 64, dtype=torch.int8), z(2, 16, 64, dtype=torch.int8)
    ks, vs = z(2, 16), z(2, 16)
    q1 = z(4, 1, 64)
    signs = torch.ones(64, dtype=torch.int8)
    calls = {
        "fwd_out_shape": (lambda: fa.flash_attention(q, k, v, out=z(4, 7, 64)), "out must have shape"),
        "fwd_scale_dtype": (lambda: fa.flash_attention(q, k8, v8, k_scale=ks.double(), v_scale=vs), "k_scale must be"),
        "fwd_scale_shape": (lambda: fa.flash_attention(q, k8, v8, k_scale=z(2, 15), v_scale=vs), "k_scale must have shape"),
        "fwd_scale_missing": (lambda: fa.flash_attention(q, k8, v8), "need k_scale"),
        "dec_out_shape": (lambda: fa.decode(q1, k8, v8, ks, vs, out=z(4, 2, 64)), "out must have shape"),
        "dec_scale_dtype": (lambda: fa.decode(q1, k8, v8, ks, vs.half()), "v_scale must be"),
        "tqd_norms_rows": (lambda: fa.tq_decode(z(5, 32, dtype=torch.uint8), z(4), signs, 4, [0.0] * 16), "norms must have shape"),
        "tqd_out_shape": (lambda: fa.tq_decode(z(5, 32, dtype=torch.uint8), z(5), signs, 4, [0.0] * 16, out=z(4, 64)), "out must have shape"),
        "tqe_codes_shape": (lambda: fa.tq_encode(z(5, 64), signs, 4, [0.0] * 16, codes=z(5, 16, dtype=torch.uint8)), "codes must have shape"),
        "tqe_norms_dtype": (lambda: fa.tq_encode(z(5, 64), signs, 4, [0.0] * 16, norms=z(5, dtype=torch.float64)), "norms must be"),
        "tqe_bits": (lambda: fa.tq_encode(z(5, 64), signs, 5, [0.0] * 32), "bits must be"),
        "merge_out_shape": (lambda: fa.merge_lse(z(3, 10, 64), z(3, 10), out=z(9, 64)), "out must have the shape"),
    }
    fn, msg = calls[case]
    with pytest.raises(ValueError, match=msg):
        fn()


def test_python_layer_checks_devices():
    torch = pytest.importorskip("torch")
    q, k, v = torch.zeros(4, 8, 64), torch.zeros(2, 16, 64), torch.zeros(2, 16, 64, device="meta")
    with pytest.raises(ValueError, match="v is on meta"):
        fa.flash_attention(q, k, v)


def test_append_rope_arguments_checked_on_host(L):
    vp = ctypes.c_void_p
    p = vp(1 << 20)
    # only one of the two tables
    assert L.fa_append_kv_rope(p, p, 0, 4, 1, 128, p, 100, p, None, p, p, p, p, None) == -1
    # misaligned table
    assert L.fa_append_kv_rope(p, p, 0, 4, 1, 128, p, 100, vp((1 << 20) + 4), p, p, p, p, p, None) == -1
    assert L.fa_append_kv_rope(p, p, 0, 4, 0, 128, p, 100, p, p, p, p, p, p, None) == 0   # no tokens: no-op


def test_tq_attention_code_widths_checked_on_host(L):
    """2-, 3- and 4-bit K and V codes pass the host checks (here stopped by the missing workspace,
    before any HIP call); other widths and head dims are refused as unsupported."""
    import numpy as np
    vp = ctypes.c_void_p
    p = vp(1 << 20)
    books = {b: np.linspace(-1.0, 1.0, 1 << b).astype(np.float32) for b in (1, 2, 3, 4, 5)}

    def call(kb, vb, d=128):
        return L.fa_tq_attention_decode(p, 1, p, p, p, kb, vp(books[kb].ctypes.data), p, p, p, vb,
                                        vp(books[vb].ctypes.data), p, 0, None, 8, 2, 100, d, 0.0, 0, 0, None, 0,
                                        None, 0, None)

    for kb in (2, 3, 4):
        for vb in (2, 3, 4):
            assert call(kb, vb) == -3 and "workspace" in fa.last_error(), (kb, vb)
            assert call(kb, vb, d=64) == -3
    for kb, vb in ((5, 3), (3, 1), (1, 2), (3, 5)):
        assert call(kb, vb) == -2 and "2-, 3- or 4-bit" in fa.last_error()
    assert call(3, 3, d=96) == -2 and "head_dim" in fa.last_error()
