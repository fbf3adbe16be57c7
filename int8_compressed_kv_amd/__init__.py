"""Exact attention with a per-token int8 KV cache on MI355X (gfx950).

Thin Python binding over the C ABI of libfa.so (include/fa.h): arguments are
checked for shape and dtype, torch tensors are passed as device pointers with
the current HIP stream, and every step of the computation runs in the HIP
kernels.  There is no CPU path: if the library is missing or no GPU is
present, the calls raise.

    codes, scales = compress_kv(k)                       # int8 + fp32 per token
    out = flash_attention(q, k, v, causal=True)          # bf16 or fp32
    out = flash_attention(q, kc, vc, k_scale=ks, v_scale=vs, causal=True,
                          epilogue=[Mul(2.0), Add(0.5)])
    append_kv(k1, v1, pos, kc, vc, ks, vs)               # quantize new tokens into the cache
    out = decode(q1, kc, vc, ks, vs)                     # split-KV decode step
    out = merge_lse(o_parts, lse_parts)                  # attention over a union of key chunks
    cb = tq_codebook(128, 4)                             # TurboQuant: Lloyd-Max codebook (host)
    codes, norms = tq_encode(k, signs, 4, cb)            # 4-bit codes + fp32 norm per token
    k_hat = tq_decode(codes, norms, signs, 4, cb)        # back to fp32 / bf16
    out = tq_attention_decode(q1, kc, kn, ks, 4, kcb, vc, vn, vs, 2, vcb)   # decode step over codes

Layout (batch*heads, seq, head_dim), head_dim a multiple of 32 up to 256.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = ["Mul", "Add", "Bias", "ReLU", "compress_kv", "append_kv", "tq_codebook", "tq_encode", "tq_decode", "tq_attention_decode", "flash_attention", "merge_lse", "decode", "decode_workspace_bytes",
           "decode_num_splits", "decode_noalloc", "last_kernel", "last_error", "lib", "LIB_PATH", "FAError",
           "F32", "BF16", "I8"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

F32, BF16, I8 = 0, 1, 2
_EPI_MUL, _EPI_ADD, _EPI_BIAS, _EPI_RELU = 1, 2, 3, 4
_MAX_EPI = 8


class FAError(RuntimeError):
    """A non-OK status from the library; .code holds the fa_status value."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"fa error {code}: {msg}")
        self.code = code


@dataclass(frozen=True)
class Mul:
    """Epilogue op: out = out * value (fp32, applied inside the kernel)."""
    value: float


@dataclass(frozen=True)
class Add:
    """Epilogue op: out = out + value (fp32, applied inside the kernel)."""
    value: float


@dataclass(frozen=True, eq=False)
class Bias:
    """Epilogue op: out[..., c] = out[..., c] + vec[c] for a device fp32 vector of head_dim values;
    as a score op, score[j] + vec[j] for a vector of s_k values (one per key position)."""
    vec: object


@dataclass(frozen=True)
class ReLU:
    """Epilogue op: out = max(out, 0) (x > 0 ? x : +0)."""


class _EpiOp(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("value", ctypes.c_float), ("vec", ctypes.c_void_p),
                ("scope", ctypes.c_int32)]


_SCOPE_OUTPUT_TILE, _SCOPE_K_TILE = 0, 1


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by int8_compressed_kv_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m int8_compressed_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.fa_compress_kv.argtypes = [vp, i32, i64, i32, vp, vp, vp]
    L.fa_compress_kv.restype = ctypes.c_int
    L.fa_append_kv.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp]
    L.fa_append_kv.restype = ctypes.c_int
    L.fa_append_kv_rope.argtypes = [vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    L.fa_append_kv_rope.restype = ctypes.c_int
    L.fa_forward.argtypes = [vp, i32, vp, vp, i32, vp, vp, vp, i32, vp,
                             i32, i32, i32, i32, i32, f32, i32, i32, ctypes.POINTER(_EpiOp), i32, vp]
    L.fa_forward.restype = ctypes.c_int
    L.fa_tq_codebook.argtypes = [i32, i32, vp]
    L.fa_tq_codebook.restype = ctypes.c_int
    L.fa_tq_encode.argtypes = [vp, i32, i64, i32, i32, vp, vp, vp, vp, vp]
    L.fa_tq_encode.restype = ctypes.c_int
    L.fa_tq_decode.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, i32, vp]
    L.fa_tq_decode.restype = ctypes.c_int
    L.fa_merge_lse.argtypes = [vp, vp, i32, i64, i32, vp, i32, vp, ctypes.POINTER(_EpiOp), i32, vp]
    L.fa_merge_lse.restype = ctypes.c_int
    L.fa_decode_num_splits.argtypes = [i32, i32, i32, i32]
    L.fa_decode_num_splits.restype = i32
    L.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.fa_decode.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, f32, i32, i32,
                            ctypes.POINTER(_EpiOp), i32, vp, ctypes.c_size_t, vp]
    L.fa_decode.restype = ctypes.c_int
    L.fa_tq_attention_decode.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, vp,
                                         i32, i32, i32, i32, f32, i32, i32, ctypes.POINTER(_EpiOp), i32, vp,
                                         ctypes.c_size_t, vp]
    L.fa_tq_attention_decode.restype = ctypes.c_int
    L.fa_tq_attention_num_splits.argtypes = [i32, i32, i32, i32]
    L.fa_tq_attention_num_splits.restype = i32
    L.fa_tq_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.fa_tq_attention_workspace_bytes.restype = ctypes.c_size_t
    L.fa_decode_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, f32, i32, i32,
                                    ctypes.POINTER(_EpiOp), i32, vp]
    L.fa_decode_noalloc.restype = ctypes.c_int
    L.fa_decode_noalloc_max_bytes.argtypes = []
    L.fa_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_last_kernel.argtypes = []
    L.fa_last_kernel.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = i32
    _lib = L
    return L


def last_error() -> str:
    return lib().fa_last_error().decode()


def last_kernel() -> str:
    return lib().fa_last_kernel().decode()


def _check(rc: int):
    if rc != 0:
        raise FAError(rc, last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.int8:
        return I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _out_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported output dtype {dt}")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _same_device(ref, **tensors):
    """Every named tensor (None skipped) must sit on ref's device."""
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _want(t, name, shape, dtype):
    """t must have exactly this shape and dtype (a caller buffer the kernels read or write)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _epilogue(ops, head_dim=None, score_ops=(), s_k=None):
    """Op array for the C ABI: `ops` on the output rows (a Bias has head_dim values), then
    `score_ops` on the raw scores q.k before the softmax scale (a Bias has s_k values, one per
    key position)."""
    ops = list(ops or [])
    score_ops = list(score_ops or [])
    if len(ops) + len(score_ops) > _MAX_EPI:
        raise ValueError(f"at most {_MAX_EPI} epilogue ops in all")
    arr = (_EpiOp * max(1, len(ops) + len(score_ops)))()
    tagged = [(op, _SCOPE_OUTPUT_TILE, head_dim, "head_dim") for op in ops]
    tagged += [(op, _SCOPE_K_TILE, s_k, "s_k") for op in score_ops]
    for i, (op, scope, n_vec, what) in enumerate(tagged):
        if isinstance(op, Mul):
            arr[i] = _EpiOp(_EPI_MUL, float(op.value), None, scope)
        elif isinstance(op, Add):
            arr[i] = _EpiOp(_EPI_ADD, float(op.value), None, scope)
        elif isinstance(op, Bias):
            torch = _torch()
            vec = op.vec
            if not isinstance(vec, torch.Tensor) or vec.dtype != torch.float32 or vec.dim() != 1:
                raise ValueError("Bias needs a 1-D fp32 device tensor")
            if n_vec is not None and vec.numel() != n_vec:
                raise ValueError(f"Bias vector has {vec.numel()} values, {what} is {n_vec}")
            arr[i] = _EpiOp(_EPI_BIAS, 0.0, _dev(vec, "bias vector"), scope)
        elif isinstance(op, ReLU):
            arr[i] = _EpiOp(_EPI_RELU, 0.0, None, scope)
        else:
            raise TypeError(f"epilogue ops must be Mul, Add, Bias or ReLU, got {op!r}")
    return arr, len(tagged)


def compress_kv(x, out=None, scales=None):
    """Quantize (..., head_dim) fp32/bf16 rows to int8 codes with one fp32 scale per row."""
    torch = _torch()
    d = x.shape[-1]
    n = x.numel() // d if d else 0
    if out is None:
        out = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if out.dtype != torch.int8 or out.shape != x.shape:
        raise ValueError("codes output must be int8 with the input's shape")
    if scales.dtype != torch.float32 or scales.shape != x.shape[:-1]:
        raise ValueError("scales output must be fp32 with the input's leading shape")
    _same_device(x, codes=out, scales=scales)
    _check(lib().fa_compress_kv(_dev(x, "x"), _dtype_code(x), n, d, _dev(out, "codes"),
                                _dev(scales, "scales"), _stream()))
    return out, scales


def append_kv(k_new, v_new, pos, k_cache, v_cache, k_scale, v_scale, rope_cos=None, rope_sin=None):
    """Quantize new tokens k_new, v_new (bh_kv, n_new, d) fp32/bf16 into the int8 cache
    (bh_kv, capacity, d) with scales (bh_kv, capacity): token j of head b goes to row pos[b] + j,
    pos an int32 device tensor (bh_kv,).  Rows outside the cache are skipped.  With rope_cos,
    rope_sin (capacity, d/2) fp32 device tables, K rows are rotated (rotate-half RoPE at their
    cache position) before they are quantized."""
    torch = _torch()
    if k_new.dim() != 3 or tuple(v_new.shape) != tuple(k_new.shape) or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must be (bh_kv, n_new, head_dim) tensors of one dtype")
    bh_kv, n_new, d = k_new.shape
    if k_cache.dim() != 3 or k_cache.shape[0] != bh_kv or k_cache.shape[2] != d:
        raise ValueError("k_cache must be (bh_kv, capacity, head_dim)")
    cap = k_cache.shape[1]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.dtype != torch.int8 or v_cache.dtype != torch.int8:
        raise ValueError("k_cache and v_cache must be int8 tensors of one shape")
    if tuple(k_scale.shape) != (bh_kv, cap) or tuple(v_scale.shape) != (bh_kv, cap):
        raise ValueError("scales must have shape (bh_kv, capacity)")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise ValueError("scales must be fp32")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (bh_kv,):
        raise ValueError("pos must be an int32 tensor of shape (bh_kv,)")
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("give both rope_cos and rope_sin, or neither")
    if rope_cos is not None:
        if d % 2:
            raise ValueError("RoPE needs an even head_dim")
        _want(rope_cos, "rope_cos", (cap, d // 2), torch.float32)
        _want(rope_sin, "rope_sin", (cap, d // 2), torch.float32)
    _same_device(k_new, v_new=v_new, pos=pos, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
                 rope_cos=rope_cos, rope_sin=rope_sin)
    _check(lib().fa_append_kv_rope(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new), bh_kv, n_new, d,
                                   _dev(pos, "pos"), cap, _dev(rope_cos, "rope_cos"), _dev(rope_sin, "rope_sin"),
                                   _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_scale, "k_scale"),
                                   _dev(v_scale, "v_scale"), _stream()))
    return k_cache, v_cache, k_scale, v_scale


def flash_attention(q, k, v, *, causal=False, window=0, scale=None, epilogue=(), k_scale=None,
                    v_scale=None, out_dtype=None, out=None, return_lse=False, score_ops=()):
    """softmax(Q K^T * scale) V for q (bh_q, s_q, d) over k, v (bh_kv, s_k, d).

    k, v: fp32 / bf16 tensors, or int8 codes with k_scale, v_scale (bh_kv, s_k) fp32.
    epilogue: ops on the normalised output; score_ops: ops on every raw score q.k before the
    softmax scale (a Bias there holds s_k values, one per key position).
    out_dtype defaults to q's dtype.  Returns out, or (out, lse) with return_lse.
    """
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D (batch*heads, seq, head_dim)")
    bh_q, s_q, d = q.shape
    bh_kv, s_k, dk = k.shape
    if dk != d or tuple(v.shape) != (bh_kv, s_k, d):
        raise ValueError("k and v must have shape (bh_kv, s_k, head_dim) matching q's head_dim")
    if k.dtype != v.dtype:
        raise ValueError("k and v must share a dtype")
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale, or neither")
    if k_scale is not None:
        _want(k_scale, "k_scale", (bh_kv, s_k), torch.float32)
        _want(v_scale, "v_scale", (bh_kv, s_k), torch.float32)
    if (k.dtype == torch.int8) != (k_scale is not None):
        raise ValueError("int8 k, v need k_scale and v_scale; other dtypes take none")
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((bh_q, s_q, d), dtype=odt, device=q.device)
    elif tuple(out.shape) != (bh_q, s_q, d):
        raise ValueError(f"out must have shape {(bh_q, s_q, d)}, got {tuple(out.shape)}")
    _same_device(q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, out=out)
    lse = torch.empty((bh_q, s_q), dtype=torch.float32, device=q.device) if return_lse else None
    epi, n_epi = _epilogue(epilogue, d, score_ops, s_k)
    _check(lib().fa_forward(_dev(q, "q"), _dtype_code(q), _dev(k, "k"), _dev(v, "v"), _dtype_code(k),
                            _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(out, "out"),
                            _out_code(out.dtype), _dev(lse, "lse"), bh_q, bh_kv, s_q, s_k, d,
                            float(scale) if scale else 0.0, int(bool(causal)), int(window), epi, n_epi,
                            _stream()))
    return (out, lse) if return_lse else out


def tq_codebook(head_dim: int, bits: int):
    """The library's TurboQuant Lloyd-Max centroids (2^bits, ascending) as a host float32 array."""
    import numpy as np
    out = np.zeros(1 << bits, np.float32)
    _check(lib().fa_tq_codebook(int(head_dim), int(bits), ctypes.c_void_p(out.ctypes.data)))
    return out


def _host_f32(cb):
    import numpy as np
    cb = np.ascontiguousarray(np.asarray(cb, dtype=np.float32))
    return cb, ctypes.c_void_p(cb.ctypes.data)


def tq_encode(x, signs, bits, codebook, codes=None, norms=None):
    """TurboQuant codes (..., head_dim * bits / 8) uint8 and fp32 norms (...) of fp32/bf16 rows x
    (..., head_dim); signs: int8 +-1 device tensor (head_dim,); codebook: host (2^bits,) centroids."""
    torch = _torch()
    d = x.shape[-1]
    n = x.numel() // d if d else 0
    if signs.dtype != torch.int8 or tuple(signs.shape) != (d,):
        raise ValueError("signs must be an int8 tensor of shape (head_dim,)")
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    cshape = tuple(x.shape[:-1]) + (d * bits // 8,)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if norms is None:
        norms = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    _want(codes, "codes", cshape, torch.uint8)
    _want(norms, "norms", tuple(x.shape[:-1]), torch.float32)
    _same_device(x, signs=signs, codes=codes, norms=norms)
    cb, cbp = _host_f32(codebook)
    _check(lib().fa_tq_encode(_dev(x, "x"), _dtype_code(x), n, d, int(bits), _dev(signs, "signs"), cbp,
                              _dev(codes, "codes"), _dev(norms, "norms"), _stream()))
    return codes, norms


def tq_decode(codes, norms, signs, bits, codebook, out_dtype=None, out=None):
    """Rows (..., head_dim) decoded from TurboQuant codes and norms (fp32 by default)."""
    torch = _torch()
    if signs.dim() != 1 or signs.dtype != torch.int8:
        raise ValueError("signs must be an int8 tensor of shape (head_dim,)")
    if bits not in (2, 3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    d = signs.shape[0]
    if codes.dtype != torch.uint8 or codes.dim() < 1 or codes.shape[-1] != d * bits // 8:
        raise ValueError("codes must be uint8 (..., head_dim * bits / 8)")
    lead = tuple(codes.shape[:-1])
    _want(norms, "norms", lead, torch.float32)
    n = norms.numel()
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(lead + (d,), dtype=odt, device=codes.device)
    elif tuple(out.shape) != lead + (d,):
        raise ValueError(f"out must have shape {lead + (d,)}, got {tuple(out.shape)}")
    _same_device(codes, norms=norms, signs=signs, out=out)
    cb, cbp = _host_f32(codebook)
    _check(lib().fa_tq_decode(_dev(codes, "codes"), _dev(norms, "norms"), n, d, int(bits), _dev(signs, "signs"),
                              cbp, _dev(out, "out"), _out_code(out.dtype), _stream()))
    return out


def merge_lse(o_parts, lse_parts, *, epilogue=(), out_dtype=None, out=None, return_lse=False):
    """Attention over the union of disjoint key chunks from per-chunk results: o_parts
    (n_parts, ..., head_dim) fp32 normalised outputs and lse_parts (n_parts, ...) fp32
    log-sum-exps, as flash_attention(..., out_dtype=float32, return_lse=True) returns them.
    Returns out (..., head_dim), or (out, lse) with return_lse."""
    torch = _torch()
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts and lse_parts must be fp32")
    if o_parts.dim() < 2 or tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError("lse_parts must have the shape of o_parts without its last dimension")
    n_parts, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel() if n_parts else 0
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(tuple(o_parts.shape[1:]), dtype=odt, device=o_parts.device)
    if tuple(out.shape) != tuple(o_parts.shape[1:]):
        raise ValueError("out must have the shape of one part")
    _same_device(o_parts, lse_parts=lse_parts, out=out)
    lse = torch.empty(tuple(lse_parts.shape[1:]), dtype=torch.float32, device=o_parts.device) if return_lse else None
    epi, n_epi = _epilogue(epilogue, d)
    _check(lib().fa_merge_lse(_dev(o_parts, "o_parts"), _dev(lse_parts, "lse_parts"), n_parts, rows, d,
                              _dev(out, "out"), _out_code(out.dtype), _dev(lse, "lse"), epi, n_epi, _stream()))
    return (out, lse) if return_lse else out


def decode_num_splits(bh_q, bh_kv, s_k, head_dim) -> int:
    return int(lib().fa_decode_num_splits(bh_q, bh_kv, s_k, head_dim))


def decode_workspace_bytes(bh_q, bh_kv, s_k, head_dim, num_splits=0) -> int:
    return int(lib().fa_decode_workspace_bytes(bh_q, bh_kv, s_k, head_dim, num_splits))


def decode(q, k, v, k_scale, v_scale, *, window=0, scale=None, num_splits=0, epilogue=(),
           out_dtype=None, out=None, workspace=None, return_lse=False, score_ops=()):
    """One decode step: q (bh_q, 1, d) against the int8 cache k, v (bh_kv, s_k, d) with fp32
    per-token scales (bh_kv, s_k).  score_ops act on the raw scores as in flash_attention.
    Output fp32 by default."""
    torch = _torch()
    if q.dim() != 3 or q.shape[1] != 1:
        raise ValueError("q must have shape (bh_q, 1, head_dim)")
    bh_q, _, d = q.shape
    bh_kv, s_k, dk = k.shape
    if dk != d or tuple(v.shape) != (bh_kv, s_k, d):
        raise ValueError("k and v must have shape (bh_kv, s_k, head_dim)")
    if k.dtype != torch.int8 or v.dtype != torch.int8:
        raise ValueError("decode reads the int8 cache: k and v must be int8 codes")
    _want(k_scale, "k_scale", (bh_kv, s_k), torch.float32)
    _want(v_scale, "v_scale", (bh_kv, s_k), torch.float32)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((bh_q, 1, d), dtype=odt, device=q.device)
    elif tuple(out.shape) != (bh_q, 1, d):
        raise ValueError(f"out must have shape {(bh_q, 1, d)}, got {tuple(out.shape)}")
    _same_device(q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, out=out, workspace=workspace)
    need = decode_workspace_bytes(bh_q, bh_kv, s_k, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    lse = torch.empty((bh_q,), dtype=torch.float32, device=q.device) if return_lse else None
    epi, n_epi = _epilogue(epilogue, d, score_ops, s_k)
    _check(lib().fa_decode(_dev(q, "q"), _dtype_code(q), _dev(k, "k"), _dev(v, "v"), _dev(k_scale, "k_scale"),
                           _dev(v_scale, "v_scale"), _dev(out, "out"), _out_code(out.dtype), _dev(lse, "lse"),
                           bh_q, bh_kv, s_k, d, float(scale) if scale else 0.0, int(window), int(num_splits),
                           epi, n_epi, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                           _stream()))
    return (out, lse) if return_lse else out


def decode_noalloc(q, k, v, k_scale, v_scale, out, *, lse=None, window=0, scale=None, num_splits=0, epilogue=(),
                   score_ops=()):
    """decode() through fa_decode_noalloc: the partial states go to the library's fixed device
    scratch array, and nothing is allocated here either, so the caller passes `out` (bh_q, 1, d)
    (and optionally `lse` (bh_q,) fp32).  Calls that may overlap on one GPU race on that array."""
    torch = _torch()
    if q.dim() != 3 or q.shape[1] != 1:
        raise ValueError("q must have shape (bh_q, 1, head_dim)")
    bh_q, _, d = q.shape
    bh_kv, s_k, dk = k.shape
    if dk != d or tuple(v.shape) != (bh_kv, s_k, d):
        raise ValueError("k and v must have shape (bh_kv, s_k, head_dim)")
    if k.dtype != torch.int8 or v.dtype != torch.int8:
        raise ValueError("decode reads the int8 cache: k and v must be int8 codes")
    _want(k_scale, "k_scale", (bh_kv, s_k), torch.float32)
    _want(v_scale, "v_scale", (bh_kv, s_k), torch.float32)
    if tuple(out.shape) != (bh_q, 1, d):
        raise ValueError(f"out must have shape {(bh_q, 1, d)}, got {tuple(out.shape)}")
    if lse is not None:
        _want(lse, "lse", (bh_q,), torch.float32)
    _same_device(q, k=k, v=v, k_scale=k_scale, v_scale=v_scale, out=out, lse=lse)
    epi, n_epi = _epilogue(epilogue, d, score_ops, s_k)
    _check(lib().fa_decode_noalloc(_dev(q, "q"), _dtype_code(q), _dev(k, "k"), _dev(v, "v"), _dev(k_scale, "k_scale"),
                                   _dev(v_scale, "v_scale"), _dev(out, "out"), _out_code(out.dtype), _dev(lse, "lse"),
                                   bh_q, bh_kv, s_k, d, float(scale) if scale else 0.0, int(window), int(num_splits),
                                   epi, n_epi, _stream()))
    return out


def tq_attention_decode(q, k_codes, k_norms, k_signs, k_bits, k_codebook, v_codes, v_norms, v_signs, v_bits,
                        v_codebook, *, window=0, scale=None, num_splits=0, epilogue=(), out_dtype=None, out=None,
                        workspace=None, return_lse=False, score_ops=()):
    """One decode step of q (bh_q, 1, d) over a KV cache held as TurboQuant codes: k_codes
    (bh_kv, s_k, d k_bits / 8) uint8 with k_norms (bh_kv, s_k) fp32 and k_signs (d,) int8 as
    tq_encode wrote them, k_codebook the host centroids; likewise for V.  score_ops act on the
    scores n_j (q'.c[code]) before the softmax scale, as in flash_attention.  Output fp32 by default."""
    torch = _torch()
    if q.dim() != 3 or q.shape[1] != 1:
        raise ValueError("q must have shape (bh_q, 1, head_dim)")
    bh_q, _, d = q.shape
    if k_codes.dim() != 3 or v_codes.dim() != 3:
        raise ValueError("codes must be (bh_kv, s_k, head_dim * bits / 8)")
    bh_kv, s_k = k_codes.shape[0], k_codes.shape[1]
    _want(k_codes, "k_codes", (bh_kv, s_k, d * k_bits // 8), torch.uint8)
    _want(v_codes, "v_codes", (bh_kv, s_k, d * v_bits // 8), torch.uint8)
    _want(k_norms, "k_norms", (bh_kv, s_k), torch.float32)
    _want(v_norms, "v_norms", (bh_kv, s_k), torch.float32)
    _want(k_signs, "k_signs", (d,), torch.int8)
    _want(v_signs, "v_signs", (d,), torch.int8)
    odt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((bh_q, 1, d), dtype=odt, device=q.device)
    elif tuple(out.shape) != (bh_q, 1, d):
        raise ValueError(f"out must have shape {(bh_q, 1, d)}, got {tuple(out.shape)}")
    _same_device(q, k_codes=k_codes, v_codes=v_codes, k_norms=k_norms, v_norms=v_norms, k_signs=k_signs,
                 v_signs=v_signs, out=out, workspace=workspace)
    L = lib()
    need = int(L.fa_tq_attention_workspace_bytes(bh_q, bh_kv, s_k, d, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    lse = torch.empty((bh_q,), dtype=torch.float32, device=q.device) if return_lse else None
    kcb, kcbp = _host_f32(k_codebook)
    vcb, vcbp = _host_f32(v_codebook)
    epi, n_epi = _epilogue(epilogue, d, score_ops, s_k)
    _check(L.fa_tq_attention_decode(_dev(q, "q"), _dtype_code(q), _dev(k_codes, "k_codes"), _dev(k_norms, "k_norms"),
                                    _dev(k_signs, "k_signs"), int(k_bits), kcbp, _dev(v_codes, "v_codes"),
                                    _dev(v_norms, "v_norms"), _dev(v_signs, "v_signs"), int(v_bits), vcbp,
                                    _dev(out, "out"), _out_code(out.dtype), _dev(lse, "lse"), bh_q, bh_kv, s_k, d,
                                    float(scale) if scale else 0.0, int(window), int(num_splits), epi, n_epi,
                                    _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                    _stream()))
    return (out, lse) if return_lse else out
