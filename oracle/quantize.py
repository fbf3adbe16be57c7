"""Per-token int8 quantizer reference, numpy float32 (test infrastructure only).

fkl.flash_attention PR ("FA-2 forward with fused epilogue + compressed int8 KV
cache"), Summary: compress_kv() quantizes each token to int8 with one fp32
scale per token, for a bounded (~1e-3) error.  The page gives neither the
scale rule, the rounding nor the clamp; readings used here:

* Symmetric absmax scaling, the plainest reading of a single fp32 scale for
  each token: the token's largest magnitude maps to code 127,
  s = fp32(absmax) / fp32(127), one IEEE fp32 division.
* q = rint(x / s) with the IEEE fp32 quotient (not a reciprocal product),
  rounding half to even, clamped to [-127, 127]; -128 is never produced.
* An all-zero token gets s = 0 and q = 0 (no division by zero).

Computed in float32 on purpose: the quantized codes are an integer decision
taken in fp32, the precision the library takes it in, so both sides can agree
bit for bit.

compression_ratio: fkl PR, Verification (the KV compression-ratio check,
3.76x at head_dim 64 against a 3.5x threshold) -- bytes of an fp32 token (4d)
over bytes of its int8 codes plus the fp32 scale (d + 4).

rope_rotate_half: FlashRT QKV Cache RoPE, the decode K write that applies
rotate-half RoPE from half-width cos/sin vectors before writing the cache slot
selected by a device position.  Channel i < d/2 pairs with channel i + d/2:
out_i = x_i cos_i - x_{i+d/2} sin_i, out_{i+d/2} = x_{i+d/2} cos_i + x_i sin_i,
each product and the sum rounded to fp32 on its own (the precision the cache
write takes it in, so that the quantized codes can agree bit for bit).
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_per_token", "compression_ratio", "append_kv", "rope_rotate_half"]


def quantize_per_token(x) -> tuple[np.ndarray, np.ndarray]:
    """x: float array (..., d) (float32 or values exactly representable in it).
    Returns (codes int8 (..., d), scales float32 (...))."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)                          # exact in fp32
    s = (a / np.float32(127.0)).astype(np.float32)          # IEEE fp32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.rint(x / safe[..., None])                     # fp32 quotient, half-to-even
    r = np.clip(r, -127, 127)
    r = np.where((s > 0)[..., None], r, 0.0)
    return r.astype(np.int8), s.astype(np.float32)


def compression_ratio(head_dim: int, src_bytes_per_elem: int = 4) -> float:
    """Bytes of an uncompressed token over bytes of its int8 codes + one fp32 scale."""
    return (src_bytes_per_elem * head_dim) / (head_dim + 4)


def rope_rotate_half(x, cos, sin):
    """Rotate-half RoPE of rows x (..., d) in fp32 with half-width cos, sin (..., d/2)."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(np.float32)


def append_kv(k_cache, v_cache, k_scale, v_scale, k_new, v_new, pos, rope_cos=None, rope_sin=None):
    """Decode-time cache write, on copies of the caches: token j of KV head b (of k_new and
    v_new, (bh_kv, n_new, d)) is quantized as above and stored at row pos[b] + j of its head;
    rows outside [0, capacity) are skipped.  The pages keep the compressed cache for long-context
    decode (fkl PR, Summary); placing each new token at its position is the plain reading.
    With rope_cos, rope_sin ((capacity, d/2), row p for cache position p), K is rotated by
    rope_rotate_half at its position before it is quantized; V is not (FlashRT QKV Cache RoPE,
    the decode K write).  Returns (k_cache, v_cache, k_scale, v_scale) as new arrays."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks, vs = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    cap = kc.shape[1]
    for b in range(k_new.shape[0]):
        for j in range(k_new.shape[1]):
            p = int(pos[b]) + j
            if not 0 <= p < cap:
                continue
            krow = np.asarray(k_new[b, j], dtype=np.float32)
            if rope_cos is not None:
                krow = rope_rotate_half(krow, rope_cos[p], rope_sin[p])
            for row, codes, scales in ((krow, kc, ks), (v_new[b, j], vc, vs)):
                q, s = quantize_per_token(row)
                codes[b, p] = q
                scales[b, p] = s
    return kc, vc, ks, vs
