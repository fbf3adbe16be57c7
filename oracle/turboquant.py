"""TurboQuant KV-cache codec reference, fp64 numpy (test infrastructure only).

Foundry attention/ README, section "TurboQuant KV Cache Compression": each K or V
vector is rotated by a randomized Hadamard transform (random signs applied first,
then the Hadamard transform), normalised by its L2 norm, quantized coordinate by
coordinate with a Lloyd-Max scalar quantizer designed for the Beta(d/2, d/2)
coordinate distribution, at 2 to 4 bits per channel, and bit-packed.  The
default K4/V2 is 9.14x smaller than fp32; quality is quoted as an attention-output
cosine of about 0.94 (K4/V2, synthetic) and 0.99 (K4/V4).

Readings where the page is silent (its spec is not on the pages):

* Rotation: y = H (s * x) / sqrt(d), H the Sylvester Hadamard matrix (entries +-1),
  s a random +-1 vector given as an input; d must be a power of two.  The inverse
  is x = s * (H y) / sqrt(d) (H H = d I).
* Normalisation: n = ||x||_2 (= ||y||_2), stored as fp32 per vector; u = y / n.
* Coordinate model: (u + 1) / 2 ~ Beta(d/2, d/2), as the page states.
* Codebook: the Lloyd-Max quantizer of that law with 2^b levels: each centroid is
  the conditional mean of its cell, each threshold the midpoint of its two
  centroids (iterated to convergence).  A coordinate exactly on a threshold takes
  the upper cell.
* Decode: x_hat = s * H (n * c[code]) / sqrt(d) (no renormalisation).
* Packing: the codes of a vector form one little-endian bit stream, channel i's
  b-bit code at bits i b .. i b + b - 1 (bit k of the stream is bit k mod 8 of
  byte k // 8); b in {2, 3, 4}, the page's "2-4 bits per channel" (a 3-bit code
  may straddle two bytes).
* An all-zero vector has n = 0 and decodes to 0 whatever its codes.
"""
from __future__ import annotations

import numpy as np
from scipy import special

__all__ = ["hadamard", "beta_codebook", "tq_encode", "tq_decode", "tq_pack", "tq_unpack",
           "tq_compression_ratio", "tq_attention_decode"]


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1, by doubling."""
    if d < 1 or d & (d - 1):
        raise ValueError("the Hadamard rotation needs a power-of-two head_dim")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def _cell_mass_and_moment(a, lo, hi):
    """P(lo <= u < hi) and E[u ; lo <= u < hi] for u = 2B - 1, B ~ Beta(a, a)."""
    xl, xh = (np.asarray(lo) + 1) / 2, (np.asarray(hi) + 1) / 2
    p = special.betainc(a, a, xh) - special.betainc(a, a, xl)
    eb = 0.5 * (special.betainc(a + 1, a, xh) - special.betainc(a + 1, a, xl))   # E[B; cell], mean a/(2a)
    return p, 2 * eb - p


def beta_codebook(d: int, bits: int, iters: int = 20000, tol: float = 1e-15):
    """Lloyd-Max centroids (ascending, fp64) and thresholds for the Beta(d/2, d/2) coordinate law."""
    a = d / 2.0
    n = 1 << bits
    # start from the cell means of equal-probability cells
    edges = 2 * special.betaincinv(a, a, np.linspace(0, 1, n + 1)) - 1
    edges[0], edges[-1] = -1.0, 1.0
    p, m = _cell_mass_and_moment(a, edges[:-1], edges[1:])
    c = m / p
    for _ in range(iters):
        t = (c[:-1] + c[1:]) / 2
        e = np.concatenate([[-1.0], t, [1.0]])
        p, m = _cell_mass_and_moment(a, e[:-1], e[1:])
        c_new = m / p
        done = np.max(np.abs(c_new - c)) < tol
        c = c_new
        if done:
            break
    c = (c - c[::-1]) / 2          # the law is symmetric, so is its codebook: remove iteration round-off
    return c, (c[:-1] + c[1:]) / 2


def tq_encode(x, signs, bits: int, codebook=None):
    """x: (..., d) real.  Returns (codes uint8 (..., d) unpacked, norms float32 (...))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = hadamard(d)
    c, t = codebook if codebook is not None else beta_codebook(d, bits)
    y = (x * np.asarray(signs, np.float64)) @ h.T / np.sqrt(d)
    n = np.sqrt(np.sum(x * x, axis=-1))
    u = y / np.where(n > 0, n, 1.0)[..., None]
    codes = np.searchsorted(t, u, side="right").astype(np.uint8)
    return codes, n.astype(np.float32)


def tq_decode(codes, norms, signs, bits: int, codebook=None):
    """Inverse of tq_encode up to quantization: fp64 (..., d)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    h = hadamard(d)
    c, _ = codebook if codebook is not None else beta_codebook(d, bits)
    y = np.asarray(norms, np.float64)[..., None] * c[codes]
    return np.asarray(signs, np.float64) * (y @ h.T) / np.sqrt(d)


def tq_pack(codes, bits: int) -> np.ndarray:
    """Pack b-bit codes (..., d) into (..., d b / 8) bytes: one little-endian bit stream per
    vector, channel i's code at stream bits i b .. i b + b - 1."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    if (d * bits) % 8:
        raise ValueError("d * bits must be a whole number of bytes")
    planes = (codes[..., None] >> np.arange(bits, dtype=np.uint8)) & 1        # (..., d, bits), LSB first
    stream = planes.reshape(codes.shape[:-1] + (d * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def tq_unpack(packed, bits: int, d: int) -> np.ndarray:
    """Inverse of tq_pack: (..., d b / 8) bytes -> (..., d) codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(packed, axis=-1, bitorder="little")[..., :d * bits]
    planes = stream.reshape(packed.shape[:-1] + (d, bits)).astype(np.uint8)
    return (planes << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


def tq_compression_ratio(d: int, k_bits: int, v_bits: int) -> float:
    """fp32 K + V bytes of a token over its packed codes plus one fp32 norm each."""
    return (2 * 4 * d) / (d * k_bits / 8 + d * v_bits / 8 + 8)


def tq_attention_decode(q, k_packed, k_norms, k_signs, k_bits: int, v_packed, v_norms, v_signs, v_bits: int, *,
                        k_codebook=None, v_codebook=None, window: int = 0, scale=None, epilogue=(),
                        score_epilogue=()):
    """Decode attention over a KV cache held as TurboQuant codes: the plain definition, i.e. the
    vectors tq_decode reconstructs from the packed codes and norms, attended by the fp64 decode
    (Foundry attention/ README, TurboQuant section: the coded cache stands in for K and V).
    q (bh_q, 1, d); packed codes (bh_kv, s_k, d bits / 8); norms (bh_kv, s_k); codebooks are the
    centroid arrays (default: beta_codebook).  score_epilogue acts on the scores against the
    decoded keys, as in oracle.decode.  Returns (out, lse) as oracle.decode does."""
    from .attention import decode
    kp = np.asarray(k_packed)
    vp = np.asarray(v_packed)
    d = np.asarray(q).shape[-1]
    kcb = None if k_codebook is None else (np.asarray(k_codebook, np.float64), None)
    vcb = None if v_codebook is None else (np.asarray(v_codebook, np.float64), None)
    kh = tq_decode(tq_unpack(kp, k_bits, d), k_norms, k_signs, k_bits, kcb)
    vh = tq_decode(tq_unpack(vp, v_bits, d), v_norms, v_signs, v_bits, vcb)
    return decode(q, kh, vh, window=window, scale=scale, epilogue=epilogue, score_epilogue=score_epilogue)
