"""fp64 reference attention (test infrastructure only).

What is computed, and where it is defined:

* Scaled dot-product attention softmax(Q K^T / sqrt(d)) V, computed the plain
  way with the whole score matrix held in memory -- Foundry attention/ README,
  section "What it is (and is not)" and the fa_attention entry of its API
  block.  The fkl.flash_attention PR ("FA-2 forward with fused epilogue +
  compressed int8 KV cache"), Summary, presents its FA-2 kernel as an exact
  forward of this same function, so the oracle is the plain definition, not
  the tiled method.
* Causal flag and ragged s_q != s_k shapes -- fkl PR, Summary example and the
  Verification table (the d32 case with 33 queries and 127 keys).  Reading:
  causal alignment is bottom-right, key j is visible to query row i iff
  j <= i + (s_k - s_q); it is the only alignment under which the decode check
  of the Verification table (one query against 256 cached keys) sees the
  whole cache.
* Sliding-window band -- SKaiNET PR #419, Summary (the fused kernel also
  serves sliding-window layers and masks through its loop bounds).  Reading:
  a window of W keys includes the diagonal, visible iff i' - W < j <= i',
  defined only together with causal.
* GQA head groups -- SKaiNET PR #419, Summary (one task per head or per GQA
  group).  Reading: contiguous groups, query head h uses KV head h // G in the
  flat (batch*heads) layout, G = bh_q / bh_kv.
* A row with no visible key (not reachable by the workloads) -> output 0,
  LSE = -inf.  (The SKaiNET engine gives a uniform softmax for an empty band;
  this library returns zeros instead, stated as a reading.)
* The epilogue list runs on the attention output, in list order, after the
  softmax normalisation -- fkl PR, Summary (epilogue=[Mul(2.0), Add(0.5)],
  applied to the attention output inside the kernel).
* Merging results over disjoint key sets (merge_lse): the partial running states
  reduced into one -- kernbench2 ADR-0060 commit (split decode / ring prefill
  with a reduce of the running (m, l, O) states); written here in the plain
  log-sum-exp form: LSE = log sum_p exp(LSE_p), O = sum_p exp(LSE_p - LSE) O_p.
* int8 K/V enter as their dequantized values q * s (one fp32 scale per token)
  -- fkl PR, Summary (compress_kv) and the Verification row that compares the
  int8-KV kernel with an oracle fed the dequantized cache.
* Score-scope ops (score_epilogue) -- kernbench2 commit page, the tl.composite()
  epilogue list whose ops each carry a scope: a k_tile op runs on every K tile
  right after its GEMM, an output_tile op once on the finished tile.  Reading for
  attention: the K-tile GEMM is the score product, so a score-scope op acts on
  the raw score x_ij = q_i . k_j of every key (K dequantized, the built-in
  k_tile dequant of that page's example), in list order, before the softmax
  scale and the mask: s_ij = sigma * f(x_ij).  A bias op adds vec[j], j the key
  position in [0, s_k); the epilogue list above is the output_tile scope.
"""
from __future__ import annotations

import numpy as np

__all__ = ["dequantize", "visible_mask", "attention", "apply_epilogue", "decode", "merge_lse"]

ROW_BLOCK = 256  # rows of the score matrix materialised at once (memory bound only)


def dequantize(q_int8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Dequantized fp64 values q * s of a per-token int8 tensor (..., s, d) with scales (..., s).

    fkl PR, Summary: one fp32 scale per token.  No re-rounding: the products are exact in fp64.
    """
    return q_int8.astype(np.float64) * scale.astype(np.float64)[..., None]


def visible_mask(s_q: int, s_k: int, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean (s_q, s_k) matrix: True where query row i may attend to key j.

    Bottom-right causal alignment (i' = i + s_k - s_q) and a window of `window`
    keys that includes the diagonal; see the module docstring for the readings.
    """
    if window and not causal:
        raise ValueError("a window band is defined only together with causal masking")
    i_abs = np.arange(s_q)[:, None] + (s_k - s_q)
    j = np.arange(s_k)[None, :]
    vis = np.ones((s_q, s_k), dtype=bool)
    if causal:
        vis &= j <= i_abs
    if window:
        vis &= j > i_abs - window
    return vis


def apply_epilogue(x: np.ndarray, ops) -> np.ndarray:
    """Apply the post-ops in list order, in fp64.  ops: iterable of (kind, value) with kind
    "mul" / "add" (scalar value), "bias" (value: a vector over the last axis -- the head dim of
    an output row, the key position of a score row) or "relu" (value ignored; x > 0 ? x : 0).

    fkl PR, Summary: epilogue=[fkl.Mul(2.0), fkl.Add(0.5)] scales then shifts the output, and
    any compute op may be chained; kernbench2 commit page (the tl.composite epilogue list):
    bias, relu and scale ops applied in order to an output tile.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    for kind, val in ops:
        if kind == "mul":
            y = y * float(val)
        elif kind == "add":
            y = y + float(val)
        elif kind == "bias":
            b = np.asarray(val, dtype=np.float64)
            if b.shape != y.shape[-1:]:
                raise ValueError("a bias vector has one value per element of the last axis")
            y = y + b
        elif kind == "relu":
            y = np.where(y > 0, y, 0.0)
        else:
            raise ValueError(f"unknown epilogue op {kind!r}")
    return y


def attention(q, k, v, *, causal: bool, window: int = 0, scale: float | None = None,
              epilogue=(), k_scale=None, v_scale=None, heads=None, rows=None, score_epilogue=()):
    """Exact attention in fp64.

    q: (bh_q, s_q, d); k, v: (bh_kv, s_k, d), any real dtype (int8 when k_scale/v_scale given).
    k_scale, v_scale: (bh_kv, s_k) per-token scales for int8 K/V, or None.
    heads: optional iterable of query-head indices to compute (others left as NaN).
    rows: optional iterable of query-row indices to compute (others left as NaN).
    score_epilogue: ops applied to the raw scores q.k before the softmax scale (bias: a vector
    over the s_k keys); epilogue: ops applied to the normalised output rows.
    Returns (out (bh_q, s_q, d) fp64, lse (bh_q, s_q) fp64 natural-log log-sum-exp of the
    scaled scores over visible keys).
    """
    q = np.asarray(q)
    bh_q, s_q, d = q.shape
    bh_kv, s_k, dk = np.asarray(k).shape
    if dk != d or np.asarray(v).shape != (bh_kv, s_k, d):
        raise ValueError("shape mismatch")
    if bh_q % bh_kv:
        raise ValueError("bh_q must be a multiple of bh_kv")
    group = bh_q // bh_kv
    sm = 1.0 / np.sqrt(d) if scale is None else float(scale)
    heads = range(bh_q) if heads is None else list(heads)
    rows = np.arange(s_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    mask_full = visible_mask(s_q, s_k, causal, window)

    out = np.full((bh_q, s_q, d), np.nan)
    lse = np.full((bh_q, s_q), np.nan)
    kv_cache = {}
    for h in heads:
        kvh = h // group
        if kvh not in kv_cache:
            kv_cache.clear()
            if k_scale is not None:
                kh = dequantize(np.asarray(k)[kvh], np.asarray(k_scale)[kvh])
                vh = dequantize(np.asarray(v)[kvh], np.asarray(v_scale)[kvh])
            else:
                kh = np.asarray(k)[kvh].astype(np.float64)
                vh = np.asarray(v)[kvh].astype(np.float64)
            kv_cache[kvh] = (kh, vh)
        kh, vh = kv_cache[kvh]
        qh = q[h].astype(np.float64)
        for r0 in range(0, len(rows), ROW_BLOCK):
            rr = rows[r0:r0 + ROW_BLOCK]
            s = apply_epilogue(qh[rr] @ kh.T, score_epilogue) * sm   # full score rows
            vis = mask_full[rr]
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            empty = ~vis.any(axis=1)
            mx[empty] = 0.0
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            den_safe = np.where(den > 0, den, 1.0)
            o = (p / den_safe) @ vh
            o[empty] = 0.0
            l = (mx[:, 0] + np.log(den_safe[:, 0]))
            l[empty] = -np.inf
            out[h, rr] = apply_epilogue(o, epilogue)
            lse[h, rr] = l
    return out, lse


def decode(q, k, v, *, window: int = 0, scale: float | None = None, epilogue=(),
           k_scale=None, v_scale=None, heads=None, score_epilogue=()):
    """One decode step: each query head has a single row (s_q = 1) that sees every cached key
    (bottom-right alignment), optionally limited to the last `window` keys.

    fkl PR, Verification: the decode check, one query row against an int8 cache of 256 keys.
    """
    q = np.asarray(q)
    if q.ndim != 3 or q.shape[1] != 1:
        raise ValueError("decode expects q of shape (bh_q, 1, d)")
    return attention(q, k, v, causal=True, window=window, scale=scale, epilogue=epilogue,
                     k_scale=k_scale, v_scale=v_scale, heads=heads, score_epilogue=score_epilogue)


def merge_lse(o_parts, lse_parts, epilogue=()):
    """Attention over the union of disjoint key sets from per-set results, in fp64.

    o_parts: (n_parts, ..., d) normalised outputs; lse_parts: (n_parts, ...) natural-log
    log-sum-exps (-inf where a set has no visible key).  Softmax over the union weights set p by
    its share of the total exponential mass, exp(LSE_p) / sum_q exp(LSE_q) (kernbench2 ADR-0060
    commit: reduce of the running (m, l, O) states).  A row no set covers gives 0 and -inf.
    The epilogue runs once on the merged row.  Returns (out, lse).
    """
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    m = l.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(l - m_safe[None])                          # exp(-inf) = 0 for empty sets
    tot = w.sum(axis=0)
    tot_safe = np.where(tot > 0, tot, 1.0)
    out = (w[..., None] * np.where(np.isneginf(l)[..., None], 0.0, o)).sum(axis=0) / tot_safe[..., None]
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))
    return apply_epilogue(out, epilogue), lse
