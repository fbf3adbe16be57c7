"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and bench.py.

This module draws random numbers and rounds them to the storage dtypes the
workloads name; it contains none of the attention or quantization arithmetic.
Both the CPU oracle and the HIP path consume exactly the arrays produced here.

Workloads (the five configurations the measurements and parity tests use):

  c1  causal fp32 self-attention, bh=2, s_q=s_k=128, d=64
  c2  ragged non-causal fp32, bh=8, s_q=33, s_k=127, d=32 (+ epilogue x*2.0+0.5)
  c3  int8-KV causal prefill, batch 4 x 32 heads, s=4096, d=128; Q bf16, K/V fp32
      (to be compressed per token), bf16 output
  c4  GQA decode, batch 16, 32 query / 8 KV heads, s_q=1, s_k=32768, d=128;
      Q bf16, K/V fp32 (to be compressed per token), fp32 output
  c5  GQA causal prefill bf16, batch 1, 64 query / 8 KV heads, s=32768, d=128;
      run with no window and with a 4096-token window

Recipe: config cN uses numpy Generator(PCG64(N)) and draws Q, then K, then V
as float32 standard normals in (batch*heads, seq, head_dim) layout.  Where the
workload says bf16, the float32 draw is rounded to bf16 (round to nearest even)
and both sides consume the rounded values.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Workload", "WORKLOADS", "draw_qkv", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "round_bf16", "rng_normal", "random_signs", "score_profile",
           "decode_profile_inputs"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    bh_q: int
    bh_kv: int
    s_q: int
    s_k: int
    d: int
    causal: bool
    window: int          # 0 = no band
    q_dtype: str         # "f32" | "bf16"
    kv_dtype: str        # "f32" | "bf16" | "i8" (i8: drawn as f32, compressed by the library)
    out_dtype: str       # "f32" | "bf16"

    @property
    def group(self) -> int:
        return self.bh_q // self.bh_kv


WORKLOADS = {
    "c1": Workload("c1_causal_f32_bh2_s128_d64", 1, 2, 2, 128, 128, 64, True, 0, "f32", "f32", "f32"),
    "c2": Workload("c2_ragged_f32_bh8_sq33_sk127_d32", 2, 8, 8, 33, 127, 32, False, 0, "f32", "f32", "f32"),
    "c3": Workload("c3_int8kv_causal_b4h32_s4096_d128", 3, 128, 128, 4096, 4096, 128, True, 0, "bf16", "i8", "bf16"),
    "c4": Workload("c4_gqa_decode_b16_h32kv8_sk32768_d128", 4, 512, 128, 1, 32768, 128, False, 0, "bf16", "i8", "f32"),
    "c5": Workload("c5_gqa_causal_bf16_h64kv8_s32768_d128", 5, 64, 8, 32768, 32768, 128, True, 0, "bf16", "bf16", "bf16"),
    "c5w": Workload("c5w_gqa_window4096_bf16_h64kv8_s32768_d128", 5, 64, 8, 32768, 32768, 128, True, 4096, "bf16", "bf16", "bf16"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values stay below 0xFF800000, so the rounding increment cannot wrap in uint32
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly representable in bfloat16 (RNE of x)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def rng_normal(seed: int, *shapes):
    """Standard-normal float32 arrays drawn in order from Generator(PCG64(seed))."""
    g = np.random.Generator(np.random.PCG64(seed))
    return [g.standard_normal(size=s, dtype=np.float32) for s in shapes]


def draw_qkv(w: Workload, bh_kv: int | None = None, s_q: int | None = None,
             s_k: int | None = None, seed: int | None = None):
    """Q, K, V float32 arrays for a workload (Q rounded to bf16 values when q_dtype is bf16,
    K/V rounded when kv_dtype is bf16).  bh_kv / s_q / s_k / seed may change the draw for
    reduced cases; the draw order (Q, then K, then V) is fixed."""
    bh_kv = w.bh_kv if bh_kv is None else bh_kv
    s_q = w.s_q if s_q is None else s_q
    s_k = w.s_k if s_k is None else s_k
    seed = w.seed if seed is None else seed
    bh_q = bh_kv * w.group
    q, k, v = rng_normal(seed, (bh_q, s_q, w.d), (bh_kv, s_k, w.d), (bh_kv, s_k, w.d))
    if w.q_dtype == "bf16":
        q = round_bf16(q)
    if w.kv_dtype == "bf16":
        k = round_bf16(k)
        v = round_bf16(v)
    return q, k, v


def random_signs(seed: int, n: int) -> np.ndarray:
    """n independent fair +-1 signs (int8) from PCG64(seed): the random diagonal the TurboQuant
    rotation draws, passed to both the oracle and the library as an input."""
    g = np.random.Generator(np.random.PCG64(seed))
    return np.where(g.random(n) < 0.5, -1, 1).astype(np.int8)


def score_profile(kind: str, s_k: int) -> np.ndarray:
    """Per-key offsets a_j (in nats) that decode_profile_inputs adds to the scores of a cache:
      "sink12", "sink16"  key 0 sits 12 / 16 nats above the rest (an attention sink);
      "rising"            the offset climbs linearly from 0 to 30 nats over the cache (recency);
      "step"              0 for the first third, 7 octaves (7 ln 2 nats) for the second, and
                          20 nats more for the last third.
      "flat"              all zero."""
    a = np.zeros(s_k, np.float64)
    if kind in ("sink12", "sink16"):
        a[0] = float(kind[4:])
    elif kind == "rising":
        a = np.linspace(0.0, 30.0, s_k)
    elif kind == "step":
        a[s_k // 3:] = 7.0 * np.log(2.0)
        a[2 * s_k // 3:] += 20.0
    elif kind != "flat":
        raise ValueError(kind)
    return a


def decode_profile_inputs(seed: int, bh_kv: int, group: int, s_k: int, d: int, kind: str, v_mean: float = 0.5):
    """Decode inputs whose scores follow a profile: the query heads of a KV head share a random
    direction w (q_h = w + 0.25 z_h, rounded to bf16) and key j is z_j + a_j sqrt(d) w / |w|^2, so
    its score q_h . k_j / sqrt(d) is about a_j plus a unit-variance term.  V has channel mean
    v_mean.  Returns q (bh_kv*group, 1, d) bf16-valued float32, k and v (bh_kv, s_k, d) float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    a = score_profile(kind, s_k)
    w = g.standard_normal(size=(bh_kv, d), dtype=np.float32)
    zq = g.standard_normal(size=(bh_kv, group, d), dtype=np.float32)
    q = round_bf16((w[:, None, :] + np.float32(0.25) * zq).reshape(bh_kv * group, 1, d))
    k = g.standard_normal(size=(bh_kv, s_k, d), dtype=np.float32)
    dirn = (np.sqrt(d) * w / (w * w).sum(axis=1, keepdims=True)).astype(np.float32)
    k += (a[None, :, None] * dirn[:, None, :]).astype(np.float32)
    v = g.standard_normal(size=(bh_kv, s_k, d), dtype=np.float32) + np.float32(v_mean)
    return q, k, v
