#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: prefill TFLOP/s against the bf16 MFMA peak and int8-KV
decode GB/s against the HBM peak.

Legs (each timed separately with HIP events on the stream the kernels run on):
  c5     GQA causal prefill, bf16, batch 1, 64 query / 8 KV heads, 32768 tokens, d 128  <- `value`
  c5w    the same with a 4096-token sliding window
  c3     int8-KV causal prefill, bf16 Q, 4 x 32 heads, 4096 tokens, d 128, bf16 output
  c4     GQA split-KV decode over the int8 cache, 16 x 32 query / 8 KV heads, 32768 keys, d 128
  c4g8   the same cache with a GQA group of 8 (16 x 64 query / 8 KV heads): one workgroup serves
         all 8 query heads of a KV head, so the cache is still read once
  comp   per-token compression of the c4 K and V caches (fp32 -> int8 + fp32 scales)
  append decode-time cache write of the c4 shape: one new fp32 K and V token per KV head (128),
         quantized into the 32768-row int8 cache at device-held positions (latency-bound)
  tq     TurboQuant 4-bit encode of the c4 K cache (fp32 in) and decode of it back to bf16
  tqattn decode attention read straight from TurboQuant codes of the c4 cache (K 4-bit, V 2-bit,
         the page's default), 16 x 32 query / 8 KV heads, 32768 keys, d 128
  tqattn33 (not in the default set) the same with 3-bit K and V codes, which straddle bytes
  tqattn_g8 (not in the default set) K4/V2 with a GQA group of 8 (16 x 64 query / 8 KV heads)
  merge  log-sum-exp merge of 8 key-chunk results for one 4096-row query chunk of the c5 shape
         (64 heads x 4096 rows, d 128, fp32 parts, bf16 output): the exchange of a ring prefill
  copy   (not in the default set) a plain 1 GiB device-to-device copy, the known-size reference
         that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to HBM bytes

One JSON line on stdout; progress on stderr.  `--gpus N` with N > 1 exits: this path runs on one
GPU (a multi-GPU run would give each GPU a share of the KV heads, with their query heads, and
run the same kernels on it; no data moves between GPUs for the prefill or the decode).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = "prefill attn TFLOP/s (% MFMA peak); int8-KV decode GB/s (% HBM peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(s_q, s_k, causal, window):
    i = np.arange(s_q, dtype=np.int64) + (s_k - s_q)
    hi = np.minimum(i + 1, s_k) if causal else np.full(s_q, s_k, np.int64)
    lo = np.maximum(i - window + 1, 0) if window else np.zeros(s_q, np.int64)
    return int(np.clip(hi - lo, 0, None).sum())


# kernel sources behind each leg: a counter reading is used only while these are unchanged
LEG_SOURCES = {
    "c5": ("prefill_bf16.hip", "device_common.hpp", "kernel_args.hpp"),
    "c5w": ("prefill_bf16.hip", "device_common.hpp", "kernel_args.hpp"),
    "c3": ("prefill_i8kv.hip", "device_common.hpp", "kernel_args.hpp"),
    "c4": ("decode.hip", "device_common.hpp", "kernel_args.hpp"),
    "c4g8": ("decode.hip", "device_common.hpp", "kernel_args.hpp"),
    "comp": ("compress.hip", "device_common.hpp", "kernel_args.hpp"),
    "append": ("compress.hip", "device_common.hpp", "kernel_args.hpp"),
    "merge": ("merge.hip", "device_common.hpp", "kernel_args.hpp"),
    "tq": ("tq.hip", "device_common.hpp", "kernel_args.hpp"),
    "tq_dec": ("tq.hip", "device_common.hpp", "kernel_args.hpp"),
    "tqattn": ("tq_attn.hip", "device_common.hpp", "kernel_args.hpp"),
    "tqattn33": ("tq_attn.hip", "device_common.hpp", "kernel_args.hpp"),
    "tqattn_g8": ("tq_attn.hip", "device_common.hpp", "kernel_args.hpp"),
}


def source_sha(leg):
    h = hashlib.sha256()
    for n in LEG_SOURCES[leg]:
        with open(os.path.join(ROOT, "int8_compressed_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(leg):
    """HBM bytes per launch of the leg's kernels from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by the copy calibration), or None if they were taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f).get("legs", {}).get(leg)
    if not rec or rec.get("source_sha") != source_sha(leg):
        return None
    return rec.get("hbm_bytes_per_launch")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def shader_clock_under_load(torch, fn, seconds=2.0):
    """Median shader clock (MHz) that `rocm-smi --showclocks` reports while `fn` runs back to back
    for about `seconds` (untimed; the caller's timed steps are already done), or None when the tool
    is missing or prints no clock."""
    import re
    import shutil
    import subprocess
    import threading
    exe = shutil.which("rocm-smi")
    if exe is None:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                txt = subprocess.run([exe, "--showclocks"], capture_output=True, text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            m = re.search(r"sclk clock level:\s*\S+:?\s*\((\d+)\s*Mhz\)", txt, re.IGNORECASE)
            if m:
                samples.append(int(m.group(1)))

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.time()
    fn()
    torch.cuda.synchronize()
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    return float(np.median(samples)) if samples else None


class Timer:
    """HIP events around each call on the current stream; returns per-call milliseconds.

    `warm_s`: after the `warmup` calls, keep calling until that much wall time has passed, so a leg
    is timed at the clock the GPU settles to under it (the first tens of milliseconds of a short
    kernel run below it: about 830 us against 677 us per int8-cache prefill call on one box).  The
    headline leg uses exactly the `--warmup` calls."""

    def __init__(self, torch, warm_s=0.0):
        self.torch = torch
        self.warm_s = warm_s

    def run(self, fn, steps, warmup, flush=None, settle=True):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if settle and self.warm_s > 0:
            t0 = time.time()
            while time.time() - t0 < self.warm_s:
                for _ in range(4):
                    fn()
                torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            if flush is not None:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            times.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in times]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="c5,c5w,c3,c4,c4g8,comp,append,merge,tq,tqattn")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--settle", type=float, default=0.25,
                    help="seconds of extra untimed calls before each leg other than the headline c5 (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget per baseline")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the rocm-smi clock sampling (for runs under a profiler, whose preload would "
                         "follow the rocm-smi child process)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); this build has no "
              "multi-GPU path: the kernels would run unchanged on each GPU's share of KV heads.", file=sys.stderr)
        sys.exit(2)

    import torch
    import int8_compressed_kv_amd as fa
    from synth_inputs import WORKLOADS, draw_qkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    legs = set(args.legs.split(","))
    timer = Timer(torch, warm_s=args.settle)
    res = {}
    flush_buf = torch.zeros(512 * 1024 * 1024, dtype=torch.float32, device="cuda")   # 2 GiB > MALL
    flush_sum = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        # a read sweep over 2 GiB evicts the leg's inputs from the caches without leaving them full of
        # dirty lines, whose write-back a zero fill would charge to the timed call (about 60 us on
        # the TurboQuant encode in interleaved timings; none on the read-only decode)
        torch.sum(flush_buf, dim=0, out=flush_sum)

    def bf16_dev(x):
        return torch.from_numpy(x).to("cuda").to(torch.bfloat16)

    cpu = {}
    # ------------------------------------------------------------------ prefill legs c5 / c5w
    if legs & {"c5", "c5w"}:
        w = WORKLOADS["c5"]
        log(f"[bench] generating {w.name}")
        q, k, v = draw_qkv(w)
        qd, kd, vd = bf16_dev(q), bf16_dev(k), bf16_dev(v)
        out = torch.empty_like(qd)
        for name, window in (("c5", 0), ("c5w", 4096)):
            if name not in legs:
                continue
            ww = WORKLOADS[name]
            flops = 4.0 * w.d * visible_pairs(w.s_q, w.s_k, True, window) * w.bh_q
            fn = lambda: fa.flash_attention(qd, kd, vd, causal=True, window=window, out=out)   # noqa: E731
            log(f"[bench] timing {ww.name}")
            ms = timer.run(fn, args.steps, args.warmup, settle=name != "c5")
            avg = float(np.mean(ms))
            res[name] = {"workload": ww.name, "ms": avg, "ms_min": float(np.min(ms)),
                         "ms_median": float(np.median(ms)), "kernel": fa.last_kernel(),
                         "flop_per_launch": flops, "tflops": flops / avg / 1e9,
                         "frac_of_peak": flops / avg / 1e9 / PEAK_BF16_TFLOPS}
            log(f"[bench] {name}: {avg:.3f} ms  {res[name]['tflops']:.1f} TFLOP/s")
            if name == "c5" and not args.no_clock:
                mhz = shader_clock_under_load(torch, fn)
                res[name]["clock_mhz"] = mhz
                if mhz:
                    log(f"[bench] c5: shader clock under this load {mhz:.0f} MHz (rocm-smi)")
            if name == "c5" and not args.no_cpu:
                cpu["c5"] = prefill_cpu_baseline(q, k, v, out, w, args.cpu_seconds)
        del qd, kd, vd, out, q, k, v

    # ------------------------------------------------------------------ int8-KV prefill c3
    if "c3" in legs:
        w = WORKLOADS["c3"]
        log(f"[bench] generating {w.name}")
        q, k, v = draw_qkv(w)
        qd = bf16_dev(q)
        kc, ks = fa.compress_kv(torch.from_numpy(k).cuda())
        vc, vs = fa.compress_kv(torch.from_numpy(v).cuda())
        out = torch.empty_like(qd)
        flops = 4.0 * w.d * visible_pairs(w.s_q, w.s_k, True, 0) * w.bh_q
        fn = lambda: fa.flash_attention(qd, kc, vc, k_scale=ks, v_scale=vs, causal=True, out=out)   # noqa: E731
        log(f"[bench] timing {w.name}")
        ms = timer.run(fn, args.steps, args.warmup)
        avg = float(np.mean(ms))
        res["c3"] = {"workload": w.name, "ms": avg, "ms_min": float(np.min(ms)), "ms_median": float(np.median(ms)),
                     "kernel": fa.last_kernel(),
                     "flop_per_launch": flops, "tflops": flops / avg / 1e9,
                     "frac_of_peak": flops / avg / 1e9 / PEAK_BF16_TFLOPS}
        log(f"[bench] c3: {avg:.3f} ms  {res['c3']['tflops']:.1f} TFLOP/s")
        del qd, kc, ks, vc, vs, out, q, k, v

    # ------------------------------------------------------------------ compress + decode c4
    if legs & {"c4", "c4g8", "comp", "append", "tq", "tqattn", "tqattn33", "tqattn_g8"}:
        w = WORKLOADS["c4"]
        log(f"[bench] generating {w.name}")
        q, k, v = draw_qkv(w)
        qd = bf16_dev(q)
        kf = torch.from_numpy(k).cuda()
        vf = torch.from_numpy(v).cuda()
        kc = torch.empty(kf.shape, dtype=torch.int8, device="cuda")
        vc = torch.empty_like(kc)
        ks = torch.empty(kf.shape[:-1], dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        n_tok = w.bh_kv * w.s_k
        if "comp" in legs:
            fn = lambda: fa.compress_kv(kf, kc, ks)   # noqa: E731
            log("[bench] timing compress (c4 K cache)")
            ms = timer.run(fn, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = n_tok * w.d * 4 + n_tok * w.d + n_tok * 4
            res["comp"] = {"workload": "compress_c4_k_cache_128x32768x128_f32", "ms": avg,
                           "ms_min": float(np.min(ms)), "ms_median": float(np.median(ms)),
                           "kernel": fa.last_kernel(), "bytes_per_launch": nbytes, "gbs": nbytes / avg / 1e6,
                           "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] comp: {avg:.3f} ms  {res['comp']['gbs']:.0f} GB/s")
        if "tq" in legs:
            from synth_inputs import random_signs
            bits = 4
            cb = fa.tq_codebook(w.d, bits)
            signs = torch.from_numpy(random_signs(64, w.d)).cuda()
            codes = torch.empty((w.bh_kv, w.s_k, w.d * bits // 8), dtype=torch.uint8, device="cuda")
            norms = torch.empty((w.bh_kv, w.s_k), dtype=torch.float32, device="cuda")
            fn = lambda: fa.tq_encode(kf, signs, bits, cb, codes, norms)   # noqa: E731
            log("[bench] timing TurboQuant encode (c4 K cache, 4 bits)")
            ms = timer.run(fn, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = n_tok * (w.d * 4 + w.d * bits // 8 + 4)
            res["tq"] = {"workload": "tq4_encode_c4_k_cache_128x32768x128_f32", "ms": avg,
                         "ms_min": float(np.min(ms)), "ms_median": float(np.median(ms)),
                         "kernel": fa.last_kernel(), "bytes_per_launch": nbytes, "gbs": nbytes / avg / 1e6,
                         "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] tq encode: {avg:.3f} ms  {res['tq']['gbs']:.0f} GB/s")
            kb16 = torch.empty(kf.shape, dtype=torch.bfloat16, device="cuda")
            fn = lambda: fa.tq_decode(codes, norms, signs, bits, cb, out=kb16)   # noqa: E731
            ms = timer.run(fn, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = n_tok * (w.d * bits // 8 + 4 + w.d * 2)
            res["tq_dec"] = {"workload": "tq4_decode_c4_k_cache_128x32768x128_to_bf16", "ms": avg,
                             "ms_min": float(np.min(ms)),
                             "ms_median": float(np.median(ms)), "kernel": fa.last_kernel(), "bytes_per_launch": nbytes,
                             "gbs": nbytes / avg / 1e6, "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] tq decode: {avg:.3f} ms  {res['tq_dec']['gbs']:.0f} GB/s")
            del codes, norms, kb16, signs
        for tq_leg, kbits, vbits, grp in (("tqattn", 4, 2, 4), ("tqattn33", 3, 3, 4), ("tqattn_g8", 4, 2, 8)):
            if tq_leg not in legs:
                continue
            from synth_inputs import random_signs
            # group 8: the c4 queries twice over, 64 query heads per batch against the same cache
            q_t = qd if grp == 4 else torch.cat([qd, qd], 0)
            bh_q_t = w.bh_kv * grp
            kcb, vcb = fa.tq_codebook(w.d, kbits), fa.tq_codebook(w.d, vbits)
            sk = torch.from_numpy(random_signs(64, w.d)).cuda()
            sv = torch.from_numpy(random_signs(65, w.d)).cuda()
            kcode, kn = fa.tq_encode(kf, sk, kbits, kcb)
            vcode, vn = fa.tq_encode(vf, sv, vbits, vcb)
            out_t = torch.empty((bh_q_t, 1, w.d), dtype=torch.float32, device="cuda")
            splits_t = int(fa.lib().fa_tq_attention_num_splits(bh_q_t, w.bh_kv, w.s_k, w.d))
            ws_t = torch.empty(int(fa.lib().fa_tq_attention_workspace_bytes(bh_q_t, w.bh_kv, w.s_k, w.d, splits_t)),
                               dtype=torch.uint8, device="cuda")
            fn = lambda: fa.tq_attention_decode(q_t, kcode, kn, sk, kbits, kcb, vcode, vn, sv, vbits, vcb,   # noqa: E731
                                                num_splits=splits_t, out=out_t, workspace=ws_t)
            log(f"[bench] timing decode attention over TurboQuant codes (K{kbits}/V{vbits}, c4 cache, group {grp})")
            ms = timer.run(fn, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = n_tok * (w.d * kbits // 8 + 4 + w.d * vbits // 8 + 4) + bh_q_t * w.d * 2 + bh_q_t * w.d * 4
            res[tq_leg] = {"workload": f"tq_attention_decode_k{kbits}v{vbits}_b16_h{grp * 8}kv8_sk32768_d128",
                           "ms": avg, "ms_min": float(np.min(ms)),
                           "ms_median": float(np.median(ms)), "kernel": fa.last_kernel(), "num_splits": splits_t,
                           "bytes_per_launch": nbytes, "gbs": nbytes / avg / 1e6,
                           "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] {tq_leg}: {avg * 1e3:.1f} us  {res[tq_leg]['gbs']:.0f} GB/s")
            del kcode, kn, vcode, vn, out_t, ws_t, sk, sv, q_t
        fa.compress_kv(kf, kc, ks)
        fa.compress_kv(vf, vc, vs)
        if "append" in legs:
            # the cache's last token of every KV head written again from its fp32 values (the
            # codes written are the ones already there, so the decode leg sees the same cache)
            kn = kf[:, -1:].contiguous()
            vn = vf[:, -1:].contiguous()
            pos = torch.full((w.bh_kv,), w.s_k - 1, dtype=torch.int32, device="cuda")
            fn = lambda: fa.append_kv(kn, vn, pos, kc, vc, ks, vs)   # noqa: E731
            log("[bench] timing append (c4 shape, one token per KV head)")
            ms = timer.run(fn, max(args.steps, 50), args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = 2 * w.bh_kv * (w.d * 4 + w.d + 4) + w.bh_kv * 4
            res["append"] = {"workload": "append_c4_1tok_kv128_d128_f32", "ms": avg, "ms_min": float(np.min(ms)),
                             "ms_median": float(np.median(ms)),
                             "kernel": fa.last_kernel(), "bytes_per_launch": nbytes, "gbs": nbytes / avg / 1e6,
                             "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS, "bound": "launch latency"}
            log(f"[bench] append: {avg * 1e3:.1f} us")
            del kn, vn, pos
        del kf, vf
        out = torch.empty((w.bh_q, 1, w.d), dtype=torch.float32, device="cuda")
        splits = fa.decode_num_splits(w.bh_q, w.bh_kv, w.s_k, w.d)
        ws = torch.empty(fa.decode_workspace_bytes(w.bh_q, w.bh_kv, w.s_k, w.d, splits), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: fa.decode(qd, kc, vc, ks, vs, num_splits=splits, out=out, workspace=ws)   # noqa: E731
        if "c4" in legs:
            log(f"[bench] timing {w.name}")
            ms = timer.run(fn, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = (2 * w.bh_kv * w.s_k * w.d + 2 * w.bh_kv * w.s_k * 4 + w.bh_q * w.d * 2 + w.bh_q * w.d * 4)
            res["c4"] = {"workload": w.name, "ms": avg, "ms_min": float(np.min(ms)),
                         "ms_median": float(np.median(ms)), "kernel": fa.last_kernel(),
                         "num_splits": splits, "bytes_per_launch": nbytes, "gbs": nbytes / avg / 1e6,
                         "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] c4: {avg * 1e3:.1f} us  {res['c4']['gbs']:.0f} GB/s")
            if not args.no_cpu:
                cpu["c4"] = decode_cpu_baseline(q, kc, ks, vc, vs, out, w, args.cpu_seconds)
        if "c4g8" in legs:
            # 8 query heads per KV head over the same cache: Q drawn from PCG64(48), bf16
            g8 = 8
            bh_q8 = w.bh_kv * g8
            q8 = bf16_dev(np.random.Generator(np.random.PCG64(48)).standard_normal((bh_q8, 1, w.d), dtype=np.float32))
            out8 = torch.empty((bh_q8, 1, w.d), dtype=torch.float32, device="cuda")
            splits8 = fa.decode_num_splits(bh_q8, w.bh_kv, w.s_k, w.d)
            ws8 = torch.empty(fa.decode_workspace_bytes(bh_q8, w.bh_kv, w.s_k, w.d, splits8), dtype=torch.uint8,
                              device="cuda")
            fn8 = lambda: fa.decode(q8, kc, vc, ks, vs, num_splits=splits8, out=out8, workspace=ws8)   # noqa: E731
            log("[bench] timing decode with GQA group 8")
            ms = timer.run(fn8, args.steps, args.warmup, flush=flush)
            avg = float(np.mean(ms))
            nbytes = (2 * w.bh_kv * w.s_k * w.d + 2 * w.bh_kv * w.s_k * 4 + bh_q8 * w.d * 2 + bh_q8 * w.d * 4)
            res["c4g8"] = {"workload": "decode_g8_b16_h64kv8_sk32768_d128", "ms": avg, "ms_min": float(np.min(ms)),
                           "ms_median": float(np.median(ms)),
                           "kernel": fa.last_kernel(), "num_splits": splits8, "bytes_per_launch": nbytes,
                           "gbs": nbytes / avg / 1e6, "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
            log(f"[bench] c4g8: {avg * 1e3:.1f} us  {res['c4g8']['gbs']:.0f} GB/s")
            del q8, out8, ws8
        del qd, kc, vc, ks, vs, out, ws

    if "merge" in legs:
        n_parts, rows, d = 8, 64 * 4096, 128
        g = torch.Generator(device="cuda")
        g.manual_seed(9)
        o_parts = torch.randn((n_parts, rows, d), generator=g, device="cuda", dtype=torch.float32)
        lse_parts = torch.randn((n_parts, rows), generator=g, device="cuda", dtype=torch.float32) * 4
        out = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
        fn = lambda: fa.merge_lse(o_parts, lse_parts, out=out)   # noqa: E731
        log("[bench] timing merge (8 parts x 64 heads x 4096 rows, d 128)")
        ms = timer.run(fn, args.steps, args.warmup, flush=flush)
        avg = float(np.mean(ms))
        nbytes = n_parts * rows * (d * 4 + 4) + rows * d * 2
        res["merge"] = {"workload": "merge_8parts_h64_4096rows_d128_f32_to_bf16", "ms": avg,
                        "ms_min": float(np.min(ms)),
                        "ms_median": float(np.median(ms)), "kernel": fa.last_kernel(), "bytes_per_launch": nbytes,
                        "gbs": nbytes / avg / 1e6, "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
        log(f"[bench] merge: {avg * 1e3:.1f} us  {res['merge']['gbs']:.0f} GB/s")
        del o_parts, lse_parts, out

    if "copy" in legs:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        fn = lambda: dst.copy_(src)   # noqa: E731
        log("[bench] timing copy 1 GiB")
        ms = timer.run(fn, args.steps, args.warmup, flush=flush)
        avg = float(np.mean(ms))
        nbytes = 2 * src.numel() * 4
        res["copy"] = {"workload": "device_copy_1GiB", "ms": avg, "bytes_per_launch": nbytes,
                       "gbs": nbytes / avg / 1e6, "frac_of_peak": nbytes / avg / 1e6 / PEAK_HBM_GBS}
        log(f"[bench] copy: {avg:.3f} ms  {res['copy']['gbs']:.0f} GB/s")
        del src, dst

    line = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": WORKLOADS["c5"].name, "batch": 1, "heads_q": 64, "heads_kv": 8,
                       "seq_len": 32768, "head_dim": 128, "causal": True, "parallelism": "single-gpu"}}
    if "c5" in res:
        r = res["c5"]
        line["value"] = round(r["tflops"], 2)
        line["ms_per_step"] = round(r["ms"], 4)
        line["roofline"] = {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(r["frac_of_peak"], 4),
                            "traffic": traffic_for("c5"),
                            "kernel": r["kernel"], "flop_per_launch": r["flop_per_launch"]}
        # the same fraction against the peak at the shader clock measured under this load
        mhz = r.get("clock_mhz")
        line["roofline"]["clock_mhz"] = mhz
        line["roofline"]["frac_at_clock"] = (round(r["tflops"] / (PEAK_BF16_TFLOPS * mhz / 2400.0), 4)
                                             if mhz else None)
    if "c4" in res:
        r = res["c4"]
        line["decode"] = {"metric": "int8-KV decode GB/s", "value": round(r["gbs"], 1), "unit": "GB/s",
                          "ms": round(r["ms"], 5), "workload": r["workload"], "num_splits": r["num_splits"],
                          "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(r["frac_of_peak"], 4),
                                       "traffic": traffic_for("c4"),
                                       "bytes_per_launch": r["bytes_per_launch"]}}
        if "c4" in cpu:
            line["decode"]["cpu_baseline"] = cpu["c4"]
    for k, r in res.items():
        if k in LEG_SOURCES:
            r["source_sha"] = source_sha(k)
            r["traffic"] = traffic_for(k)
    line["legs"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                    for k, r in res.items()}
    if "c5" in cpu:
        line["cpu_baseline"] = cpu["c5"]
    print(json.dumps(line), flush=True)


def prefill_cpu_baseline(q, k, v, out_gpu, w, budget_s):
    """The oracle on the host cores over the last rows of query heads of the c5 workload (the rows
    that see the most keys), for about `budget_s` seconds; also checks those rows of the GPU output."""
    import oracle
    import torch
    G = w.group
    rows_per = 256
    t0 = time.perf_counter()
    flops = 0.0
    err = 0.0
    done = []
    h = 0
    while time.perf_counter() - t0 < budget_s and h < w.bh_q:
        rows = list(range(w.s_q - rows_per, w.s_q))
        o, _ = oracle.attention(q[h:h + 1], k[h // G:h // G + 1], v[h // G:h // G + 1], causal=True, rows=rows)
        flops += 4.0 * w.d * sum(min(i + 1, w.s_k) for i in rows)
        g = out_gpu[h, rows[0]:rows[-1] + 1].float().cpu().numpy()
        err = max(err, float(np.abs(g - o[0, rows]).max()))
        done.append(h)
        h += 1
    dt = time.perf_counter() - t0
    log(f"[bench] oracle c5 sample: {len(done)} heads x {rows_per} rows in {dt:.1f}s, gpu max err {err:.2e}")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle, {len(done)} query heads x the last {rows_per} rows of {w.name} "
                      f"({flops / 1e9:.1f} GFLOP, {dt:.1f} s)",
            "seconds": round(dt, 2), "host_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "gpu_max_abs_err_on_sample": err}


def decode_cpu_baseline(q, kc, ks, vc, vs, out_gpu, w, budget_s):
    """The oracle decode over whole KV heads of the c4 cache for about `budget_s` seconds; the bytes
    it covers are counted like the GPU leg's (codes, scales, Q, output)."""
    import oracle
    G = w.group
    wall0 = time.perf_counter()
    t_oracle = 0.0
    nbytes = 0
    err = 0.0
    kvh = 0
    og = out_gpu.cpu().numpy()
    while time.perf_counter() - wall0 < budget_s and kvh < w.bh_kv:
        kq = kc[kvh:kvh + 1].cpu().numpy()
        vq = vc[kvh:kvh + 1].cpu().numpy()
        ksh = ks[kvh:kvh + 1].cpu().numpy()
        vsh = vs[kvh:kvh + 1].cpu().numpy()
        t1 = time.perf_counter()
        o, _ = oracle.decode(q[kvh * G:(kvh + 1) * G], kq, vq, k_scale=ksh, v_scale=vsh)
        t_oracle += time.perf_counter() - t1
        err = max(err, float(np.abs(og[kvh * G:(kvh + 1) * G] - o).max()))
        nbytes += 2 * w.s_k * w.d + 2 * w.s_k * 4 + G * w.d * 6
        kvh += 1
    dt = t_oracle
    log(f"[bench] oracle c4 sample: {kvh} KV heads in {dt:.1f}s, gpu max err {err:.2e}")
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle decode, {kvh} of {w.bh_kv} KV heads of {w.name}",
            "seconds": round(dt, 2), "gpu_max_abs_err_on_sample": err}


if __name__ == "__main__":
    main()
