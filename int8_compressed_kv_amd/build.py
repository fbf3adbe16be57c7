"""Build the gfx950 shared library libfa.so in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, and linked with the C-ABI dispatcher into libfa.so next to
this file.  Run as `python -m int8_compressed_kv_amd.build` or via build().
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")

HIP_SOURCES = ["compress.hip", "prefill_f32.hip", "prefill_bf16.hip", "prefill_i8kv.hip", "decode.hip", "merge.hip", "tq.hip", "tq_attn.hip"]
CPP_SOURCES = ["api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", CSRC, "-I", INCLUDE,
          "-Wall", "-Wno-unused-function"]
# packed fp32 (v_pk_*_f32) selection off for device code
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]
# The decode kernels keep their int32 MFMA accumulators in VGPRs: left to its heuristic the
# compiler allocates them to AGPRs and then copies them through VGPRs on every tile (the
# accumulators are also read by the fp32 flush), 50-150 extra moves per tile.
PER_FILE_FLAGS = {
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "tq_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library needs ROCm's hipcc")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, DEVICE_FLAGS + PER_FILE_FLAGS.get(s, [])) for s in HIP_SOURCES] + [(s, []) for s in CPP_SOURCES]
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")) or 1)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
