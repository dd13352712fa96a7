"""Build libpa.so (the HIP library) in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_attention_26_amd.build`` (also called by
``__graft_entry__.build()``).  Every call recompiles every source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpa.so")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build", "libpa")

SOURCES = [
    "api.cpp",
    "block_manager.cpp",
    "debug_bounds.cpp",
    "store_copy.hip",
    "decode_f32.hip",
    "decode_bf16.hip",
    "decode_fp8.hip",
    "verify.hip",
    "prefill.hip",
    "noalloc.hip",
]

# HBM reference kernels, a library of their own (measurement only, no part of
# libpa's C ABI): the benchmark's --hbm-probe mode and its hbm_probe group
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_OUT = os.path.join(HERE, "libpa_probe.so")

# A measurement build of libpa whose bf16 decode kernels record per-wave time
# stamps (PA_DECODE_TRACE; pa_decode_trace_next arms a buffer): the
# benchmark's --decode-trace mode.  Only these sources differ from libpa.
TRACE_SOURCES = ["api.cpp", "decode_bf16.hip"]
TRACE_OUT = os.path.join(HERE, "libpa_trace.so")

ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-variable",
    f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: the compiler forms them from plain
    # float code, and this library never needs them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division (the fp8 store divides by the per-head scale)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libpa needs ROCm's hipcc to build")


def _compile(src: str, defines=()) -> str:
    tag = "".join("." + d.lower() for d in defines)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *COMMON, *("-D" + d for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(f"[build] {src}:\n{err}", file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"[build] wrote {out}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs_in = [(s, ()) for s in SOURCES + PROBE_SOURCES] + [(s, ("PA_DECODE_TRACE",)) for s in TRACE_SOURCES]
    jobs = min(len(jobs_in), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(lambda j: _compile(*j), jobs_in))
    objs = {j: o for j, o in zip(jobs_in, done)}
    _link([objs[(s, ())] for s in SOURCES], OUT, verbose)
    _link([objs[(s, ())] for s in PROBE_SOURCES], PROBE_OUT, verbose)
    _link([objs[(s, ("PA_DECODE_TRACE",))] if s in TRACE_SOURCES else objs[(s, ())] for s in SOURCES], TRACE_OUT,
          verbose)
    return OUT


if __name__ == "__main__":
    build()
