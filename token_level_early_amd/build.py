"""Builds libriver.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object in parallel, then linked into
token_level_early_amd/libriver.so. Called by __graft_entry__.build() and usable as
``python -m token_level_early_amd.build``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libriver.so")
# the same sources with -DRIVER_DEBUG_KV_COUNT: per-element KV write counters (tests only)
OUT_KVCOUNT = os.path.join(HERE, "libriver_kvcount.so")
# the same sources with -DRIVER_PHASE_TRACE: phase timestamps of the persistent kernel (profiling)
OUT_PHASETRACE = os.path.join(HERE, "libriver_phasetrace.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
SOURCES = ["api.cpp", "quant.hip", "decode.hip", "prefill.hip", "persist.hip", "batched.hip"]


# debug variants: object suffix and define
VARIANTS = {"": [], "kvcount": ["-DRIVER_DEBUG_KV_COUNT"], "phasetrace": ["-DRIVER_PHASE_TRACE"]}
# the phase-trace library recompiles only what the define changes and links the rest as released
PHASETRACE_SOURCES = ["api.cpp", "persist.hip"]


def _compile(job):
    src, variant = job
    obj = os.path.join(BUILD, os.path.basename(src) + (f".{variant}.o" if variant else ".o"))
    extra = VARIANTS[variant]
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)


def build(verbose=False, kvcount=True, phasetrace=True):
    """Builds libriver.so, (kvcount) libriver_kvcount.so and (phasetrace)
    libriver_phasetrace.so; the slowest sources first."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, "") for s in SOURCES]
    if kvcount:
        jobs += [(s, "kvcount") for s in SOURCES]
    if phasetrace:
        jobs += [(s, "phasetrace") for s in PHASETRACE_SOURCES]
    jobs.sort(key=lambda j: SOURCES.index(j[0]) < SOURCES.index("persist.hip"))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = dict(zip(jobs, ex.map(_compile, jobs)))
    if verbose:
        for _, err in results.values():
            if err.strip():
                print(err, file=sys.stderr)
    _link([results[(s, "")][0] for s in SOURCES], OUT)
    if kvcount:
        _link([results[(s, "kvcount")][0] for s in SOURCES], OUT_KVCOUNT)
    if phasetrace:
        _link([results[(s, "phasetrace" if s in PHASETRACE_SOURCES else "")][0] for s in SOURCES], OUT_PHASETRACE)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
