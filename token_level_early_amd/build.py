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


def _compile(job):
    src, debug = job
    obj = os.path.join(BUILD, os.path.basename(src) + (".kvcount.o" if debug else ".o"))
    extra = ["-DRIVER_DEBUG_KV_COUNT"] if debug else []
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


def build(verbose=False, kvcount=True):
    """Builds libriver.so and (kvcount) libriver_kvcount.so; the slowest sources first."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + ([(s, True) for s in SOURCES] if kvcount else [])
    jobs.sort(key=lambda j: SOURCES.index(j[0]) < SOURCES.index("persist.hip"))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = dict(zip(jobs, ex.map(_compile, jobs)))
    if verbose:
        for _, err in results.values():
            if err.strip():
                print(err, file=sys.stderr)
    _link([results[(s, False)][0] for s in SOURCES], OUT)
    if kvcount:
        _link([results[(s, True)][0] for s in SOURCES], OUT_KVCOUNT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
