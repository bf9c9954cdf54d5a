"""Build libpagedkv.so (HIP kernels + C ABI + host allocator) for gfx950, in-tree.

    python -m paged_kv_cache_397_amd.build

The library is compiled with hipcc for --offload-arch=gfx950 only.  Packed
fp32 instructions are disabled for the device code.  The library loads on a
machine without a GPU (the HIP runtime starts lazily), so the host allocator
can be exercised there.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
# A read-bandwidth probe with the decode kernel's access pattern, for measuring the
# part's ceiling; a library of its own, never loaded by the paged-attention path.
PROBE_LIB = os.path.join(PKG, "libpagedkv_probe.so")
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.cpp", "allocator.cpp", "scheduler.cpp", "kernels_cache.hip", "kernels_decode.hip",
           "kernels_prefill.hip"]
# decode_variant.hip is compiled once per decode kernel variant (load policy, decode
# step, block size 8) so that the variants build in parallel.
VARIANTS = [(stream, step, half) for stream in (0, 1) for step in (0, 1) for half in (0, 1)]
PROBE_SOURCES = ["bandwidth_probe.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; keep other output
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if verbose and rest:
        print("\n".join(rest))


def build(verbose: bool = False) -> str:
    """Compile every source, link libpagedkv.so and libpagedkv_probe.so; return the
    path of libpagedkv.so."""
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wall", "-Wno-unused-function"]
    objs = {}
    cmds = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs[src] = obj
        lang = ["-x", "hip"] if src.endswith(".hip") or src == "api.cpp" else ["-x", "c++"]
        cmds.append([hipcc, *common, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    variant_objs = []
    for stream, step, half in VARIANTS:
        obj = os.path.join(OBJ_DIR, f"decode_variant_{stream}{step}{half}.o")
        variant_objs.append(obj)
        cmds.append([hipcc, *common, "-x", "hip", f"-DPKV_STREAM={stream}", f"-DPKV_STEP={step}",
                     f"-DPKV_HALF={half}", "-c", os.path.join(CSRC, "decode_variant.hip"), "-o", obj])
    # the slowest (the decode variants) first
    cmds.sort(key=lambda c: "decode_variant.hip" not in " ".join(c))
    workers = max(1, min(len(cmds), os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, objs_of in ((LIB, [objs[s] for s in SOURCES] + variant_objs),
                         (PROBE_LIB, [objs[s] for s in PROBE_SOURCES])):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs_of, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
