"""Build the HIP libraries in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_357_amd.build

produces paged_kv_cache_357_amd/libpagedkv.so (the C-ABI library),
paged_kv_cache_357_amd/libpkv_probes.so (benchmark probes) and
paged_kv_cache_357_amd/libpagedkv_timing.so (the library with per-wave timing
of the shared-prefix stage 1, for measurement).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the device compiler from emitting packed fp32 ALU ops.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I", os.path.join(ROOT, "include"), "-I", CSRC]

# Host-only C++ (the block manager) is built with the host compiler.
HOST_CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", "-I", os.path.join(ROOT, "include")]

LIBS = {
    "libpagedkv.so": ["pagedkv_api.hip", "decode.hip", "decode_shared.hip", "prefill.hip", "append.hip",
                      "block_manager.cpp"],
    "libpkv_probes.so": ["bench_probes.hip"],
    # The same library with per-wave timing in the shared-prefix stage 1
    # (include/pagedkv_timing.h); only bench.py --wave-timing loads it.
    "libpagedkv_timing.so": ["pagedkv_api.hip", "decode.hip", "decode_shared.hip:timing", "prefill.hip",
                             "append.hip", "block_manager.cpp"],
}
# Sources compiled a second time with extra flags: "name:variant".
VARIANT_FLAGS = {"timing": ["-DPKV_WAVE_TIMING"]}


def _compile(src: str, verbose: bool) -> str:
    name, _, variant = src.partition(":")
    obj = os.path.join(BUILD, os.path.basename(name) + (f".{variant}" if variant else "") + ".o")
    if name.endswith(".cpp"):
        cmd = [HOST_CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, name), "-o", obj]
    else:
        cmd = [HIPCC, *DEVICE_FLAGS, *VARIANT_FLAGS.get(variant, []), "-c", os.path.join(CSRC, name), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> dict:
    """Compile every HIP source and link the shared libraries.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted({s for v in LIBS.values() for s in v})
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    out = {}
    for lib, parts in LIBS.items():
        dst = os.path.join(PKG, lib)
        tmp = dst + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[objs[p] for p in parts], "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {lib} failed:\n{r.stderr}")
        os.replace(tmp, dst)
        out[lib] = dst
    return out


if __name__ == "__main__":
    for k, v in build(verbose="-v" in sys.argv).items():
        print(k, "->", v)
