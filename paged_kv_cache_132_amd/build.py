"""Build libpa.so (the C-ABI library of HIP kernels for gfx950) in-tree.

    python -m paged_kv_cache_132_amd.build

compiles every source under csrc/ with hipcc for gfx950 (one object per
source, in parallel, under _build/) and links them into
paged_kv_cache_132_amd/libpa.so.  Packed-fp32 VALU instructions are disabled
for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(REPO, "include")
OBJ_DIR = os.path.join(REPO, "_build")
LIB = os.path.join(PKG, "libpa.so")
BENCH_LIB = os.path.join(PKG, "libpa_bench.so")

SOURCES = ["pa_api.cpp", "block_manager.cpp", "cache_write.hip", "copy_blocks.hip", "decode.hip",
           "decode_gqa_mfma.hip", "decode_gqa16_mfma.hip", "decode_noalloc.hip", "prefill.hip"]
BENCH_SOURCES = ["bench_util.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: with AGPR accumulators the compiler moves
    # them through VGPRs around every rescale (the fp8 GQA decode kernel)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed: {what}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines))


def _compile_one(src, tag, verbose):
    obj = os.path.join(OBJ_DIR, f"{tag}_{os.path.splitext(src)[0]}.o")
    _run([hipcc(), *COMPILE_FLAGS, "-x", "hip", f"-I{INCLUDE}", f"-I{CSRC}", "-c",
          os.path.join(CSRC, src), "-o", obj], src, verbose)
    return obj


def _compile(sources, out, verbose, jobs):
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = os.path.splitext(os.path.basename(out))[0]
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(sources)))) as ex:
        objs = list(ex.map(lambda s: _compile_one(s, tag, verbose), sources))
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], f"link {out}", verbose)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libpa.so (the decode path) and libpa_bench.so (measurement helpers)."""
    jobs = min(8, os.cpu_count() or 1)
    _compile(BENCH_SOURCES, BENCH_LIB, verbose, jobs)
    return _compile(SOURCES, LIB, verbose, jobs)


if __name__ == "__main__":
    print(build(verbose=True))
