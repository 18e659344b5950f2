"""Build libq4mi.so in-tree with hipcc for gfx950.

    python moe_w4a16_skinny_amd/build.py   (a path, not -m: the package import would load the old library)

Every source is compiled to its own object in parallel (one hipcc per file,
objects under _build/), then the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq4mi.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["q4mi_host.cpp", "q4mi_gemm.hip", "q4mi_moe.hip", "q4mi_quant.hip", "q4mi_prefill.hip", "q4mi_block.hip",
           "q4mi_affineb.hip", "q4mi_ceiling.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _filter(text: str):
    # the host pass does not know the gfx feature flag; drop that one warning
    return [l for l in text.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l]


def _compile(src: str, verbose: bool):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return obj, res.returncode, _filter(res.stdout + res.stderr)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    errors = [(o, m) for o, rc, m in results if rc != 0]
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n".join("\n".join(m) for _, m in errors))
    if verbose:
        for _, _, m in results:
            if m:
                print("\n".join(m))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_filter(res.stdout + res.stderr)))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
