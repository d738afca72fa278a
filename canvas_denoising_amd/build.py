"""Build libdg.so in-tree with hipcc for gfx950.

    python -m canvas_denoising_amd.build [--jobs N] [--debug]

Every HIP source is compiled with packed-FP32 instruction selection turned
off (plain float code only) and linked into canvas_denoising_amd/libdg.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdg.so")

SOURCES = ["api.cpp", "prof.cpp", "model.cpp", "sampler.hip", "synth.hip", "gemm.hip", "attention.hip", "moe.hip",
           "elementwise.hip", "vocab.hip", "fp8.hip"]


# per-source compiler flags: the routed-expert streams keep their MFMA accumulators in ordinary
# VGPRs (with the accumulation registers the allocator gives every token-tile branch of a kernel
# its own set, which halves the waves per SIMD)
SOURCE_FLAGS: dict[str, list[str]] = {"moe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; libdg needs ROCm's hipcc to build")


def flags(debug: bool) -> list[str]:
    f = ["-std=c++17", "-fPIC", "--offload-arch=gfx950", f"-I{INCLUDE}", f"-I{CSRC}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas", "-Wno-unused-command-line-argument"]
    f += ["-O1", "-g", "-DDG_DEBUG=1"] if debug else ["-O3", "-DNDEBUG"]
    # extra preprocessor definitions for a measured variant build (DG_BUILD_DEFINES="NAME=VALUE ...")
    f += [f"-D{d}" for d in os.environ.get("DG_BUILD_DEFINES", "").split()]
    return f


def compile_one(src: str, debug: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + flags(debug) + SOURCE_FLAGS.get(src, []) + ["-c", path, "-o", obj]
    # extra compiler flags for one source of a measured variant build (DG_FLAGS_moe="...")
    cmd[1:1] = os.environ.get("DG_FLAGS_" + src.split(".")[0], "").split()
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # keep genuine warnings visible, drop the host pass's notice about the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, debug: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(8, os.cpu_count() or 4, len(srcs))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(objs)} sources")
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args()
    build(a.jobs, a.debug)


if __name__ == "__main__":
    main()
