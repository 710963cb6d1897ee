"""Build librehyat.so (HIP for gfx950) in-tree with hipcc.

    python -m linear_attention_video_rehyat_amd.build [--jobs N]

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "librehyat.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librehyat)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# LLVM's iterative ILP scheduler for the kernels of the whole-clip forward: the
# forward at the Wan2.1-1.3B shape (local, block-state and scan kernels) ran
# 1.2 % faster than with the default scheduler, with bit-identical results
# (interleaved timing in one process).  Other files keep the default.
SCHED_ILP = ("-mllvm", "-amdgpu-sched-strategy=iterative-ilp")
FILE_FLAGS = {"local_bf16.hip": SCHED_ILP, "state_bf16.hip": SCHED_ILP, "scan.hip": SCHED_ILP}


def file_flags(name: str):
    """Extra hipcc flags of one source file (by base name)."""
    return FILE_FLAGS.get(name, ())


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, obj: str, extra=()) -> str:
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return err


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link librehyat.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, s, o, file_flags(os.path.basename(s))): s for s, o in zip(srcs, objs)}
        for f in cf.as_completed(futs):
            warn = f.result()
            if verbose and warn.strip():
                print(f"[{os.path.basename(futs[f])}]\n{warn}", file=sys.stderr)
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    # a kernel whose host stub was silently dropped leaves an undefined symbol
    # that only shows up when the library is loaded: refuse to install it
    nm = subprocess.run(["nm", "-u", "-C", tmp], capture_output=True, text=True)
    missing = [l.strip() for l in nm.stdout.splitlines() if "__device_stub__" in l or "rehyat::" in l]
    if missing:
        os.unlink(tmp)
        raise RuntimeError("link left undefined kernel symbols:\n" + "\n".join(missing[:10]))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
