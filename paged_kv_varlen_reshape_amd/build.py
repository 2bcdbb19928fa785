"""Build libpa.so (HIP kernels for gfx950 + C-ABI + host allocator) in-tree.

    python -m paged_kv_varlen_reshape_amd.build [--jobs N] [--debug]

Objects go to paged_kv_varlen_reshape_amd/_build/, the library to
paged_kv_varlen_reshape_amd/libpa.so.  Every source is compiled every time.
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
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed-fp32 VALU forms are kept out of the device code: hipcc -O3 would
# otherwise pair float ops into v_pk_* instructions on its own.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]

# per-file device flags: in the chunk kernel no NaN reaches a maximum or the
# softmax (keys past a row's position are replaced by -inf before the maximum,
# V rows past the sequence are zeroed, and the factor the raw scores are
# multiplied by is positive, the host having folded a negative or zero scale
# into Q), so max/min need no NaN canonicalisation
FILE_FLAGS = {"chunk.hip": ["-fno-honor-nans"],
              # the work-queue claim is one lane's atomic whose result is used two steps
              # later; the atomic optimizer would rewrite it into a wave-wide read-back
              # that waits for it (and for every copy in flight) at once
              "chunk_pp.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}

SOURCES = ["errors.cpp", "pool.cpp", "validate.cpp", "api.hip", "reshape.hip", "plan.hip",
           "decode.hip", "decode_mfma.hip", "chunk.hip", "chunk_pp.hip", "measure.hip", "noalloc.hip"]


def _compile(src: str, opt: list[str]) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", f"--offload-arch={ARCH}", *opt, *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(src, []),
               "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++", *opt, *COMMON, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    opt = ["-O1", "-g"] if debug else ["-O3"]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, opt), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    args = ap.parse_args(argv)
    build(args.jobs, args.debug, verbose=True)


if __name__ == "__main__":
    main()
