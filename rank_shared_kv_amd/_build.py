"""Compile the HIP sources under csrc/ into liblrkv.so for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblrkv.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["lrkv_api.cpp", "k_cache.hip", "k_decode_general.hip", "k_decode_mfma.hip", "k_decode_mfma_f32.hip",
           "k_merge.hip", "k_linear.hip", "k_materialize.hip"]

# Packed fp32 instructions are disabled in device code: ordinary float code
# only, scheduled by the compiler without v_pk_*_f32.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
               "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-ffp-contract=fast"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out_path: str = LIB_PATH, defines=()) -> str:
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        # .cpp files are host code that includes HIP headers; compile them as HIP too
        srcs += (["-x", "hip", path] if s.endswith(".cpp") else [path])
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that line is harmless
    lines = [l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-o", default=LIB_PATH)
    ap.add_argument("-D", action="append", default=[])
    args = ap.parse_args()
    print(build(verbose=args.v, out_path=args.o, defines=args.D))
