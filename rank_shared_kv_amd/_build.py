"""Compile the HIP sources under csrc/ into liblrkv.so for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblrkv.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

# the bf16 decode kernel's instances are spread over eight translation units so they compile in parallel
SOURCES = ["lrkv_api.cpp", "k_cache.hip", "k_decode_general.hip", "k_decode_mfma.hip",
           "k_decode_mfma_part_d64_n0.hip", "k_decode_mfma_part_d128_n0.hip", "k_decode_mfma_part_d64_n1.hip",
           "k_decode_mfma_part_d128_n1.hip", "k_decode_mfma_part_d64_q2.hip", "k_decode_mfma_part_d64_q4.hip",
           "k_decode_mfma_part_d128_q2.hip", "k_decode_mfma_part_d128_q4.hip", "k_decode_mfma_part_d128_t7.hip", "k_decode_mfma_part_d64_s.hip",
           "k_decode_mfma_part_d128_s.hip", "k_decode_mfma_f32.hip",
           "k_merge.hip", "k_linear.hip", "k_materialize.hip", "k_norm.hip", "k_rope.hip", "k_decode_rope_mfma.hip",
           "k_probe.hip"]

# Packed fp32 instructions are disabled in device code: ordinary float code
# only, scheduled by the compiler without v_pk_*_f32.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
               "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-ffp-contract=fast"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that line is harmless
    lines = [l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))


def build(verbose: bool = False, out_path: str = LIB_PATH, defines=(), jobs: int = 0) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then link the shared library."""
    jobs = jobs or max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with tempfile.TemporaryDirectory(prefix="lrkv_build_") as tmpdir:
        cmds, objs = [], []
        for s in SOURCES:
            path = os.path.join(CSRC, s)
            obj = os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
            # .cpp files are host code that includes HIP headers; compile them as HIP too
            src = ["-x", "hip", path] if s.endswith(".cpp") else [path]
            cmds.append([hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, "-c", "-o",
                         obj, *src])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = out_path + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
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
