"""Seeded synthetic inputs for LRKV decode.

This module is shared by the tests, the benchmark and the CPU reference.  It
holds no attention arithmetic: it defines the named workloads (shapes, dtypes,
value distributions, length mix) and turns (workload, layer, tensor, element)
into numbers through the counter-based generator in ``gen.c``.

Tensor layouts (row-major, element counts):
  q          [batch, H, d_h]
  k_shared   [batch, L_cap, d_h]      v_shared likewise
  z_k        [batch, H, L_cap, r]     z_v likewise
  B_k        [H, d_h, r]              B_v likewise
  seq_lens   [batch] int32            live rows per sequence

These are the logical (per-head) layouts that the CPU reference reads.  The
GPU library stores latents token-major, [batch, L_cap, H, r]; synth.device
transposes when it copies a cache to the device.

Only the live rows (j < seq_lens[b]) of the caches are generated; rows beyond
are zero.  Element (b, j, c) of k_shared uses counter b*L_cap*d_h + j*d_h + c,
so any sequence can be regenerated alone and gives the same values.

Value recipe (the variance is the second parameter of N(mean, var)):
  q, k_shared, v_shared ~ N(0, 1); z_k, z_v ~ N(0, z_var); B_k, B_v ~ N(0, 1/r).
fp64 sample -> fp32 (round to nearest even) -> bf16 (round to nearest even)
for bf16 workloads.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_BASE = 260111471
TENSOR_IDS = {"q": 0, "k_shared": 1, "v_shared": 2, "z_k": 3, "z_v": 4,
              "B_k": 5, "B_v": 6, "seq_lens": 7, "k_new": 8, "v_new": 9,
              "zk_new": 10, "zv_new": 11}


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, dbl, szt, i32 = ctypes.c_uint64, ctypes.c_double, ctypes.c_size_t, ctypes.c_int32
        vp = ctypes.c_void_p
        lib.synth_normal_f32.argtypes = [u64, dbl, u64, vp, szt, ctypes.c_int]
        lib.synth_normal_bf16.argtypes = [u64, dbl, u64, vp, szt, ctypes.c_int]
        lib.synth_normal_f64.argtypes = [u64, dbl, u64, vp, szt, ctypes.c_int]
        lib.synth_uniform_int.argtypes = [u64, i32, i32, u64, vp, szt]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_normal_f64, lib.synth_uniform_int):
            f.restype = None
        _lib = lib
    return _lib


def host_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def normal(seed: int, std: float, n: int, dtype: str, offset: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """n samples of std*N(0,1); dtype 'f32' -> float32, 'bf16' -> uint16 bit patterns, 'f64' -> float64."""
    lib = _load()
    np_dtype = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    if out is None:
        out = np.empty(n, dtype=np_dtype)
    assert out.dtype == np_dtype and out.size == n and out.flags.c_contiguous
    fn = {"f32": lib.synth_normal_f32, "bf16": lib.synth_normal_bf16, "f64": lib.synth_normal_f64}[dtype]
    if n:
        fn(seed & 0xFFFFFFFFFFFFFFFF, float(std), offset, out.ctypes.data, n, host_threads())
    return out


def uniform_int(seed: int, lo: int, hi: int, n: int, offset: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int32)
    if n:
        lib.synth_uniform_int(seed, lo, hi, offset, out.ctypes.data, n)
    return out


def gain(seed: int, shape, dtype: str, spread: float = 0.25) -> np.ndarray:
    """Per-coordinate gains 1 + spread*N(0,1) (normalisation weights), stored in dtype: fp64 -> fp32 round to
    nearest even -> (bf16) round to nearest even, as the other generated tensors."""
    n = int(np.prod(shape))
    f = (1.0 + normal(seed, spread, n, "f64")).astype(np.float32)
    if dtype == "f64":
        return f.astype(np.float64).reshape(shape)
    if dtype == "f32":
        return f.reshape(shape)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16).reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One named decode workload: shapes, dtype and value recipe."""
    name: str
    wid: int                 # workload number used in the seeds
    batch: int
    H: int
    d_h: int
    r: int
    L: int                   # context length (upper end of the range when ragged)
    dtype: str               # 'f32' or 'bf16' (q, caches and B all in this dtype)
    layers: int = 1
    z_var: float = 1.0
    ragged_lo: Optional[int] = None   # lengths uniform in [ragged_lo, L] when set
    length_wid: Optional[int] = None  # workload number whose length draw is reused
    L_cap: Optional[int] = None

    @property
    def cap(self) -> int:
        return self.L_cap if self.L_cap is not None else self.L

    @property
    def b_std(self) -> float:
        return math.sqrt(1.0 / self.r) if self.r > 0 else 0.0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def seed(self, layer: int, tensor: str) -> int:
        return SEED_BASE + 1000 * self.wid + 10 * layer + TENSOR_IDS[tensor]

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS: Dict[str, Workload] = {
    # single layer, fp32 everywhere, every position visible
    "tiny_fp32": Workload("tiny_fp32", 0, batch=1, H=4, d_h=16, r=4, L=64, dtype="f32"),
    # bf16 cache, fp32 accumulate; latents printed as [8, 8, 2048, 8]
    "small_bf16": Workload("small_bf16", 1, batch=8, H=8, d_h=64, r=8, L=2048, dtype="bf16"),
    # ~1B-parameter layer shape, 24 independent layers, cache fraction 0.4375 of MHA
    "mid_24layer": Workload("mid_24layer", 2, batch=16, H=16, d_h=128, r=48, L=8192, dtype="bf16", layers=24),
    # long context, latents N(0, 0.5), cache fraction 0.53125 of MHA
    "long_context": Workload("long_context", 3, batch=4, H=32, d_h=128, r=64, L=32768, dtype="bf16", z_var=0.5),
    # 64 sequences with lengths uniform in [512, 32768]
    "ragged": Workload("ragged", 4, batch=64, H=32, d_h=128, r=32, L=32768, dtype="bf16", ragged_lo=512),
    # the same length draw with r = 0 (MQA-style sharing), fp32 values
    "ragged_mqa_fp32": Workload("ragged_mqa_fp32", 5, batch=64, H=32, d_h=128, r=0, L=32768, dtype="f32",
                                ragged_lo=512, length_wid=4),
    # the layer shapes of the reading notes' model table (d_h 128 with the ranks of its Table 7), at the
    # pages' longer training context of 8192 tokens, 16 sequences
    "model_128m": Workload("model_128m", 6, batch=16, H=6, d_h=128, r=46, L=8192, dtype="bf16"),
    "model_1p2b": Workload("model_1p2b", 7, batch=16, H=12, d_h=128, r=51, L=8192, dtype="bf16"),
    "model_2p5b": Workload("model_2p5b", 8, batch=16, H=18, d_h=128, r=55, L=8192, dtype="bf16"),
    "model_6p3b": Workload("model_6p3b", 9, batch=16, H=32, d_h=128, r=54, L=8192, dtype="bf16"),
}


def seq_lengths(w: Workload, layer: int = 0) -> np.ndarray:
    if w.ragged_lo is None:
        return np.full(w.batch, w.L, dtype=np.int32)
    src = w if w.length_wid is None else next(x for x in WORKLOADS.values() if x.wid == w.length_wid)
    return uniform_int(src.seed(0, "seq_lens"), w.ragged_lo, w.L, w.batch)


def gen_small(w: Workload, layer: int, name: str) -> np.ndarray:
    """Whole (non-cache) tensors: q, B_k, B_v."""
    dt = w.dtype
    if name == "q":
        shape = (w.batch, w.H, w.d_h)
        std = 1.0
    elif name in ("B_k", "B_v"):
        shape = (w.H, w.d_h, w.r)
        std = w.b_std
    else:
        raise ValueError(name)
    n = int(np.prod(shape))
    return normal(w.seed(layer, name), std, n, dt).reshape(shape)


def gen_shared_rows(w: Workload, layer: int, name: str, b: int, rows: int) -> np.ndarray:
    """Rows [0, rows) of k_shared / v_shared for sequence b, shape [rows, d_h]."""
    off = b * w.cap * w.d_h
    return normal(w.seed(layer, name), 1.0, rows * w.d_h, w.dtype, offset=off).reshape(rows, w.d_h)


def gen_latent_rows(w: Workload, layer: int, name: str, b: int, h: int, rows: int) -> np.ndarray:
    """Rows [0, rows) of z_k / z_v for (sequence b, head h), shape [rows, r]."""
    off = (b * w.H + h) * w.cap * w.r
    return normal(w.seed(layer, name), math.sqrt(w.z_var), rows * w.r, w.dtype, offset=off).reshape(rows, w.r)


def gen_sequence(w: Workload, layer: int, b: int, rows: int) -> Dict[str, np.ndarray]:
    """Live rows of every cache tensor of sequence b: k/v [rows, d_h], z [H, rows, r]."""
    out = {"k_shared": gen_shared_rows(w, layer, "k_shared", b, rows),
           "v_shared": gen_shared_rows(w, layer, "v_shared", b, rows)}
    for name in ("z_k", "z_v"):
        if w.r == 0:
            out[name] = np.zeros((w.H, rows, 0), dtype=out["k_shared"].dtype)
            continue
        off = b * w.H * w.cap * w.r
        if rows == w.cap:  # one contiguous stream for all heads
            arr = normal(w.seed(layer, name), math.sqrt(w.z_var), w.H * rows * w.r, w.dtype, offset=off)
            out[name] = arr.reshape(w.H, rows, w.r)
        else:
            out[name] = np.stack([gen_latent_rows(w, layer, name, b, h, rows) for h in range(w.H)])
    return out


def gen_host(w: Workload, layer: int = 0, lengths: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """All inputs of one layer as host arrays in the cache layout (rows past seq_lens are zero)."""
    lens = seq_lengths(w, layer) if lengths is None else np.asarray(lengths, dtype=np.int32)
    np_dt = np.float32 if w.dtype == "f32" else np.uint16
    k = np.zeros((w.batch, w.cap, w.d_h), dtype=np_dt)
    v = np.zeros_like(k)
    zk = np.zeros((w.batch, w.H, w.cap, w.r), dtype=np_dt)
    zv = np.zeros_like(zk)
    for b in range(w.batch):
        n = int(lens[b])
        s = gen_sequence(w, layer, b, n)
        k[b, :n] = s["k_shared"]
        v[b, :n] = s["v_shared"]
        zk[b, :, :n] = s["z_k"]
        zv[b, :, :n] = s["z_v"]
    out = {"q": gen_small(w, layer, "q"), "k_shared": k, "v_shared": v, "z_k": zk, "z_v": zv,
           "seq_lens": lens}
    if w.r > 0:
        out["B_k"] = gen_small(w, layer, "B_k")
        out["B_v"] = gen_small(w, layer, "B_v")
    else:
        out["B_k"] = np.zeros((w.H, w.d_h, 0), dtype=np_dt)
        out["B_v"] = np.zeros((w.H, w.d_h, 0), dtype=np_dt)
    return out


def gen_new_rows(w: Workload, layer: int = 0) -> Dict[str, np.ndarray]:
    """One new token's projected rows per sequence, for the cache append."""
    dt = w.dtype
    out = {"k_new": normal(w.seed(layer, "k_new"), 1.0, w.batch * w.d_h, dt).reshape(w.batch, w.d_h),
           "v_new": normal(w.seed(layer, "v_new"), 1.0, w.batch * w.d_h, dt).reshape(w.batch, w.d_h)}
    for nm in ("zk_new", "zv_new"):
        out[nm] = normal(w.seed(layer, nm), math.sqrt(w.z_var), w.batch * w.H * w.r, dt).reshape(w.batch, w.H, w.r)
    return out

