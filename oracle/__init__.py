"""CPU reference for LRKV decode attention (fp64).  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this package.  The product library never does.

``oracle.c`` holds the arithmetic; this module compiles it with gcc and
marshals numpy arrays into it.  See the header of ``oracle.c`` for the
definition it follows and the page sections it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs: Dict[str, ctypes.CDLL] = {}

DTYPE_CODES = {"f32": 0, "bf16": 1, "f64": 2}
_NP_FOR = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("H", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("r", ctypes.c_int32), ("L_cap", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def build(force: bool = True, plant: int = 0, out_path: Optional[str] = None) -> str:
    """Compile oracle.c.  ``plant`` > 0 builds a copy with one planted mistake (tests only)."""
    path = out_path or LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               f"-DORACLE_PLANT={int(plant)}", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, path)
    return path


def _bind(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    dp = ctypes.POINTER(_Dims)
    lib.oracle_lrkv_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32p, ctypes.c_int, i32p, i32p, vp, vp,
                                       ctypes.c_int]
    lib.oracle_mqa_decode.argtypes = [dp, vp, vp, vp, i32p, ctypes.c_int, i32p, i32p, vp, ctypes.c_int]
    lib.oracle_factored_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, i32p, ctypes.c_int, i32p, i32p, vp,
                                           ctypes.c_int]
    for f in (lib.oracle_lrkv_decode, lib.oracle_mqa_decode, lib.oracle_factored_decode):
        f.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    path = path or LIB_PATH
    if path not in _libs:
        if path == LIB_PATH and not os.path.exists(path):
            build(force=True)
        _libs[path] = _bind(path)
    return _libs[path]


def _threads(n: Optional[int]) -> int:
    if n is not None:
        return max(1, n)
    c = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        c = min(c, int(env))
    return max(1, min(c, 16))


def _arr(x, dt):
    if x is None:
        return None
    a = np.ascontiguousarray(x)
    assert a.dtype == _NP_FOR[dt], (a.dtype, dt)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _infer(dtype: str, q, k_shared, z_k, seq_lens) -> _Dims:
    batch, H, d_h = q.shape
    L_cap = k_shared.shape[1]
    r = 0 if z_k is None else z_k.shape[-1]
    return _Dims(batch, H, d_h, r, L_cap, DTYPE_CODES[dtype])


def _pairs(pairs, batch, H):
    if pairs is None:
        pairs = [(b, h) for b in range(batch) for h in range(H)]
    pb = np.ascontiguousarray([p[0] for p in pairs], dtype=np.int32)
    ph = np.ascontiguousarray([p[1] for p in pairs], dtype=np.int32)
    return pairs, pb, ph


def lrkv_decode(dtype: str, q, k_shared, v_shared, z_k, z_v, B_k, B_v, seq_lens,
                pairs: Optional[Sequence[Tuple[int, int]]] = None, want_weights: bool = False,
                threads: Optional[int] = None, lib_path: Optional[str] = None):
    """Reconstruct-then-attend reference.  Returns out[npairs, d_h] (and weights[npairs, L_cap])."""
    q, k_shared, v_shared = _arr(q, dtype), _arr(k_shared, dtype), _arr(v_shared, dtype)
    z_k, z_v, B_k, B_v = _arr(z_k, dtype), _arr(z_v, dtype), _arr(B_k, dtype), _arr(B_v, dtype)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    dims = _infer(dtype, q, k_shared, z_k, lens)
    pairs, pb, ph = _pairs(pairs, dims.batch, dims.H)
    out = np.zeros((len(pairs), dims.d_h), dtype=np.float64)
    w = np.zeros((len(pairs), dims.L_cap), dtype=np.float64) if want_weights else None
    rc = load(lib_path).oracle_lrkv_decode(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared), _ptr(z_k),
                                           _ptr(z_v), _ptr(B_k), _ptr(B_v), _ptr(lens), len(pairs), _ptr(pb),
                                           _ptr(ph), _ptr(out), _ptr(w), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_lrkv_decode rejected its arguments")
    return (out, w) if want_weights else out


def mqa_decode(dtype: str, q, k_shared, v_shared, seq_lens, pairs=None, threads=None, lib_path=None):
    """MQA reference: all heads read the shared keys and values."""
    q, k_shared, v_shared = _arr(q, dtype), _arr(k_shared, dtype), _arr(v_shared, dtype)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    dims = _infer(dtype, q, k_shared, None, lens)
    pairs, pb, ph = _pairs(pairs, dims.batch, dims.H)
    out = np.zeros((len(pairs), dims.d_h), dtype=np.float64)
    rc = load(lib_path).oracle_mqa_decode(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared), _ptr(lens),
                                          len(pairs), _ptr(pb), _ptr(ph), _ptr(out), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_mqa_decode rejected its arguments")
    return out


def factored_decode(dtype: str, q, k_shared, v_shared, z_k, z_v, B_k, B_v, seq_lens, pairs=None, threads=None,
                    lib_path=None):
    """Associative evaluation (used only to check the identity against lrkv_decode)."""
    q, k_shared, v_shared = _arr(q, dtype), _arr(k_shared, dtype), _arr(v_shared, dtype)
    z_k, z_v, B_k, B_v = _arr(z_k, dtype), _arr(z_v, dtype), _arr(B_k, dtype), _arr(B_v, dtype)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    dims = _infer(dtype, q, k_shared, z_k, lens)
    pairs, pb, ph = _pairs(pairs, dims.batch, dims.H)
    out = np.zeros((len(pairs), dims.d_h), dtype=np.float64)
    rc = load(lib_path).oracle_factored_decode(ctypes.byref(dims), _ptr(q), _ptr(k_shared), _ptr(v_shared),
                                               _ptr(z_k), _ptr(z_v), _ptr(B_k), _ptr(B_v), _ptr(lens), len(pairs),
                                               _ptr(pb), _ptr(ph), _ptr(out), _threads(threads))
    if rc != 0:
        raise ValueError("oracle_factored_decode rejected its arguments")
    return out


def _widen(dtype: str, a) -> np.ndarray:
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def absorb_query(dtype: str, q, B_k) -> np.ndarray:
    """The projected query p[b][h][i] = sum_c q[b][h][c] B_k[h][c][i] in fp64 from the exactly widened stored
    inputs ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4 Eq. (6): the key basis moves onto
    the query; "Low-Rank Key Value Attention | What a shared cache can preserve", sec. 3, one small product
    per head per step).  q [batch][H][d_h], B_k [H][d_h][r]; returns [batch][H][r] fp64."""
    qf, bf = _widen(dtype, q), _widen(dtype, B_k)
    B, H, d_h = qf.shape
    p = np.zeros((B, H, bf.shape[-1]))
    for h in range(H):
        p[:, h] = qf[:, h] @ bf[h]
    return p


def relative_error(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows are (sequence, head) outputs)."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den)) if num.size else 0.0


def lrkv_decode_multi(dtype: str, q, k_shared, v_shared, z_k, z_v, B_k, B_v, seq_lens, threads=None,
                      lib_path=None) -> np.ndarray:
    """Q query tokens per sequence, the last Q tokens of each sequence (already in the cache): query i sits
    at position L_b - Q + i and attends to rows j <= L_b - Q + i, the causal mask inside the chunk
    ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4, the score of Eq. (6) under the causal
    softmax; review sec. 3).  That is the single-query reference at length L_b - Q + i + 1 for every i.
    q [batch][Q][H][d_h]; returns out [batch][Q][H][d_h] (0 where a query sees no row)."""
    q = np.asarray(q)
    B, Q, H, d_h = q.shape
    lens = np.asarray(seq_lens, dtype=np.int32)
    out = np.zeros((B, Q, H, d_h), dtype=np.float64)
    for i in range(Q):
        li = np.clip(lens - Q + i + 1, 0, None).astype(np.int32)
        out[:, i] = lrkv_decode(dtype, np.ascontiguousarray(q[:, i]), k_shared, v_shared, z_k, z_v, B_k, B_v, li,
                                threads=threads, lib_path=lib_path).reshape(B, H, d_h)
    return out
