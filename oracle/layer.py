"""CPU reference for one LRKV layer decode step around the attention core (fp64).
TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does.

What it computes, for a batch of new tokens x_t (one per sequence):

  1. the projections of the new token ("Low-Rank Key Value Attention | What a
     shared cache can preserve", sec. 3, Algorithm 1; "Low-Rank Key Value
     Attention: Chinese reading notes", sec. 2.1 Eqs. (2)-(5) and sec. 2.3):
        q_h = x W_q,h          k_s = x W_S^K       v_s = x W_S^V
        z^K_h = x U^K_h        z^V_h = x U^V_h
     as one product y = x W_in^T with the rows of W_in stacked in the order
     [W_q (H*d_h) | W_S^K (d_h) | W_S^V (d_h) | U^K (H*r, head h at rows h*r) |
     U^V (H*r)];
  2. the new rows stored in the cache dtype (round to nearest even, through
     fp32 for bf16) and appended at index seq_lens[b]; q stored likewise;
  3. LRKV decode over the grown cache (oracle.lrkv_decode: per-head keys and
     values rebuilt in full, one softmax);
  4. the output projection y_out = concat_h(o_h) W_o^T (review, Algorithm 2's
     last step; reading notes sec. 2.4, after Eq. (7)).

A matrix product (numpy, fp64) serves as the product step; nothing is fused
or reordered.  ``plant`` > 0 plants one known mistake (tests only).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import lrkv_decode


def widen(dtype: str, a) -> np.ndarray:
    """Stored values (fp32, bf16 bit patterns as uint16, or fp64) as exact fp64."""
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to(dtype: str, a64: np.ndarray) -> np.ndarray:
    """fp64 -> stored dtype: fp32 round to nearest even, then for bf16 to nearest even again."""
    a64 = np.asarray(a64, dtype=np.float64)
    if dtype == "f64":
        return a64.copy()
    f = a64.astype(np.float32)
    if dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def linear(x_dtype: str, x, w_dtype: str, W) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] W[n][k] in fp64 (W holds one output feature per row)."""
    return widen(x_dtype, x) @ widen(w_dtype, W).T


def split_projection(y: np.ndarray, H: int, d_h: int, r: int, plant: int = 0) -> Dict[str, np.ndarray]:
    """Cut the stacked projection [batch][H*d_h + 2*d_h + 2*H*r] into its parts."""
    B = y.shape[0]
    o = 0
    q = y[:, o:o + H * d_h].reshape(B, H, d_h); o += H * d_h
    k = y[:, o:o + d_h]; o += d_h
    v = y[:, o:o + d_h]; o += d_h
    zk = y[:, o:o + H * r].reshape(B, H, r); o += H * r
    zv = y[:, o:o + H * r].reshape(B, H, r); o += H * r
    assert o == y.shape[1]
    if plant == 1:
        k, v = v, k
    if plant == 3:
        zv = zv[:, ::-1, :]
    return {"q": q, "k_new": k, "v_new": v, "zk_new": zk, "zv_new": zv}


def project_history(dtype: str, X, W_in, H: int, d_h: int, r: int, L_cap: int, lens) -> Dict[str, np.ndarray]:
    """Caches built by projecting a history of tokens X[batch][L][d_model] (Algorithm 1), stored in dtype.
    Rows at or past lens[b] are zero."""
    B, L, dm = np.asarray(X).shape
    y = linear(dtype, np.asarray(X).reshape(B * L, dm), dtype, W_in).reshape(B, L, -1)
    parts = split_projection(y.reshape(B * L, -1), H, d_h, r)
    npdt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    cache = {"k_shared": np.zeros((B, L_cap, d_h), npdt), "v_shared": np.zeros((B, L_cap, d_h), npdt),
             "z_k": np.zeros((B, H, L_cap, r), npdt), "z_v": np.zeros((B, H, L_cap, r), npdt)}
    k = round_to(dtype, parts["k_new"]).reshape(B, L, d_h)
    v = round_to(dtype, parts["v_new"]).reshape(B, L, d_h)
    zk = round_to(dtype, parts["zk_new"]).reshape(B, L, H, r)
    zv = round_to(dtype, parts["zv_new"]).reshape(B, L, H, r)
    for b in range(B):
        n = int(lens[b])
        cache["k_shared"][b, :n] = k[b, :n]
        cache["v_shared"][b, :n] = v[b, :n]
        cache["z_k"][b, :, :n] = zk[b, :n].transpose(1, 0, 2)
        cache["z_v"][b, :, :n] = zv[b, :n].transpose(1, 0, 2)
    return cache


def layer_step(dtype: str, x, W_in, W_o, B_k, B_v, cache: Dict[str, np.ndarray], seq_lens, H: int, d_h: int,
               r: int, plant: int = 0, lib_path: Optional[str] = None, threads: Optional[int] = None):
    """One decode step of a layer for every sequence.  Returns a dict with y (fp64 [batch][d_model]),
    the stored q and new rows, o (fp64 [batch][H][d_h]) and the grown lengths.  The cache arrays are
    not modified (the step works on copies)."""
    B = np.asarray(x).shape[0]
    L_cap = cache["k_shared"].shape[1]
    parts = split_projection(linear(dtype, x, dtype, W_in), H, d_h, r, plant)
    stored = {k: round_to(dtype, v) for k, v in parts.items()}
    c = {k: np.array(v, copy=True) for k, v in cache.items()}
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    for b in range(B):
        j = int(lens[b])
        if plant == 4 or j < 0 or j >= L_cap:
            continue
        c["k_shared"][b, j] = stored["k_new"][b]
        c["v_shared"][b, j] = stored["v_new"][b]
        if r > 0:
            c["z_k"][b, :, j] = stored["zk_new"][b]
            c["z_v"][b, :, j] = stored["zv_new"][b]
        lens[b] = j + 1
    o = lrkv_decode(dtype, stored["q"], c["k_shared"], c["v_shared"], c["z_k"], c["z_v"], B_k, B_v, lens,
                    threads=threads, lib_path=lib_path).reshape(B, H, d_h)
    Wo = widen(dtype, W_o)
    y = o.reshape(B, H * d_h) @ (Wo if plant == 2 else Wo.T)
    return {"y": y, "o": o, "lens": lens, **stored}


def materialize(dtype: str, k_shared, v_shared, z_k, z_v, B_k, B_v, seq_lens, rounded: bool = True):
    """Per-head keys and values of every live row, rebuilt from the factored cache and stored in dtype:
    K_h = K_S + Z^K_h (B^K_h)^T, V_h = V_S + Z^V_h (B^V_h)^T (reading notes sec. 2.1 Eqs. (2)-(5); review
    sec. 3, the materialised path used for training and prefill).  Inputs in the per-head layout; returns
    (K, V) as [batch][H][L_cap][d_h] in dtype, rows at or past seq_lens[b] zero.  rounded=False returns the
    exact fp64 values before the one rounding to dtype."""
    ks, vs = widen(dtype, k_shared), widen(dtype, v_shared)
    zk, zv = widen(dtype, z_k), widen(dtype, z_v)
    bk, bv = widen(dtype, B_k), widen(dtype, B_v)
    B, H, L_cap, r = zk.shape
    d_h = ks.shape[-1]
    K = np.zeros((B, H, L_cap, d_h))
    V = np.zeros((B, H, L_cap, d_h))
    for b in range(B):
        n = int(seq_lens[b])
        for h in range(H):
            K[b, h, :n] = ks[b, :n] + zk[b, h, :n] @ bk[h].T
            V[b, h, :n] = vs[b, :n] + zv[b, h, :n] @ bv[h].T
    if not rounded:
        return K, V
    return round_to(dtype, K), round_to(dtype, V)
