"""CPU reference for the normalised LRKV variant (fp64).
TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does.

The variant ("Low-Rank Key Value Attention | What a shared cache can preserve",
sec. 8, the paragraphs on post-projection normalisation and its cache cost;
"Low-Rank Key Value Attention: Chinese reading notes", sec. 2.7, last
paragraph): the key of head h at token j,
    k_{h,j} = k_s[j] + z^K_{h,j} (B^K_h)^T,
is RMS-normalised as a whole (the shared and private parts together) with a
per-head gain g^K_h, and the query likewise with g^Q_h:
    khat_{h,j} = g^K_h * k_{h,j} * rho_{h,j},   rho_{h,j} = 1 / sqrt(|k_{h,j}|^2 / d_h + eps)
    qhat_h     = g^Q_h * q_h / sqrt(|q_h|^2 / d_h + eps)
    logit_{h,j} = qhat_h . khat_{h,j} / sqrt(d_h)
Values are not normalised.  The exact factored evaluation the review
describes caches the joint reciprocal scale rho once per (head, token) and
multiplies the summed logit by it, with the key gain moved to the query side:
    q_eff_h = g^K_h * qhat_h
    logit_{h,j} = rho_{h,j} * (q_eff_h . k_s[j] + (q_eff_h B^K_h) . z^K_{h,j}) / sqrt(d_h).

Stored values: rho is kept in the cache dtype, one scalar per (sequence, token,
head) (the review's accounting prices it as one bf16 scalar per head and
position); q_eff is kept in the cache dtype like the query of the plain path.
``decode_normed`` reads both as stored.

Layout here is the pages' per-head one: latents [batch][H][L_cap][r], rho
[batch][H][L_cap].  ``plant`` > 0 plants one known mistake (tests only).
"""
from __future__ import annotations

import numpy as np

from .layer import round_to, widen


def _keys(ks: np.ndarray, zk: np.ndarray, bk: np.ndarray, b: int, h: int, n: int) -> np.ndarray:
    """K_h rows 0..n-1 of sequence b in fp64: k_s[j] + z^K_{h,j} (B^K_h)^T."""
    return ks[b, :n] + zk[b, h, :n] @ bk[h].T


def key_scales(dtype: str, k_shared, z_k, B_k, seq_lens, eps: float, plant: int = 0) -> np.ndarray:
    """rho[b][h][j] = 1 / sqrt(|k_{h,j}|^2 / d_h + eps) for the live rows j < L_b, fp64 and not rounded;
    0 at rows past L_b.  The norm is taken of the whole key, shared and private parts summed (review sec. 8:
    the denominator of the summed key; reading notes sec. 2.7: the two parts cannot be normalised apart)."""
    ks, zk, bk = widen(dtype, k_shared), widen(dtype, z_k), widen(dtype, B_k)
    B, H, L_cap, r = zk.shape
    d_h = ks.shape[-1]
    rho = np.zeros((B, H, L_cap))
    for b in range(B):
        n = max(0, min(int(seq_lens[b]), L_cap))
        for h in range(H):
            K = ks[b, :n] if plant == 1 else _keys(ks, zk, bk, b, h, n)
            ms = np.sum(K * K, axis=-1) / d_h
            rho[b, h, :n] = (1.0 / (np.sqrt(ms) + eps)) if plant == 3 else 1.0 / np.sqrt(ms + eps)
    return rho


def norm_query(dtype: str, q, g_q, g_k, eps: float, plant: int = 0) -> np.ndarray:
    """q_eff[b][h] = g^K_h * g^Q_h * q[b][h] / sqrt(|q[b][h]|^2 / d_h + eps) in fp64, not rounded: the
    RMS-normalised query with the key gain folded in (review sec. 8)."""
    qq, gq, gk = widen(dtype, q), widen(dtype, g_q), widen(dtype, g_k)
    d_h = qq.shape[-1]
    inv = 1.0 / np.sqrt(np.sum(qq * qq, axis=-1, keepdims=True) / d_h + eps)
    qhat = gq * qq * inv
    return qhat if plant == 2 else gk * qhat


def decode_normed(dtype: str, q_eff, k_shared, v_shared, z_k, z_v, B_k, B_v, rho, seq_lens,
                  plant: int = 0) -> np.ndarray:
    """o[b][h] = sum_j a_j V_h[j] with a = softmax_j(rho[b][h][j] * (q_eff[b][h] . K_h[j]) / sqrt(d_h)) over the
    live rows, K_h and V_h rebuilt in full from the factors; q_eff and rho as stored in dtype.  fp64 result
    [batch][H][d_h]; a sequence with no live row gives 0."""
    qe, r64 = widen(dtype, q_eff), widen(dtype, rho)
    ks, vs = widen(dtype, k_shared), widen(dtype, v_shared)
    zk, zv = widen(dtype, z_k), widen(dtype, z_v)
    bk, bv = widen(dtype, B_k), widen(dtype, B_v)
    B, H, L_cap, r = zk.shape
    d_h = ks.shape[-1]
    out = np.zeros((B, H, d_h))
    for b in range(B):
        n = max(0, min(int(seq_lens[b]), L_cap))
        if n == 0:
            continue
        for h in range(H):
            K = _keys(ks, zk, bk, b, h, n)
            V = vs[b, :n] + zv[b, h, :n] @ bv[h].T
            if plant == 4:  # the scale on the shared part of the logit only
                s = (r64[b, h, :n] * (ks[b, :n] @ qe[b, h]) + (K - ks[b, :n]) @ qe[b, h]) / np.sqrt(d_h)
            else:
                s = r64[b, h, :n] * (K @ qe[b, h]) / np.sqrt(d_h)
            e = np.exp(s - np.max(s))
            out[b, h] = (e / np.sum(e)) @ V
    return out


def stored(dtype: str, x64: np.ndarray) -> np.ndarray:
    """An fp64 result kept in the cache dtype (round to nearest even through fp32 for bf16)."""
    return round_to(dtype, x64)
