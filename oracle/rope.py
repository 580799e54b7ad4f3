"""CPU reference for LRKV decode under rotary position embedding (fp64).
TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the product library never does.

The variant ("Low-Rank Key Value Attention | What a shared cache can preserve", sec. 8, "Full RoPE needs a
stronger identity"; "Low-Rank Key Value Attention: Chinese reading notes", sec. 2.7): the head-width
rotation of the key position acts on the whole key of head h,
    ktilde_{h,j} = (k_s[j] + z^K_{h,j} (B^K_h)^T) D_j,
and the query is rotated by its own position, qtilde = q D_i.  A rotation cannot be moved into the rank-r
latent for a generic B_h, so the exact decode keeps the latents unrotated and contracts position by position
(the review's (qtilde D_j^T B_h) z_j^T).  Values are not rotated.

Rotation (the original rotary embedding, adjacent coordinate pairs): pair k = (2k, 2k+1) of a row vector x at
position t turns by phi = t * theta_k, theta_k = base^(-2k / d_h):
    (x_2k, x_2k+1) -> (x_2k cos phi - x_2k+1 sin phi, x_2k sin phi + x_2k+1 cos phi).
Positions: row j of a sequence sits at position j + pos0; the query is the sequence's last token, at
position L_b - 1 + pos0.  ``plant`` > 0 plants one known mistake (tests only).
"""
from __future__ import annotations

import numpy as np

from .layer import widen


def angles(d_h: int, positions, base: float = 10000.0) -> np.ndarray:
    """phi[t][k] = positions[t] * base^(-2k / d_h), k < d_h / 2 (fp64)."""
    k = np.arange(d_h // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d_h)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rotate(x: np.ndarray, phi: np.ndarray, plant: int = 0) -> np.ndarray:
    """Rows x[t] (fp64, even width) turned pair by pair by phi[t]."""
    c, s = np.cos(phi), np.sin(phi)
    if plant == 2:  # the opposite direction
        s = -s
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def decode_rope(dtype: str, q, k_shared, v_shared, z_k, z_v, B_k, B_v, seq_lens, base: float = 10000.0,
                pos0: int = 0, plant: int = 0) -> np.ndarray:
    """o[b][h] = sum_j a_j V_h[j], a = softmax_j(qtilde . ktilde_{h,j} / sqrt(d_h)) over the live rows, with the
    whole key of every head rotated at its position (module docstring).  Inputs as stored (per-head latent
    layout [batch][H][L_cap][r]); fp64 result [batch][H][d_h]; a sequence with no live row gives 0."""
    qq = widen(dtype, q)
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
        phi_k = angles(d_h, np.arange(n) + pos0, base)
        phi_q = angles(d_h, [n - 1 + pos0], base)
        if plant == 3:  # the query left at position 0
            phi_q = angles(d_h, [0], base)
        for h in range(H):
            if plant == 1:  # only the shared part rotated, the private part added unrotated
                K = rotate(ks[b, :n], phi_k) + zk[b, h, :n] @ bk[h].T
            else:
                K = rotate(ks[b, :n] + zk[b, h, :n] @ bk[h].T, phi_k, plant)
            V = vs[b, :n] + zv[b, h, :n] @ bv[h].T
            qt = rotate(qq[b, h][None, :], phi_q, plant)[0]
            s = (K @ qt) / np.sqrt(d_h)
            e = np.exp(s - np.max(s))
            out[b, h] = (e / np.sum(e)) @ V
    return out
