"""CPU reference for the paged cache layout.  TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product library never does.

A paged cache ("Low-Rank Key Value Attention | What a shared cache can preserve", sec. 4, the paged allocation
a serving system uses; sec. 9, append after prefill at page boundaries) stores the same rows as the contiguous
cache in fixed-size pages drawn from one pool per tensor: logical row t of sequence b lives in pool page
block_table[b][t // page_rows], at row t % page_rows of that page.  It changes where rows are kept, not what
attention computes, so the paged decode is defined as the decode of the gathered contiguous rows.

Pool layouts (as on the device): shared rows [n_pages][page_rows][d_h], latents token-major
[n_pages][page_rows][H][r].  ``gather`` returns the per-head layout the decode reference takes: k/v
[batch][L_cap][d_h], latents [batch][H][L_cap][r], rows past seq_lens zero.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def pool_row(block_table, b: int, t: int, page_rows: int) -> int:
    """Index of logical row t of sequence b among all pool rows (page-major)."""
    return int(block_table[b][t // page_rows]) * page_rows + t % page_rows


def gather(k_pages, v_pages, zk_pages, zv_pages, block_table, seq_lens, page_rows: int, max_pages: int,
           plant: int = 0) -> Dict[str, np.ndarray]:
    """The contiguous cache holding the live rows of a paged cache (L_cap = max_pages * page_rows)."""
    n_pages, P, d_h = np.asarray(k_pages).shape
    assert P == page_rows
    _, _, H, r = np.asarray(zk_pages).shape
    B = len(seq_lens)
    L_cap = max_pages * page_rows
    kp = np.asarray(k_pages).reshape(n_pages * P, d_h)
    vp = np.asarray(v_pages).reshape(n_pages * P, d_h)
    zkp = np.asarray(zk_pages).reshape(n_pages * P, H, r)
    zvp = np.asarray(zv_pages).reshape(n_pages * P, H, r)
    out = {"k_shared": np.zeros((B, L_cap, d_h), kp.dtype), "v_shared": np.zeros((B, L_cap, d_h), kp.dtype),
           "z_k": np.zeros((B, H, L_cap, r), kp.dtype), "z_v": np.zeros((B, H, L_cap, r), kp.dtype)}
    for b in range(B):
        for t in range(max(0, min(int(seq_lens[b]), L_cap))):
            g = pool_row(block_table, b, t, page_rows)
            if plant == 1:  # the row within the page taken from the wrong end
                g = int(block_table[b][t // page_rows]) * page_rows + (page_rows - 1 - t % page_rows)
            out["k_shared"][b, t] = kp[g]
            out["v_shared"][b, t] = vp[g]
            out["z_k"][b, :, t] = zkp[g]
            out["z_v"][b, :, t] = zvp[g]
    return out


def append(k_pages, v_pages, zk_pages, zv_pages, block_table, seq_lens, page_rows: int, max_pages: int, k_new,
           v_new, zk_new, zv_new) -> None:
    """One new row per sequence written in place at logical row seq_lens[b], which then grows by one; a full
    sequence (seq_lens[b] == max_pages * page_rows) or a negative length is left unchanged."""
    P = page_rows
    H, r = np.asarray(zk_pages).shape[2:]
    for b in range(len(seq_lens)):
        j = int(seq_lens[b])
        if j < 0 or j >= max_pages * P:
            continue
        g = pool_row(block_table, b, j, P)
        page, row = divmod(g, P)
        k_pages[page, row] = k_new[b]
        v_pages[page, row] = v_new[b]
        if r:
            zk_pages[page, row] = zk_new[b]
            zv_pages[page, row] = zv_new[b]
        seq_lens[b] = j + 1
