"""Put seeded workload inputs into GPU memory (torch tensors).  Plumbing only.

Large caches are generated one sequence at a time on the host and copied into
preallocated device tensors, so host memory stays at one sequence's worth.
The generators (and the oracle) index latents per head, [b][h][j][i]; the
device cache stores them token-major, [b][j][h][i].
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import Workload, gen_new_rows, gen_sequence, gen_small, seq_lengths


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 -> torch.float32; uint16 bf16 bit patterns -> torch.bfloat16."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def alloc_cache(w: Workload, L_cap: Optional[int] = None, device="cuda") -> Dict[str, torch.Tensor]:
    cap = w.cap if L_cap is None else L_cap
    dt = torch_dtype(w)
    r = max(w.r, 0)
    return {"k_shared": torch.zeros((w.batch, cap, w.d_h), dtype=dt, device=device),
            "v_shared": torch.zeros((w.batch, cap, w.d_h), dtype=dt, device=device),
            "z_k": torch.zeros((w.batch, cap, w.H, r), dtype=dt, device=device),
            "z_v": torch.zeros((w.batch, cap, w.H, r), dtype=dt, device=device)}


def fill_layer(w: Workload, layer: int = 0, L_cap: Optional[int] = None, lengths: Optional[np.ndarray] = None,
               device="cuda") -> Dict[str, torch.Tensor]:
    """All inputs of one layer on the device; cache rows past each sequence's length stay zero."""
    lens = seq_lengths(w, layer) if lengths is None else np.asarray(lengths, dtype=np.int32)
    cap = w.cap if L_cap is None else L_cap
    assert int(lens.max(initial=0)) <= cap
    dev = alloc_cache(w, cap, device)
    for b in range(w.batch):
        n = int(lens[b])
        if n == 0:
            continue
        s = gen_sequence(w, layer, b, n)
        dev["k_shared"][b, :n].copy_(to_device(s["k_shared"], device))
        dev["v_shared"][b, :n].copy_(to_device(s["v_shared"], device))
        if w.r > 0:
            # generated per head ([H][n][r]); stored token-major ([n][H][r])
            dev["z_k"][b, :n].copy_(to_device(s["z_k"], device).transpose(0, 1))
            dev["z_v"][b, :n].copy_(to_device(s["z_v"], device).transpose(0, 1))
    dev["q"] = to_device(gen_small(w, layer, "q"), device)
    if w.r > 0:
        dev["B_k"] = to_device(gen_small(w, layer, "B_k"), device)
        dev["B_v"] = to_device(gen_small(w, layer, "B_v"), device)
    else:
        dev["B_k"] = torch.zeros((w.H, w.d_h, 0), dtype=torch_dtype(w), device=device)
        dev["B_v"] = torch.zeros((w.H, w.d_h, 0), dtype=torch_dtype(w), device=device)
    dev["seq_lens"] = torch.from_numpy(lens.copy()).to(device)
    return dev


def new_rows(w: Workload, layer: int = 0, device="cuda") -> Dict[str, torch.Tensor]:
    return {k: to_device(v, device) for k, v in gen_new_rows(w, layer).items()}
