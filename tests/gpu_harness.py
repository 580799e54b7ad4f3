"""Shared helpers of the GPU tests: run the library through its C ABI and
compare with the CPU reference.  Not a test module itself."""
from __future__ import annotations

import sys
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

# Tolerances, on the metric max over (b, h) of ||gpu - ref||_inf / ||ref||_inf:
#   fp32 inputs: 1e-5 relative; bf16 caches with fp32 accumulation: 2e-3.
TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_of(w: synth.Workload, L_cap: Optional[int] = None) -> lk.Dims:
    return lk.make_dims(w.batch, w.H, w.d_h, w.r, w.cap if L_cap is None else L_cap,
                        lk.LRKV_F32 if w.dtype == "f32" else lk.LRKV_BF16)


def cache_of(dev: Dict[str, torch.Tensor], r: int) -> lk.Cache:
    return lk.make_cache(dev["k_shared"], dev["v_shared"], dev["z_k"] if r > 0 else None,
                         dev["z_v"] if r > 0 else None, dev["seq_lens"])


def gpu_decode(w: synth.Workload, dev: Dict[str, torch.Tensor], max_len: int, L_cap: Optional[int] = None,
               stream=None, split_calls: bool = False) -> torch.Tensor:
    """absorb + decode through the C ABI; returns out [batch, H, d_h] fp32."""
    dims = dims_of(w, L_cap)
    cache = cache_of(dev, w.r)
    p = torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    if w.r > 0:
        lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p, stream)
    pp = p if w.r > 0 else None
    bv = dev["B_v"] if w.r > 0 else None
    if split_calls:
        lk.lrkv_decode_partial(dims, cache, max_len, dev["q"], pp, ws, nbytes, stream)
        lk.lrkv_decode_merge(dims, dev["seq_lens"], max_len, bv, out, ws, nbytes, stream)
    else:
        lk.lrkv_decode(dims, cache, max_len, dev["q"], pp, bv, out, ws, nbytes, stream)
    torch.cuda.synchronize()
    return out


def host_inputs_for(w: synth.Workload, layer: int, b: int, rows: int) -> Dict[str, np.ndarray]:
    """Host arrays of one sequence (batch of 1) for the reference."""
    s = synth.gen_sequence(w, layer, b, rows)
    q = synth.gen_small(w, layer, "q")[b:b + 1]
    out = {"q": q, "k_shared": s["k_shared"][None], "v_shared": s["v_shared"][None], "z_k": s["z_k"][None],
           "z_v": s["z_v"][None], "seq_lens": np.array([rows], dtype=np.int32)}
    if w.r > 0:
        out["B_k"] = synth.gen_small(w, layer, "B_k")
        out["B_v"] = synth.gen_small(w, layer, "B_v")
    else:
        np_dt = np.float32 if w.dtype == "f32" else np.uint16
        out["B_k"] = out["B_v"] = np.zeros((w.H, w.d_h, 0), dtype=np_dt)
    return out


def oracle_pairs(w: synth.Workload, layer: int, lens: np.ndarray, pairs: Sequence[Tuple[int, int]],
                 mqa: bool = False) -> np.ndarray:
    """Reference outputs for the given (b, h) pairs, one sequence at a time."""
    out = np.zeros((len(pairs), w.d_h))
    by_b: Dict[int, List[int]] = {}
    for i, (b, h) in enumerate(pairs):
        by_b.setdefault(b, []).append(i)
    for b, idx in by_b.items():
        x = host_inputs_for(w, layer, b, int(lens[b]))
        sub = [(0, pairs[i][1]) for i in idx]
        if mqa:
            res = oracle.mqa_decode(w.dtype, x["q"], x["k_shared"], x["v_shared"], x["seq_lens"], pairs=sub)
        else:
            res = oracle.lrkv_decode(w.dtype, x["q"], x["k_shared"], x["v_shared"], x["z_k"], x["z_v"], x["B_k"],
                                     x["B_v"], x["seq_lens"], pairs=sub)
        out[idx] = res
    return out


def compare(w: synth.Workload, got: torch.Tensor, ref: np.ndarray, pairs: Sequence[Tuple[int, int]],
            label: str) -> float:
    g = got.detach().cpu().numpy().astype(np.float64)
    sel = np.stack([g[b, h] for (b, h) in pairs])
    assert np.all(np.isfinite(sel)), f"{label}: non-finite output"
    err = oracle.relative_error(sel, ref)
    say(f"  {label}: max rel err {err:.3e} (tol {TOL[w.dtype]:.0e}) over {len(pairs)} (b,h) pairs")
    assert err <= TOL[w.dtype], f"{label}: rel err {err} > {TOL[w.dtype]}"
    return err
