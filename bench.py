#!/usr/bin/env python3
"""Benchmark of LRKV factored decode on one MI355X.

One step is one decode step of the whole path on a batch of sequences:
  append the new token's projected rows + absorb the query (p = q B^K), one
  launch -> split-L partial pass -> split merge + B^V epilogue,
all through the C ABI on one HIP stream, with the inputs resident in HBM.  A
workload with several independent layers (the 24-layer one) runs every layer
in turn in each step, each with its own cache, query and bases.
Before the timed region the caches hold L - 1 - warmup rows per sequence, so
the first timed step decodes over exactly L rows; every step appends one row,
so step k decodes over L + k rows.

Output: one JSON line with the metric (cached-token·heads/s over the timed
steps), achieved HBM bandwidth, the roofline of the dominant kernel (the
split pass, timed live with HIP events on the launch stream) and the CPU
reference timed on the host on a bounded sample of the same workload.

The steps are timed three times from the same starting lengths: once as they
are (the step time and the metric), then with a HIP event pair around each
decode call (the split pass's own duration), then with one event at every step
boundary (per-step latency quantiles).  Event pairs cost 3-6 us per step on the
bf16 kernels and about 20 us on the fp32 rank-0 step, so they are kept out of
the step time; where the decode call is a fused step (the whole step), its
duration for the roofline comes from the step-boundary pass.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LRKV decode cached-token·heads/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def launch_config(w, steps: int, capacity: int = 0):
    """(L_cap, max_len) of a benchmark run of `steps` timed steps on workload w: room for the appended rows,
    rounded up to whole 256-row pages, unless a capacity is given.  The full-size parity tests use the same."""
    import synth
    L_max = int(synth.seq_lengths(w).max())
    L_cap = (L_max + steps + 255) // 256 * 256
    if capacity:
        assert capacity >= L_max + steps and capacity % 32 == 0
        L_cap = capacity
    return L_cap, L_max + steps


# the sources that determine the bf16 split kernel's code and launch configuration
SPLIT_KERNEL_SOURCES = ("k_decode_mfma.hpp", "k_decode_mfma_part_d128_n0.hip", "k_decode_mfma_part_d128_s.hip",
                        "k_decode_mfma.hip", "k_decode_mfma_f32.hip", "lrkv_device.hpp", "lrkv_internal.hpp",
                        "lrkv_step.hpp", "k_cache.hip", "k_merge.hip", "lrkv_api.cpp")


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for name in SPLIT_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_shared_kv_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, launch_bytes: float, kind: str = "split"):
    """HBM traffic per launch of the dominant kernel (kind "split": the split pass; "step": the fused decode
    step) from the committed rocprofv3 counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", f"{kind}_kernel_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_digest = re.search(r"kernel sources digest:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per " + kind + r" launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_digest or not m_bytes or m_digest.group(1) != kernel_sources_digest():
        return None
    return float(m_bytes.group(1))


def host_cores():
    """CPU cores this process may use: the affinity mask, further limited by OMP_NUM_THREADS when that is set
    (the share of the host a GPU job is granted)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def read_sq_counters(workload: str, kind: str = "split"):
    """Matrix-core and VALU activity of the split kernel from the committed rocprofv3 counter summary, if it
    matches these sources: the counted bf16 MFMA FLOP, the matrix cores' busy fraction, and the fractions of
    wave time spent issuing VALU instructions and waiting."""
    path = os.path.join(ROOT, "profiles", f"{kind}_kernel_{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_digest = re.search(r"kernel sources digest:\s*`?([0-9a-f]{16})", text)
    if not m_digest or m_digest.group(1) != kernel_sources_digest():
        return None
    fields = {"mfma_flop_per_launch": r"bf16 MFMA FLOP per " + kind + r" launch \(counter\):\s*([0-9.eE+]+)",
              "mfma_busy_frac": r"MFMA busy fraction of the " + kind + r" launch \(counter\):\s*([0-9.eE+-]+)",
              "valu_issue_frac": r"VALU issue fraction of wave time:\s*([0-9.eE+-]+)",
              "wait_frac": r"Wait fraction of wave time:\s*([0-9.eE+-]+)"}
    out = {}
    for k, pat in fields.items():
        m = re.search(pat, text)
        if not m:
            return None
        out[k] = float(m.group(1))
    out["source"] = os.path.relpath(path, ROOT)
    return out


def cpu_baseline(w, lens, budget_s: float, threads: int):
    """The fp64 CPU reference, as it stands, on (b, h) pairs of this workload until ~budget_s of wall time."""
    import numpy as np
    import oracle
    import synth

    done_tokens, elapsed, npairs = 0, 0.0, 0
    seqs = list(range(w.batch))
    for b in seqs:
        n = int(lens[b])
        s = synth.gen_sequence(w, 0, b, n)
        q = synth.gen_small(w, 0, "q")[b:b + 1]
        Bk, Bv = synth.gen_small(w, 0, "B_k"), synth.gen_small(w, 0, "B_v")
        one = np.array([n], dtype=np.int32)
        heads = list(range(w.H))
        step = max(1, threads)
        for i in range(0, len(heads), step):
            pairs = [(0, h) for h in heads[i:i + step]]
            t0 = time.perf_counter()
            oracle.lrkv_decode(w.dtype, q, s["k_shared"][None], s["v_shared"][None], s["z_k"][None], s["z_v"][None],
                               Bk, Bv, one, pairs=pairs, threads=threads)
            elapsed += time.perf_counter() - t0
            done_tokens += n * len(pairs)
            npairs += len(pairs)
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    return {"value": done_tokens / elapsed, "unit": "cached-token·heads/s", "cores": threads, "kind": "oracle",
            "sample": f"{npairs} of {w.batch * w.H} (sequence, head) pairs of this workload at its full lengths "
                      f"({done_tokens} cached-token·heads, {elapsed:.1f} s wall, fp64 rebuild-then-attend, "
                      f"OpenMP over pairs)"}


def settle_and_probe(stream, seconds: float = 0.25):
    """Keep the GPU streaming for about `seconds` before anything is timed, and measure its streaming-read
    bandwidth meanwhile: lrkv_read_probe reads a 1 GiB buffer once per launch (HIP events on the stream).
    After the inputs are generated on the host (seconds for the larger workloads) the GPU has idled, and the
    first milliseconds of work run measurably slower; the timed steps start after this.  Returns the best
    probe read rate in GB/s."""
    import torch

    import rank_shared_kv_amd as lk
    probe_bytes = 1 << 30
    src = torch.ones(probe_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(lk.READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    best, t0, n = None, time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds or n < 12:
        evs = []
        for _ in range(8):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            lk.lrkv_read_probe(src, probe_bytes, sink, stream)
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        for a, b in evs:
            n += 1
            if n > 2:
                ms = a.elapsed_time(b)
                best = ms if best is None else min(best, ms)
    del src
    return probe_bytes / (best / 1e3) / 1e9


def quantiles(xs):
    """p10 / median / p90 (linear interpolation) of a list of durations."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    p10, p50, p90 = np.percentile(a, [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90), "mean": float(a.mean()), "n": int(a.size)}


def materialize_bench(args):
    """Time lrkv_materialize over the workload's whole live cache: per step, K_h and V_h of every live
    (row, head) are rebuilt and written.  Bytes: the factored rows read once plus both bases, and the
    rebuilt rows written once.  With --key-scales, lrkv_key_scales over the whole history instead: the key
    factors read once plus B^K, one scale per (row, head) written."""
    import numpy as np
    import torch

    import rank_shared_kv_amd as lk
    import synth
    from synth import device as sdev

    w = synth.WORKLOADS[args.workload]
    K, W = args.steps, args.warmup
    lens = synth.seq_lengths(w)
    L_cap, max_len = launch_config(w, 0, args.capacity)
    what = "key scales" if args.key_scales else "materialise"
    log(f"bench: {what}, workload {w.name} B={w.batch} H={w.H} d_h={w.d_h} r={w.r} {w.dtype} "
        f"L_max={int(lens.max())} steps={K} warmup={W}")
    dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
    dims = lk.make_dims(w.batch, w.H, w.d_h, w.r, L_cap, lk.LRKV_F32 if w.dtype == "f32" else lk.LRKV_BF16)
    cache = lk.make_cache(dev["k_shared"], dev["v_shared"], dev["z_k"] if w.r else None,
                          dev["z_v"] if w.r else None, dev["seq_lens"])
    stream = torch.cuda.current_stream()
    bk, bv = (dev["B_k"], dev["B_v"]) if w.r else (None, None)
    if args.key_scales:
        rho = torch.empty((w.batch, L_cap, w.H), dtype=sdev.torch_dtype(w), device="cuda")
        call = lambda: lk.lrkv_key_scales(dims, cache, max_len, max_len, bk, 1e-6, rho, stream)  # noqa: E731
    else:
        K_out = torch.empty((w.batch, w.H, L_cap, w.d_h), dtype=sdev.torch_dtype(w), device="cuda")
        V_out = torch.empty_like(K_out)
        call = lambda: lk.lrkv_materialize(dims, cache, max_len, bk, bv, K_out, V_out, stream)  # noqa: E731
    settle_and_probe(stream)
    for _ in range(W):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(K):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    check = rho[0, : int(lens[0])] if args.key_scales else K_out[0, :, : int(lens[0])]
    assert bool(torch.isfinite(check.float()).all())
    us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / K
    rows = int(np.sum(lens, dtype=np.int64))
    s = w.elem_bytes
    if args.key_scales:  # the key half of the cache, B^K, and the scales
        read_bytes = lk.lrkv_cache_bytes(dims, lens.tolist()) // 2 + w.H * w.d_h * w.r * s
        write_bytes = rows * w.H * s
    else:
        read_bytes = lk.lrkv_cache_bytes(dims, lens.tolist()) + 2 * w.H * w.d_h * w.r * s
        write_bytes = 2 * rows * w.H * w.d_h * s
    gbps = (read_bytes + write_bytes) / (us * 1e-6) / 1e9
    log(f"bench: {what} {us:.1f} us per call = {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBPS:.1f}% of peak)")
    rec = {
        "metric": ("LRKV key scales of the whole history (normalised variant), row-heads/s, 1 GPU" if args.key_scales
                   else "LRKV materialised keys and values, rebuilt row-heads/s (the training / prefill form), "
                        "1 GPU"),
        "value": rows * w.H / (us * 1e-6), "unit": "row·heads/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name + ("+key_scales" if args.key_scales else "+materialise"), "batch": w.batch, "H": w.H, "d_h": w.d_h, "r": w.r,
                   "L": int(lens.max()), "L_cap": L_cap},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "lrkv_key_scales" if args.key_scales else "lrkv_materialize",
                     "algorithmic_bytes_per_launch": read_bytes + write_bytes, "read_bytes": read_bytes,
                     "write_bytes": write_bytes, "avg_launch_us": us,
                     "timing": f"HIP events around each of {K} launches"},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_context")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of CPU-reference wall time (0: skip)")
    ap.add_argument("--capacity", type=int, default=0,
                    help="cache rows allocated per sequence (default: the context plus the timed appends, "
                         "rounded up to 256)")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole layer step: project + append (d_model = H*d_h), absorb, decode, output "
                         "projection (random seeded weights)")
    ap.add_argument("--queries", type=int, default=1, metavar="Q",
                    help="multi-token decode: Q new query tokens per sequence and step, causal inside the chunk "
                         "(each step appends Q rows, absorbs B*Q queries and runs lrkv_decode_multi)")
    ap.add_argument("--norm", action="store_true",
                    help="normalised variant: each step appends a row, computes its key scales, normalises the "
                         "query (gain folded in), absorbs it and runs lrkv_decode_normed")
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE_ROWS",
                    help="paged cache: the rows in PAGE_ROWS-row pages of a shuffled pool (power of two >= 32; the "
                         "capacity is rounded up to whole pages); each step appends through the block table and "
                         "runs lrkv_decode_paged")
    ap.add_argument("--rope", action="store_true",
                    help="rotary variant: each step appends a row and runs lrkv_decode_rope (every head's key "
                         "rebuilt and turned at its position)")
    ap.add_argument("--materialize", action="store_true",
                    help="materialised path: each step rebuilds K_h and V_h of every live row and head "
                         "(lrkv_materialize, the training / prefill form)")
    ap.add_argument("--key-scales", action="store_true",
                    help="normalised variant's whole-history pass: each step computes the key scale of every live "
                         "row and head (lrkv_key_scales with n_last = the whole history, as after a prefill)")
    ap.add_argument("--layers", type=int, default=0,
                    help="independent layers decoded back to back per step, each with its own cache, query and "
                         "bases (default: the workload's layer count, 24 for mid_24layer; plain decode only)")
    ap.add_argument("--separate", action="store_true",
                    help="plain decode: time the step as three launches (append + absorb, split pass, merge) instead "
                         "of the fused decode step")
    ap.add_argument("--no-stream-probe", action="store_true",
                    help="do not report the streaming-read probe (it still runs untimed before the timed steps, to "
                         "bring the GPU to its streaming state)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (for scaling HBM counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {n * 4} bytes 5 times")
        return
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    if sum([args.queries > 1, args.layer, args.norm, args.paged > 0, args.rope, args.materialize,
            args.key_scales]) > 1:
        print("bench.py: --queries, --layer, --norm, --paged, --rope, --materialize and --key-scales do not "
              "combine", file=sys.stderr)
        sys.exit(2)
    if args.materialize or args.key_scales:
        return materialize_bench(args)

    import numpy as np
    import torch

    import rank_shared_kv_amd as lk
    import synth
    from synth import device as sdev

    w = synth.WORKLOADS[args.workload]
    K, W, Q = args.steps, args.warmup, max(1, args.queries)
    plain = not (Q > 1 or args.layer or args.norm or args.paged or args.rope)
    n_layers = args.layers or (w.layers if plain else 1)
    if n_layers > 1 and not plain:
        print("bench.py: several layers per step are timed for the plain decode only", file=sys.stderr)
        sys.exit(2)
    lens_full = synth.seq_lengths(w)
    for layer in range(1, n_layers):  # the layers' caches share one capacity and length bound
        assert synth.seq_lengths(w, layer).tolist() == lens_full.tolist()
    L_cap, max_len = launch_config(w, K * Q, args.capacity)
    if args.paged:
        L_cap = (L_cap + args.paged - 1) // args.paged * args.paged
    start_lens = lens_full - Q - W * Q
    assert int(start_lens.min()) >= 0
    log(f"bench: workload {w.name} B={w.batch} H={w.H} d_h={w.d_h} r={w.r} {w.dtype} L_max={int(lens_full.max())} "
        f"steps={K} warmup={W} queries={Q} layers={n_layers}")
    t0 = time.time()
    devs = []
    for layer in range(n_layers):  # every layer its own seeded cache, query and bases
        d_l = sdev.fill_layer(w, layer, L_cap=L_cap, lengths=lens_full)
        d_l["seq_lens"].copy_(torch.from_numpy(start_lens.astype(np.int32)).cuda())
        devs.append(d_l)
    dev = devs[0]
    rows = sdev.new_rows(w)
    torch.cuda.synchronize()
    log(f"bench: inputs resident in HBM ({time.time() - t0:.1f} s to generate and copy)")

    dtype_code = lk.LRKV_F32 if w.dtype == "f32" else lk.LRKV_BF16
    dims = lk.make_dims(w.batch, w.H, w.d_h, w.r, L_cap, dtype_code)
    caches = [lk.make_cache(d_l["k_shared"], d_l["v_shared"], d_l["z_k"] if w.r else None,
                            d_l["z_v"] if w.r else None, d_l["seq_lens"]) for d_l in devs]
    cache = caches[0]
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    ps = [torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda") for _ in devs]
    outs = [torch.empty((w.batch, w.H, w.d_h), dtype=torch.float32, device="cuda") for _ in devs]
    p, out = ps[0], outs[0]
    S, chunk = lk.lrkv_decode_num_splits(dims, max_len)
    # plain decode: the whole step (append, absorb, split pass, merge) in one launch where the library fuses it
    # (bf16 matrix-core shapes), or as the split pass with the append and the merge (fp32 rank 0)
    fused = plain and not args.separate and lk.lrkv_decode_step_fused(dims, max_len)
    if fused:
        nbytes_step = lk.lrkv_decode_step_workspace_bytes(dims, max_len)
        ws_step = torch.zeros(nbytes_step // 4, dtype=torch.float32, device="cuda")  # counter words start at zero
    if Q > 1:
        nbytes = lk.lrkv_decode_multi_workspace_bytes(dims, Q, max_len)
        ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
        dims_q = lk.make_dims(w.batch * Q, w.H, w.d_h, w.r, L_cap, dtype_code)
        q_multi = sdev.to_device(synth.normal(8803, 1.0, w.batch * Q * w.H * w.d_h, w.dtype)
                                 .reshape(w.batch, Q, w.H, w.d_h))
        p = torch.empty((w.batch, Q, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
        out = torch.empty((w.batch, Q, w.H, w.d_h), dtype=torch.float32, device="cuda")
        S, chunk = None, None
    if args.norm:
        eps = 1e-6
        rho = torch.empty((w.batch, L_cap, w.H), dtype=sdev.torch_dtype(w), device="cuda")
        lk.lrkv_key_scales(dims, cache, max_len, max_len, dev["B_k"] if w.r else None, eps, rho)
        g_q = sdev.to_device(synth.gain(8804, (w.H, w.d_h), w.dtype))
        g_k = sdev.to_device(synth.gain(8805, (w.H, w.d_h), w.dtype))
        q_eff = torch.empty_like(dev["q"])
    if args.paged:  # the same rows in a shuffled pool of pages (pages past each sequence's need are spare)
        P = args.paged
        maxp = L_cap // P
        n_pages = w.batch * maxp
        perm = torch.from_numpy(np.random.default_rng(12345).permutation(n_pages).astype(np.int32))
        table = perm.reshape(w.batch, maxp).cuda()
        pools = {}
        for name in ("k_shared", "v_shared") + (("z_k", "z_v") if w.r else ()):
            src = dev[name]
            pool = torch.empty((n_pages, P) + tuple(src.shape[2:]), dtype=src.dtype, device="cuda")
            pool[table.reshape(-1).long()] = src.reshape((w.batch * maxp, P) + tuple(src.shape[2:]))
            pools[name] = pool
        pcache = lk.make_paged_cache(pools["k_shared"], pools["v_shared"], pools.get("z_k"), pools.get("z_v"), table,
                                     dev["seq_lens"], P, maxp, n_pages)
    if args.rope:
        rope_cs = torch.empty((L_cap, w.d_h // 2, 2), dtype=torch.float32, device="cuda")
        lk.lrkv_rope_table(w.d_h, L_cap, 10000.0, rope_cs)
        nbytes = lk.lrkv_decode_rope_workspace_bytes(dims, max_len)
        ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
        # the rotary plan is its own: its split count from its workspace (one record of every head per
        # split); its row granule is not exported
        S, chunk = nbytes // (4 * w.H * ((w.d_h + w.r + 2 + 3) // 4 * 4)), None
    stream = torch.cuda.current_stream()
    pp = p if w.r else None
    bv = dev["B_v"] if w.r else None
    zk_new = rows["zk_new"] if w.r else None
    zv_new = rows["zv_new"] if w.r else None

    ev_pairs = []
    layer_ev = []  # (project start, project end, output projection start, output projection end)
    d_model = w.H * w.d_h
    if args.layer:
        import math
        n_in = w.H * w.d_h + 2 * w.d_h + 2 * w.H * w.r
        W_in = sdev.to_device(synth.normal(8800, 1.0 / math.sqrt(d_model), n_in * d_model, w.dtype)
                              .reshape(n_in, d_model))
        W_o = sdev.to_device(synth.normal(8801, 1.0 / math.sqrt(d_model), d_model * d_model, w.dtype)
                             .reshape(d_model, d_model))
        x_new = sdev.to_device(synth.normal(8802, 1.0, w.batch * d_model, w.dtype).reshape(w.batch, d_model))
        q_step = torch.empty((w.batch, w.H, w.d_h), dtype=sdev.torch_dtype(w), device="cuda")
        y_step = torch.empty((w.batch, d_model), dtype=torch.float32, device="cuda")

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def step_multi(timed: bool):
        for _ in range(Q):
            lk.lrkv_cache_append(dims, cache, rows["k_new"], rows["v_new"], zk_new, zv_new, stream)
        if w.r:
            lk.lrkv_absorb_query(dims_q, q_multi, dev["B_k"], p, stream)
        if timed:
            e0 = ev()
        lk.lrkv_decode_multi(dims, Q, cache, max_len, q_multi, p if w.r else None, bv, out, ws, nbytes, stream)
        if timed:
            ev_pairs.append((e0, ev()))

    def step_norm(timed: bool):
        lk.lrkv_cache_append(dims, cache, rows["k_new"], rows["v_new"], zk_new, zv_new, stream)
        lk.lrkv_key_scales(dims, cache, max_len, 1, dev["B_k"] if w.r else None, eps, rho, stream)
        lk.lrkv_norm_query(dims, dev["q"], g_q, g_k, eps, q_eff, stream)
        if w.r:
            lk.lrkv_absorb_query(dims, q_eff, dev["B_k"], p, stream)
        if timed:
            e0 = ev()
        lk.lrkv_decode_normed(dims, cache, rho, max_len, q_eff, pp, bv, out, ws, nbytes, stream)
        if timed:
            ev_pairs.append((e0, ev()))

    def step_paged(timed: bool):
        lk.lrkv_paged_append(dims, pcache, rows["k_new"], rows["v_new"], zk_new, zv_new, stream)
        if w.r:
            lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p, stream)
        if timed:
            e0 = ev()
        lk.lrkv_decode_paged(dims, pcache, max_len, dev["q"], pp, bv, out, ws, nbytes, stream)
        if timed:
            ev_pairs.append((e0, ev()))

    def step_rope(timed: bool):
        lk.lrkv_cache_append(dims, cache, rows["k_new"], rows["v_new"], zk_new, zv_new, stream)
        if timed:
            e0 = ev()
        lk.lrkv_decode_rope(dims, cache, max_len, dev["q"], dev["B_k"] if w.r else None, rope_cs, bv, out, ws,
                            nbytes, stream)
        if timed:
            ev_pairs.append((e0, ev()))

    def step(timed: bool):
        if Q > 1:
            return step_multi(timed)
        if args.rope:
            return step_rope(timed)
        if args.paged:
            return step_paged(timed)
        if args.norm:
            return step_norm(timed)
        if args.layer:
            e_p0 = ev() if timed else None
            lk.lrkv_project_append(dims, d_model, cache, x_new, W_in, q_step, stream)
            e_p1 = ev() if timed else None
            q_use = q_step
            if w.r:
                lk.lrkv_absorb_query(dims, q_use, dev["B_k"], p, stream)
        else:
            # every layer in turn: the fused step (one launch), or the append and the query absorption in one
            # launch, the split pass, the merge (the layers share the workspace: each layer's merge has read it
            # before the next layer's split pass writes it)
            for d_l, c_l, p_l, o_l in zip(devs, caches, ps, outs):
                pp_l = p_l if w.r else None
                if fused:
                    if timed:
                        e0 = ev()
                    lk.lrkv_decode_step(dims, c_l, max_len, rows["k_new"], rows["v_new"], zk_new, zv_new, d_l["q"],
                                        d_l["B_k"] if w.r else None, d_l["B_v"] if w.r else None, pp_l, o_l, ws_step,
                                        nbytes_step, stream)
                    if timed:
                        ev_pairs.append((e0, ev()))
                    continue
                lk.lrkv_append_absorb(dims, c_l, rows["k_new"], rows["v_new"], zk_new, zv_new, d_l["q"],
                                      d_l["B_k"] if w.r else None, pp_l, stream)
                if timed:
                    e0 = ev()
                lk.lrkv_decode_partial(dims, c_l, max_len, d_l["q"], pp_l, ws, nbytes, stream)
                if timed:
                    ev_pairs.append((e0, ev()))
                lk.lrkv_decode_merge(dims, d_l["seq_lens"], max_len, d_l["B_v"] if w.r else None, o_l, ws, nbytes,
                                     stream)
            return
        if timed:
            e0 = ev()
        lk.lrkv_decode_partial(dims, cache, max_len, q_use, pp, ws, nbytes, stream)
        if timed:
            ev_pairs.append((e0, ev()))
        lk.lrkv_decode_merge(dims, dev["seq_lens"], max_len, bv, out, ws, nbytes, stream)
        if args.layer:
            e_o0 = ev() if timed else None
            lk.lrkv_output_project(dims, d_model, out, W_o, y_step, stream)
            if timed:
                layer_ev.append((e_p0, e_p1, e_o0, ev()))

    def timed_pass(instrumented: bool, marks=None) -> float:
        # the same work each time: lengths back to the start, W warm-up steps, then K timed steps
        for d_l in devs:
            d_l["seq_lens"].copy_(torch.from_numpy(start_lens.astype(np.int32)).cuda())
        for _ in range(W):
            step(False)
        torch.cuda.synchronize()
        for d_l in devs:
            assert d_l["seq_lens"].cpu().numpy().tolist() == (lens_full - Q).tolist()
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for _ in range(K):
            if marks is not None:
                marks.append(ev())
            step(instrumented)
        t_end.record(stream)
        if marks is not None:
            marks.append(t_end)
        torch.cuda.synchronize()
        for d_l, o_l in zip(devs, outs):
            assert d_l["seq_lens"].cpu().numpy().tolist() == (lens_full - Q + K * Q).tolist()
            assert bool(torch.isfinite(o_l).all())
        return t_start.elapsed_time(t_end)

    stream_gbps = settle_and_probe(stream)  # untimed: the GPU streams for a while first (and the probe reads)
    total_ms = timed_pass(False)         # the step time: nothing but the step's own launches
    total_ms_events = timed_pass(True)   # the decode launches' durations
    split_ms = [a.elapsed_time(b) for a, b in ev_pairs]
    # per-step latency: a third pass with one event at every step boundary (about 1 us each)
    marks = []
    timed_pass(False, marks)
    step_us = [1e3 * marks[k].elapsed_time(marks[k + 1]) for k in range(K)]

    # work per timed step k: sequence b holds lens_full + k*Q rows, and its query i (0-based among the Q new
    # tokens) sees the rows up to and including its own, lens_full + k*Q - Q + i + 1 of them
    token_heads = n_layers * sum(int(np.sum(Q * (lens_full + k * Q) - Q * (Q - 1) // 2, dtype=np.int64)) * w.H
                                 for k in range(K))
    value = token_heads / (total_ms / 1e3)
    s_bytes = w.elem_bytes
    cache_bytes_per_step = [lk.lrkv_cache_bytes(dims, (lens_full + k * Q).tolist()) for k in range(K)]
    q_bytes = Q * w.batch * w.H * w.d_h * s_bytes
    p_bytes = Q * w.batch * w.H * w.r * 4
    basis_bytes = 2 * w.H * w.d_h * w.r * s_bytes
    out_bytes = Q * w.batch * w.H * w.d_h * 4
    step_bytes = n_layers * (sum(cache_bytes_per_step) / K + q_bytes + basis_bytes + out_bytes)
    split_bytes = sum(cache_bytes_per_step) / K + q_bytes + p_bytes  # per split launch (one layer)
    if args.norm:  # the scales are read once per step, one per (row, head)
        rho_bytes = [sum(int(x) for x in (lens_full + k)) * w.H * s_bytes for k in range(K)]
        split_bytes += sum(rho_bytes) / K
        step_bytes += sum(rho_bytes) / K
    if args.paged:  # the block table entries of the live pages
        split_bytes += w.batch * ((int(lens_full.max()) + K + args.paged - 1) // args.paged) * 4
    if args.rope:  # the rotation table rows of the live positions (no absorbed query is read)
        split_bytes += int(lens_full.max() + K) * w.d_h * 4 - p_bytes
    if Q > 1 or args.norm or args.paged or args.rope:  # the timed call is the whole decode (split + merge)
        split_bytes += out_bytes + w.H * w.d_h * w.r * s_bytes
    if fused:  # the fused launch reads the cache, q and both bases, appends the new rows and writes out
        new_row_bytes = w.batch * 2 * (w.d_h + w.H * w.r) * s_bytes
        split_bytes = (sum(cache_bytes_per_step) / K + q_bytes + basis_bytes + out_bytes + 2 * new_row_bytes
                       + 2 * p_bytes)
    split_avg_ms = pair_avg_ms = sum(split_ms) / len(split_ms)
    if fused:
        # the fused call is the whole step: its duration comes from the pass with one event at every step
        # boundary; an event pair around each call perturbs it (2-3 us a step on the bf16 step, about 20 us on
        # the fp32 rank-0 one, whose two launches the pair separates from the rest of the stream)
        split_avg_ms = sum(step_us) / len(step_us) / n_layers / 1e3
    split_gbps = split_bytes / (split_avg_ms / 1e3) / 1e9
    step_gbps = step_bytes / (total_ms / K / 1e3) / 1e9
    flops_mfma = 2 * w.d_h * (token_heads / K / n_layers)  # shared-key score tile per split launch
    mfma_util = flops_mfma / (split_avg_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    kind = "step" if fused else "split"
    traffic = (read_traffic(w.name, split_bytes, kind)
               if not (args.layer or args.norm or args.paged or args.rope) and Q == 1 else None)
    layer = None
    if args.layer:
        assert bool(torch.isfinite(y_step).all())
        proj_us = 1e3 * sum(a.elapsed_time(b) for a, b, _, _ in layer_ev) / len(layer_ev)
        outp_us = 1e3 * sum(c.elapsed_time(d) for _, _, c, d in layer_ev) / len(layer_ev)
        w_in_bytes = W_in.numel() * W_in.element_size()
        w_o_bytes = W_o.numel() * W_o.element_size()
        layer = {"d_model": d_model, "project_append_us": proj_us,
                 "project_weight_gbps": w_in_bytes / (proj_us * 1e-6) / 1e9, "project_weight_bytes": w_in_bytes,
                 "output_project_us": outp_us, "output_weight_gbps": w_o_bytes / (outp_us * 1e-6) / 1e9,
                 "output_weight_bytes": w_o_bytes,
                 "note": "project_append_us includes its length-update kernel; weights are random and seeded"}
        step_bytes += w_in_bytes + w_o_bytes  # the weights are streamed once per step
        step_gbps = step_bytes / (total_ms / K / 1e3) / 1e9
        log(f"bench: layer step: project+append {proj_us:.1f} us ({layer['project_weight_gbps']:.0f} GB/s of "
            f"weights), output projection {outp_us:.1f} us ({layer['output_weight_gbps']:.0f} GB/s)")
    log(f"bench: {K} steps in {total_ms:.3f} ms ({total_ms / K:.4f} ms/step; {total_ms_events / K:.4f} with events); "
        f"{'fused step' if fused else 'split pass' if Q == 1 and not (args.norm or args.paged or args.rope) else 'whole decode call'} "
        f"{split_avg_ms * 1e3:.1f} us "
        f"avg = {split_gbps:.0f} GB/s ({100 * split_gbps / HBM_PEAK_GBPS:.1f}% of peak); splits={S} chunk={chunk}")

    if args.no_stream_probe:
        stream_gbps = None
    else:
        log(f"bench: streaming-read probe {stream_gbps:.0f} GB/s ({100 * stream_gbps / HBM_PEAK_GBPS:.1f}% of the peak)")

    cpu = None
    if args.cpu_budget > 0:
        cores = host_cores()
        log(f"bench: timing the CPU reference on {cores} cores (~{args.cpu_budget:.0f} s), then on one core")
        cpu = cpu_baseline(w, lens_full, args.cpu_budget, cores)
        one = cpu_baseline(w, lens_full, max(2.0, args.cpu_budget / 2), 1)
        cpu.update({"nproc": os.cpu_count(),
                    "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                    "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
                    "cores_note": "every core this process may use (its affinity mask, limited by OMP_NUM_THREADS "
                                  "when set: the host share granted to a one-GPU job)",
                    "single_core": {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}})
        log(f"bench: CPU reference {cpu['value']:.3e} token·heads/s on {cpu['cores']} threads "
            f"(nproc {cpu['nproc']}), {one['value']:.3e} on one core")

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "cached-token·heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_ms / K,
        "ms_per_step_with_kernel_events": total_ms_events / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "step_us_quantiles": dict(quantiles(step_us), timing="a third pass over the same steps with one HIP "
                                  "event at every step boundary (each event adds about 1 us)"),
        "split_launch_us_quantiles": quantiles([1e3 * x for x in split_ms]),
        "per_layer_us": (total_ms / K / n_layers * 1e3) if n_layers > 1 else None,
        "config": {"workload": w.name + ("+projections" if args.layer else "") + (f"+{Q}queries" if Q > 1 else "") + ("+normalised" if args.norm else "")
                   + (f"+paged{args.paged}" if args.paged else "") + ("+rope" if args.rope else ""), "batch": w.batch, "H": w.H, "d_h": w.d_h, "r": w.r,
                   "L": int(lens_full.max()), "L_cap": L_cap, "lengths": "uniform" if w.ragged_lo is None else
                   f"uniform integers in [{w.ragged_lo}, {w.L}]", "cache_dtype": w.dtype, "accumulate": "f32",
                   "splits": S, "chunk_tokens": chunk, "queries_per_sequence": Q, "layers": n_layers,
                   "step_launches": (2 if w.dtype == "f32" else 1) if fused else None},
        "hbm_gbps_step": step_gbps,
        "hbm_frac_step": step_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": split_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": split_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "kernel": "lrkv_decode_multi (split pass + merge)" if Q > 1 else
                     "lrkv_decode_normed (split pass + merge)" if args.norm else
                     "lrkv_decode_paged (split pass + merge)" if args.paged else
                     "lrkv_decode_rope (split pass + merge)" if args.rope else
                     ("decode step (lrkv_decode_step: the split pass, which appends the token, then the merge; two "
                      "launches)" if w.dtype == "f32" else
                      "fused decode step (lrkv_decode_step: append, absorb, split pass and merge in one launch)")
                     if fused else "split pass (lrkv_decode_partial)",
                     "algorithmic_bytes_per_launch": split_bytes, "avg_launch_us": split_avg_ms * 1e3,
                     "timing": (f"HIP events at the {K} step boundaries of a third pass over the same steps, "
                                f"{n_layers} fused call(s) per step (event pairs around each call, a second pass: "
                                f"{pair_avg_ms * 1e3:.1f} us per call)") if fused else
                               (f"HIP events around each of the {K * n_layers} decode launches of a second pass "
                                "over the same steps (the step time comes from a pass without them)"),
                     "stream_read_gbps": stream_gbps,
                     "frac_of_stream_read": (split_gbps / stream_gbps) if stream_gbps else None},
        "mfma_util_shared_score": mfma_util,
        "mfma_counters": (dict(read_sq_counters(w.name, kind), note=f"rocprofv3 counters of the {kind} kernel on "
                               "this workload; the shared-score figure above is 2 d_h FLOP per cached token-head "
                               "over the live launch time, the counted FLOP include the value products (3x)")
                          if plain and read_sq_counters(w.name, kind) else None),
        "layer_step": layer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
