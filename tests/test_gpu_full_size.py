"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The cache capacity and the host length bound are the ones `bench.py` uses for a default run (context plus
50 appended rows, rounded up to 256 rows), so the split plan (splits per sequence, granule, kernel,
occupancy) is the benchmarked one.  The CPU reference rebuilds K_h and V_h per (sequence, head) pair, so
outputs are compared on every pair of the long-context workload and on sampled pairs of the larger ones,
always including the first and last head and, for ragged batches, the shortest and longest sequence.
Metric and tolerances as in test_gpu_decode.py.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, say  # noqa: E402

BENCH_STEPS = 50  # bench.py's default number of timed steps


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _fill_and_keep(w, layer, lens, L_cap, keep):
    """Generate every sequence once, copy it to the device cache, keep the host copies of `keep`."""
    dev = sdev.alloc_cache(w, L_cap)
    host = {}
    for b in range(w.batch):
        n = int(lens[b])
        s = synth.gen_sequence(w, layer, b, n)
        dev["k_shared"][b, :n].copy_(sdev.to_device(s["k_shared"]))
        dev["v_shared"][b, :n].copy_(sdev.to_device(s["v_shared"]))
        if w.r > 0:
            dev["z_k"][b, :n].copy_(sdev.to_device(s["z_k"]).transpose(0, 1))  # [H][n][r] -> [n][H][r]
            dev["z_v"][b, :n].copy_(sdev.to_device(s["z_v"]).transpose(0, 1))
        if b in keep:
            host[b] = s
    dev["q"] = sdev.to_device(synth.gen_small(w, layer, "q"))
    if w.r > 0:
        dev["B_k"] = sdev.to_device(synth.gen_small(w, layer, "B_k"))
        dev["B_v"] = sdev.to_device(synth.gen_small(w, layer, "B_v"))
    dev["seq_lens"] = torch.from_numpy(np.asarray(lens, dtype=np.int32).copy()).cuda()
    return dev, host


def _decode(w, dev, L_cap, max_len, split_calls=False):
    dims = dims_of(w, L_cap)
    cache = cache_of(dev, w.r)
    p = torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    if w.r > 0:
        lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p)
    pp = p if w.r > 0 else None
    bv = dev["B_v"] if w.r > 0 else None
    if split_calls:
        lk.lrkv_decode_partial(dims, cache, max_len, dev["q"], pp, ws, nbytes)
        lk.lrkv_decode_merge(dims, dev["seq_lens"], max_len, bv, out, ws, nbytes)
    else:
        lk.lrkv_decode(dims, cache, max_len, dev["q"], pp, bv, out, ws, nbytes)
    torch.cuda.synchronize()
    return out


def _reference(w, layer, host, lens, pairs, mqa=False):
    q_all = synth.gen_small(w, layer, "q")
    Bk = synth.gen_small(w, layer, "B_k") if w.r > 0 else None
    Bv = synth.gen_small(w, layer, "B_v") if w.r > 0 else None
    ref = np.zeros((len(pairs), w.d_h))
    for b in sorted({b for b, _ in pairs}):
        idx = [i for i, (bb, _) in enumerate(pairs) if bb == b]
        s = host[b]
        one = np.array([int(lens[b])], dtype=np.int32)
        sub = [(0, pairs[i][1]) for i in idx]
        if mqa:
            res = oracle.mqa_decode(w.dtype, q_all[b:b + 1], s["k_shared"][None], s["v_shared"][None], one, pairs=sub)
        else:
            res = oracle.lrkv_decode(w.dtype, q_all[b:b + 1], s["k_shared"][None], s["v_shared"][None],
                                     s["z_k"][None], s["z_v"][None], Bk, Bv, one, pairs=sub)
        ref[idx] = res
    return ref


def _check(w, got, ref, pairs, label):
    g = got.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    sel = np.stack([g[b, h] for (b, h) in pairs])
    err = oracle.relative_error(sel, ref)
    say(f"  {label}: max rel err {err:.3e} (tol {TOL[w.dtype]:.0e}) over {len(pairs)} sampled (b,h) pairs")
    assert err <= TOL[w.dtype], f"{label}: rel err {err} > {TOL[w.dtype]}"


def _plan_line(w, L_cap, max_len):
    S, chunk = lk.lrkv_decode_num_splits(dims_of(w, L_cap), max_len)
    return f"L_cap={L_cap} max_len={max_len} splits={S} granule={chunk}"


def test_long_context_full_size():
    w = synth.WORKLOADS["long_context"]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w)
    say(f"[case] long_context full size B={w.batch} H={w.H} r={w.r} L={int(lens.max())} {_plan_line(w, L_cap, max_len)}")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.H)]  # every (sequence, head) pair
    dev, host = _fill_and_keep(w, 0, lens, L_cap, keep=set(range(w.batch)))
    got = _decode(w, dev, L_cap, max_len)
    _check(w, got, _reference(w, 0, host, lens, pairs), pairs, "long_context")
    # the benchmark calls the two halves separately: same bits as the one-call form
    got2 = _decode(w, dev, L_cap, max_len, split_calls=True)
    assert torch.equal(got, got2)


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("name", ["long_context", "mid_24layer", "ragged_mqa_fp32"])
def test_fused_step_full_size(name):
    """The decode step the benchmark times at these workloads (lrkv_decode_step: the new token appended, p, the
    split pass and the merge in one launch) at full size: every (sequence, head) pair against the reference on
    the cache with the appended token, and the same bits as lrkv_append_absorb + lrkv_decode on a copy of the
    cache (outputs, p, lengths, the appended rows)."""
    w = synth.WORKLOADS[name]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w)
    dims = dims_of(w, L_cap)
    assert lk.lrkv_decode_step_fused(dims, max_len), "the benchmark times the fused step at this workload"
    say(f"[case] {name} fused step full size B={w.batch} H={w.H} r={w.r} L={int(lens.max())} {_plan_line(w, L_cap, max_len)}")
    dev, host = _fill_and_keep(w, 0, lens, L_cap, keep=set(range(w.batch)))
    twin = {k: dev[k].clone() for k in ("k_shared", "v_shared", "z_k", "z_v", "seq_lens")}
    rows = sdev.new_rows(w)
    outs, ps = [], []
    for fused, d in ((True, dev), (False, twin)):
        cache = cache_of(d, w.r)
        zk_new, zv_new = (rows["zk_new"], rows["zv_new"]) if w.r else (None, None)
        B_k, B_v = (dev["B_k"], dev["B_v"]) if w.r else (None, None)
        p = torch.full((w.batch, w.H, max(w.r, 1)), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
        if fused:
            nbytes = lk.lrkv_decode_step_workspace_bytes(dims, max_len)
            ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
            lk.lrkv_decode_step(dims, cache, max_len, rows["k_new"], rows["v_new"], zk_new, zv_new, dev["q"], B_k,
                                B_v, p if w.r else None, out, ws, nbytes)
            torch.cuda.synchronize()
            words = ws[lk.lrkv_decode_step_sync_offset(dims, max_len) // 4:].view(torch.int32)
            assert int(words[1]) == 0 and int(words.abs().sum()) == 0, "step counters not back at zero"
        else:
            nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
            ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
            lk.lrkv_append_absorb(dims, cache, rows["k_new"], rows["v_new"], zk_new, zv_new, dev["q"], B_k,
                                  p if w.r else None)
            lk.lrkv_decode(dims, cache, max_len, dev["q"], p if w.r else None, B_v, out, ws, nbytes)
            torch.cuda.synchronize()
        outs.append(out)
        ps.append(p)
    grown = np.minimum(lens + 1, L_cap)
    assert dev["seq_lens"].cpu().numpy().tolist() == grown.tolist()
    assert torch.equal(dev["seq_lens"], twin["seq_lens"])
    assert torch.equal(_bits(outs[0]), _bits(outs[1])), "fused step and separate calls differ"
    assert torch.equal(_bits(ps[0]), _bits(ps[1]))
    for k in ("k_shared", "v_shared", "z_k", "z_v") if w.r else ("k_shared", "v_shared"):
        for b in range(w.batch):
            n = int(lens[b])
            assert torch.equal(_bits(dev[k][b, n]), _bits(twin[k][b, n])), f"appended {k} row of sequence {b}"
    new = synth.gen_new_rows(w, 0)
    ext = {}
    for b in range(w.batch):
        s = host[b]
        ext[b] = {"k_shared": np.concatenate([s["k_shared"], new["k_new"][b][None]]),
                  "v_shared": np.concatenate([s["v_shared"], new["v_new"][b][None]]),
                  "z_k": np.concatenate([s["z_k"], new["zk_new"][b][:, None]], axis=1),
                  "z_v": np.concatenate([s["z_v"], new["zv_new"][b][:, None]], axis=1)}
    if name == "long_context":
        pairs = [(b, h) for b in range(w.batch) for h in range(w.H)]
    else:
        pairs = [(b, h) for b in range(w.batch) for h in sorted({0, (5 * b) % w.H, w.H - 1})]
    _check(w, outs[0], _reference(w, 0, ext, grown, pairs), pairs, f"{name} fused step")


@pytest.mark.parametrize("layer", list(range(24)))
def test_mid_24layer_full_size(layer):
    w = synth.WORKLOADS["mid_24layer"]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w, layer)
    say(f"[case] mid_24layer layer {layer} B={w.batch} H={w.H} r={w.r} L={int(lens.max())} "
        f"{_plan_line(w, L_cap, max_len)}")
    bs = sorted({0, (3 * layer + 1) % w.batch, (7 * layer + 5) % w.batch, w.batch - 1})
    pairs = [(b, h) for b in bs for h in sorted({0, (5 * layer + b) % w.H, w.H - 1})]
    dev, host = _fill_and_keep(w, layer, lens, L_cap, keep=set(bs))
    got = _decode(w, dev, L_cap, max_len)
    _check(w, got, _reference(w, layer, host, lens, pairs), pairs, f"mid_24layer[{layer}]")


def _ragged_pairs(w, lens):
    order = np.argsort(lens, kind="stable")
    bs = sorted({int(order[0]), int(order[1]), int(order[-1]), int(order[-2])} | set(range(0, w.batch, 9)))
    return bs, [(b, h) for b in bs for h in sorted({0, (11 * b) % w.H, w.H - 1})]


def test_ragged_full_size():
    w = synth.WORKLOADS["ragged"]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w)
    say(f"[case] ragged full size B={w.batch} H={w.H} r={w.r} lengths {int(lens.min())}..{int(lens.max())} "
        f"{_plan_line(w, L_cap, max_len)}")
    bs, pairs = _ragged_pairs(w, lens)
    dev, host = _fill_and_keep(w, 0, lens, L_cap, keep=set(bs))
    got = _decode(w, dev, L_cap, max_len)
    _check(w, got, _reference(w, 0, host, lens, pairs), pairs, "ragged")


def test_ragged_r0_fp32_full_size_matches_mqa():
    w = synth.WORKLOADS["ragged_mqa_fp32"]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w)
    say(f"[case] ragged r=0 fp32 full size B={w.batch} H={w.H} lengths {int(lens.min())}..{int(lens.max())} "
        f"{_plan_line(w, L_cap, max_len)}")
    bs, pairs = _ragged_pairs(w, lens)
    dev, host = _fill_and_keep(w, 0, lens, L_cap, keep=set(bs))
    got = _decode(w, dev, L_cap, max_len)
    _check(w, got, _reference(w, 0, host, lens, pairs, mqa=True), pairs, "ragged_mqa_fp32")


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_small_configs_in_bench_launch_config(name):
    w = synth.WORKLOADS[name]
    L_cap, max_len = bench.launch_config(w, BENCH_STEPS)
    lens = synth.seq_lengths(w)
    say(f"[case] {name} all pairs {_plan_line(w, L_cap, max_len)}")
    pairs = [(b, h) for b in range(w.batch) for h in range(w.H)]
    dev, host = _fill_and_keep(w, 0, lens, L_cap, keep=set(range(w.batch)))
    got = _decode(w, dev, L_cap, max_len)
    _check(w, got, _reference(w, 0, host, lens, pairs), pairs, name)
