"""GPU tests of the paged cache through the C ABI.

A paged cache holds the same rows as a contiguous one, in pool pages chosen by a block table (here a seeded
permutation of the pool, with spare pages that hold NaN and are never referenced).  The paged decode runs the
same split plan as the contiguous one, so for every shape whose plan is not the fp32 matrix-core kernel the two
are compared bit for bit; every case is also compared with the reference decode of the rows gathered back
from the device pools (oracle.paged.gather), metric and tolerances as in test_gpu_decode.py.  Rows past each
sequence's length hold NaN in both layouts: they share the last 32-row block of a page and must never reach
the result.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import rank_shared_kv_amd as lk
import synth
from oracle import paged as opaged
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, gpu_decode, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _workload(dtype, B, H, d_h, r, L_cap):
    return synth.WORKLOADS["small_bf16"].with_(name="paged", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L_cap,
                                               L_cap=L_cap, ragged_lo=None)


def _poison_tail(w, dev, lens):
    """NaN in every cache row at or past each sequence's length."""
    for b, n in enumerate(lens):
        for name in ("k_shared", "v_shared") + (("z_k", "z_v") if w.r else ()):
            dev[name][b, int(n):] = float("nan")


def _to_pages(w, dev, P, spare, seed):
    """Pools holding the device cache's rows in seeded random pages; spare pages hold NaN."""
    B, L_cap = w.batch, w.cap
    maxp = L_cap // P
    n_pages = B * maxp + spare
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * maxp].astype(np.int32)
    table = torch.from_numpy(perm.reshape(B, maxp).copy()).cuda()
    idx = table.reshape(-1).long()
    pools = {}
    for name, pname in (("k_shared", "k_pages"), ("v_shared", "v_pages"), ("z_k", "zk_pages"), ("z_v", "zv_pages")):
        if name.startswith("z") and not w.r:
            pools[pname] = None
            continue
        src = dev[name]
        shape = (n_pages, P) + tuple(src.shape[2:])
        pool = torch.full(shape, float("nan"), dtype=src.dtype, device="cuda")
        pool[idx] = src.reshape((B * maxp, P) + tuple(src.shape[2:]))
        pools[pname] = pool
    seq_lens = dev["seq_lens"].clone()
    pc = lk.make_paged_cache(pools["k_pages"], pools["v_pages"], pools["zk_pages"], pools["zv_pages"], table, seq_lens,
                             P, maxp, n_pages)
    return pc, pools, table, seq_lens, n_pages


def _paged_decode(w, dev, pc, max_len):
    dims = dims_of(w)
    p = torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    if w.r:
        lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p)
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_decode_paged(dims, pc, max_len, dev["q"], p if w.r else None, dev["B_v"] if w.r else None, out, ws,
                         nbytes)
    torch.cuda.synchronize()
    return out


def _host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _reference_from_pools(w, pools, table, lens, P, maxp):
    """The reference decode of the rows gathered back from the device pools."""
    np_dt = np.uint16 if w.dtype == "bf16" else np.float32
    k, v = _host(pools["k_pages"]), _host(pools["v_pages"])
    if w.r:
        zk, zv = _host(pools["zk_pages"]), _host(pools["zv_pages"])
    else:
        zk = zv = np.zeros(k.shape[:2] + (w.H, 0), np_dt)
    c = opaged.gather(k, v, zk, zv, table.cpu().numpy(), lens, P, maxp)
    Bk = synth.gen_small(w, 0, "B_k") if w.r else np.zeros((w.H, w.d_h, 0), np_dt)
    Bv = synth.gen_small(w, 0, "B_v") if w.r else np.zeros((w.H, w.d_h, 0), np_dt)
    return oracle.lrkv_decode(w.dtype, synth.gen_small(w, 0, "q"), c["k_shared"], c["v_shared"], c["z_k"], c["z_v"],
                              Bk, Bv, np.asarray(lens, dtype=np.int32)).reshape(w.batch, w.H, w.d_h)


CASES = [  # (dtype, batch, H, d_h, r, L_cap, page_rows, lengths); plan: bf16 matrix cores unless noted
    ("bf16", 3, 32, 128, 64, 512, 64, [500, 33, 1]),
    ("bf16", 2, 8, 64, 16, 256, 32, [256, 97]),
    ("bf16", 3, 16, 128, 32, 1024, 256, [1000, 0, 257]),
    ("bf16", 2, 8, 64, 0, 128, 128, [100, 31]),
    ("bf16", 2, 4, 48, 12, 256, 64, [200, 65]),     # general kernel
    ("f32", 2, 4, 16, 4, 128, 32, [128, 3]),        # general kernel
    ("f32", 2, 32, 128, 0, 256, 64, [250, 64]),     # fp32 matrix-core shape: paged runs the general kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}_P{c[6]}")
def test_paged_decode(case):
    dtype, B, H, d_h, r, L_cap, P, lens = case
    w = _workload(dtype, B, H, d_h, r, L_cap)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] paged decode {case}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    _poison_tail(w, dev, lens)
    max_len = int(lens.max())
    pc, pools, table, _, _ = _to_pages(w, dev, P, spare=3, seed=31 + B + H)
    got = _paged_decode(w, dev, pc, max_len)
    fp32_mfma = dtype == "f32" and r == 0 and d_h in (64, 128) and H in (8, 16, 32)
    if not fp32_mfma:
        want = gpu_decode(w, dev, max_len)
        assert torch.equal(got, want), "paged and contiguous decode differ"
    ref = _reference_from_pools(w, pools, table, lens, P, L_cap // P)
    g = got.cpu().numpy()
    live = lens > 0
    assert np.all(g[~live] == 0.0)
    err = oracle.relative_error(g[live].reshape(-1, d_h), ref[live].reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,H,d_h,r", [("bf16", 8, 64, 16), ("f32", 4, 16, 4)])
def test_paged_append_across_page_boundaries(dtype, H, d_h, r):
    """Sequences 1 below, at and 1 below the next page boundary, and one full: three appends each, checked row
    for row in the pools against the reference's append, then a decode against the reference."""
    P, maxp = 32, 4
    L_cap = P * maxp
    w = _workload(dtype, 4, H, d_h, r, L_cap)
    lens = np.array([P - 1, P, 2 * P - 1, L_cap], dtype=np.int32)
    say(f"[case] paged append {dtype} H={H} d_h={d_h} r={r} lens={lens.tolist()}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    pc, pools, table, seq_lens, n_pages = _to_pages(w, dev, P, spare=2, seed=77)
    host_pools = {k: (_host(v) if v is not None else None) for k, v in pools.items()}
    np_dt = host_pools["k_pages"].dtype
    if not r:
        host_pools["zk_pages"] = host_pools["zv_pages"] = np.zeros((n_pages, P, H, 0), np_dt)
    host_lens = lens.copy()
    dims = dims_of(w)
    for step in range(3):
        rows = {k: synth.normal(9300 + 10 * step + i, 1.0, w.batch * n, dtype).reshape(w.batch, -1)
                for i, (k, n) in enumerate((("k_new", d_h), ("v_new", d_h), ("zk_new", H * r), ("zv_new", H * r)))}
        nd = {k: sdev.to_device(v) for k, v in rows.items()}
        lk.lrkv_paged_append(dims, pc, nd["k_new"], nd["v_new"], nd["zk_new"] if r else None,
                             nd["zv_new"] if r else None)
        opaged.append(host_pools["k_pages"], host_pools["v_pages"], host_pools["zk_pages"], host_pools["zv_pages"],
                      table.cpu().numpy(), host_lens, P, maxp, rows["k_new"], rows["v_new"],
                      rows["zk_new"].reshape(w.batch, H, r), rows["zv_new"].reshape(w.batch, H, r))
    torch.cuda.synchronize()
    assert seq_lens.cpu().numpy().tolist() == host_lens.tolist() == [P + 2, P + 3, 2 * P + 2, L_cap]
    for name in ("k_pages", "v_pages") + (("zk_pages", "zv_pages") if r else ()):
        a, b = _host(pools[name]), host_pools[name]
        same = (a == b) | (np.isnan(a.astype(np.float32)) & np.isnan(b.astype(np.float32))) if np_dt == np.float32 \
            else (a == b)
        assert np.all(same), f"{name}: pool contents differ from the reference append"
    dev["seq_lens"] = seq_lens
    got = _paged_decode(w, dev, pc, L_cap).cpu().numpy()
    ref = _reference_from_pools(w, pools, table, host_lens, P, maxp)
    err = oracle.relative_error(got.reshape(-1, d_h), ref.reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


@pytest.mark.timeout(600)
def test_paged_long_context_full_size_bitwise():
    """The long-context workload in the benchmark's launch configuration, paged in 256-row pages of a shuffled
    pool: bit for bit the contiguous decode."""
    w0 = synth.WORKLOADS["long_context"]
    L_cap, max_len = bench.launch_config(w0, 50)
    w = w0.with_(L_cap=L_cap)
    lens = synth.seq_lengths(w)
    say(f"[case] paged long context, L_cap={L_cap} max_len={max_len}, 256-row pages")
    dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
    pc, pools, table, _, _ = _to_pages(w, dev, 256, spare=5, seed=5)
    got = _paged_decode(w, dev, pc, max_len)
    want = gpu_decode(w, dev, max_len, L_cap=L_cap)
    assert torch.equal(got, want)
    assert bool(torch.isfinite(got).all())
