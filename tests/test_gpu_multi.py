"""GPU parity of multi-token decode (Q query tokens per sequence, causal inside the chunk) against the fp64
reference, through the C ABI.  Metric and tolerances as in test_gpu_decode.py.  On the bf16 matrix-core shapes
every case also runs with each number of query tokens per workgroup (LRKV_MULTI_QW = 1, 2, 4) besides the
default choice."""
import os

import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _multi_gpu(w, dev, Q, qh, max_len):
    dims = dims_of(w)
    B = w.batch
    q = sdev.to_device(qh)  # [B][Q][H][d_h]
    p = torch.empty((B, Q, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    if w.r:
        dq = lk.make_dims(B * Q, w.H, w.d_h, w.r, w.cap, dims.dtype)
        lk.lrkv_absorb_query(dq, q, dev["B_k"], p)
    out = torch.full((B, Q, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_multi_workspace_bytes(dims, Q, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_decode_multi(dims, Q, cache_of(dev, w.r), max_len, q, p if w.r else None, dev["B_v"] if w.r else None,
                         out, ws, nbytes)
    torch.cuda.synchronize()
    return out


def _host(w, lens):
    cap = w.cap
    npdt = np.float32 if w.dtype == "f32" else np.uint16
    c = {"k": np.zeros((w.batch, cap, w.d_h), npdt), "v": np.zeros((w.batch, cap, w.d_h), npdt),
         "zk": np.zeros((w.batch, w.H, cap, w.r), npdt), "zv": np.zeros((w.batch, w.H, cap, w.r), npdt)}
    for b in range(w.batch):
        n = int(lens[b])
        if n:
            s = synth.gen_sequence(w, 0, b, n)
            c["k"][b, :n], c["v"][b, :n] = s["k_shared"], s["v_shared"]
            if w.r:
                c["zk"][b, :, :n], c["zv"][b, :, :n] = s["z_k"], s["z_v"]
    return c


CASES = [  # (dtype, batch, Q, H, d_h, r, lengths)
    ("bf16", 3, 2, 8, 64, 16, [300, 33, 1]),
    ("f32", 2, 4, 4, 16, 4, [64, 3]),
    ("bf16", 2, 3, 32, 128, 64, [700, 2]),
    ("f32", 2, 2, 32, 128, 0, [129, 31]),
    ("bf16", 4, 8, 8, 64, 8, [40, 8, 7, 100]),
    ("bf16", 2, 16, 32, 128, 64, [1000, 5]),   # a sequence shorter than Q: its first queries see nothing
    ("bf16", 4, 8, 32, 128, 64, [2100, 1500, 17, 8]),
    ("bf16", 2, 64, 8, 64, 16, [200, 64]),
    ("bf16", 3, 4, 16, 128, 0, [333, 40, 4]),
    ("bf16", 2, 5, 16, 128, 32, [96, 40]),     # Q = 5: the last set of four holds one token
    ("bf16", 2, 4, 32, 128, 64, [33, 65]),     # last block: one row, seen by the last token only
    ("bf16", 3, 3, 8, 64, 48, [97, 129, 2]),   # four row lanes; last block of one row
]


@pytest.fixture(params=[None, "1", "2", "4"], ids=["qw_auto", "qw1", "qw2", "qw4"])
def query_width(request, monkeypatch):
    """LRKV_MULTI_QW for the call (None: the library's choice)."""
    if request.param is None:
        monkeypatch.delenv("LRKV_MULTI_QW", raising=False)
    else:
        monkeypatch.setenv("LRKV_MULTI_QW", request.param)
    return request.param


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_Q{c[2]}_H{c[3]}_d{c[4]}_r{c[5]}")
def test_multi_query_matches_reference(case, query_width):
    dtype, B, Q, H, d_h, r, lens = case
    if query_width is not None and dtype != "bf16":
        pytest.skip("the query-set width applies to the bf16 matrix-core kernel only")
    L = max(lens)
    w = synth.WORKLOADS["small_bf16"].with_(name="multi", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=(L + 31) // 32 * 32 + 32, ragged_lo=None)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] multi-query {case} LRKV_MULTI_QW={os.environ.get('LRKV_MULTI_QW')}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    qh = synth.normal(9100 + B, 1.0, B * Q * H * d_h, dtype).reshape(B, Q, H, d_h)
    got = _multi_gpu(w, dev, Q, qh, L).cpu().numpy()
    c = _host(w, lens)
    npdt = c["k"].dtype
    Bk = synth.gen_small(w, 0, "B_k") if r else np.zeros((H, d_h, 0), npdt)
    Bv = synth.gen_small(w, 0, "B_v") if r else np.zeros((H, d_h, 0), npdt)
    ref = oracle.lrkv_decode_multi(dtype, qh, c["k"], c["v"], c["zk"], c["zv"], Bk, Bv, lens)
    seen = (lens[:, None] - Q + np.arange(Q)[None, :] + 1) > 0  # [B][Q]
    assert np.all(got[~seen] == 0.0), "a query that sees no row must give 0"
    err = oracle.relative_error(got[seen].reshape(-1, d_h), ref[seen].reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e}) over {int(seen.sum()) * H} (b, query, h) rows")
    assert err <= TOL[dtype]


def test_single_query_through_multi_equals_decode():
    """Q = 1 runs the single-query kernels: bit for bit the same as lrkv_decode."""
    w = synth.WORKLOADS["small_bf16"].with_(batch=3, L=500, L_cap=512)
    lens = np.array([500, 77, 1], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    qh = sdev.to_device(synth.gen_small(w, 0, "q"))
    got = _multi_gpu(w, dev, 1, synth.gen_small(w, 0, "q").reshape(3, 1, w.H, w.d_h), 500)[:, 0]
    dims = dims_of(w)
    p = torch.empty((3, w.H, w.r), dtype=torch.float32, device="cuda")
    lk.lrkv_absorb_query(dims, qh, dev["B_k"], p)
    out = torch.empty((3, w.H, w.d_h), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, 500)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_decode(dims, cache_of(dev, w.r), 500, qh, p, dev["B_v"], out, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(got, out)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("workload", ["long_context", "ragged"])
def test_multi_query_full_size(workload):
    """The long-context workload (batch 4, H 32, d_h 128, r 64: two query tokens per workgroup) and the
    64-sequence ragged batch (r 32: four per workgroup), bf16, with Q = 4 query tokens per sequence in the
    benchmark's launch configuration; the first and last sequence are checked in full against the
    reference."""
    import bench
    Q = 4
    w0 = synth.WORKLOADS[workload]
    L_cap, max_len = bench.launch_config(w0, 50 * Q)
    w = w0.with_(L_cap=L_cap)
    lens = synth.seq_lengths(w)
    say(f"[case] multi-query {workload} Q={Q} L_cap={L_cap}")
    dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
    qh = synth.normal(9200, 1.0, w.batch * Q * w.H * w.d_h, "bf16").reshape(w.batch, Q, w.H, w.d_h)
    got = _multi_gpu(w, dev, Q, qh, max_len).cpu().numpy()
    Bk, Bv = synth.gen_small(w, 0, "B_k"), synth.gen_small(w, 0, "B_v")
    for b in (0, w.batch - 1):
        n = int(lens[b])
        sq = synth.gen_sequence(w, 0, b, n)
        ref = oracle.lrkv_decode_multi("bf16", qh[b:b + 1], sq["k_shared"][None], sq["v_shared"][None],
                                       sq["z_k"][None], sq["z_v"][None], Bk, Bv, np.array([n], dtype=np.int32))
        err = oracle.relative_error(got[b].reshape(-1, w.d_h), ref[0].reshape(-1, w.d_h))
        say(f"  seq {b}: max rel err {err:.3e} over {Q * w.H} (query, head) rows (tol {TOL['bf16']:.0e})")
        assert err <= TOL["bf16"]
