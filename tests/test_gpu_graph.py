"""A decode step captured as a HIP graph (torch.cuda.CUDAGraph around the C-ABI calls) replays to the same
results as the same step launched directly.  The step -- lrkv_append_absorb, lrkv_decode_partial,
lrkv_decode_merge -- allocates nothing, clears nothing with memset and does not synchronise, so it can be
captured; the kernels read the lengths on the device, so each replay decodes over one more row.  Two copies of
the same cache advance side by side, one by replays and one by direct launches, with eager work and
synchronisations between the replays; outputs, lengths and cache rows must agree bit for bit after every
step."""
import numpy as np
import pytest
import torch

import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import cache_of, dims_of, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


@pytest.mark.parametrize("shape", [("bf16", 3, 32, 128, 64), ("bf16", 2, 16, 128, 48), ("f32", 2, 8, 64, 0)],
                         ids=lambda s: f"{s[0]}_B{s[1]}_H{s[2]}_d{s[3]}_r{s[4]}")
def test_graph_replays_match_direct_launches(shape):
    dtype, B, H, d_h, r = shape
    steps = 4
    lens = np.array([300 + 97 * b for b in range(B)], dtype=np.int32)
    L_cap = int(lens.max()) + 32 + steps
    L_cap = (L_cap + 31) // 32 * 32
    max_len = int(lens.max()) + steps
    w = synth.WORKLOADS["small_bf16"].with_(name="graph", batch=B, H=H, d_h=d_h, r=r, dtype=dtype,
                                            L=int(lens.max()), L_cap=L_cap, ragged_lo=None)
    say(f"[case] graph replay {shape}")
    runs = []
    for _ in range(3):
        dev = sdev.fill_layer(w, 0, lengths=lens)
        rows = sdev.new_rows(w)
        dims = dims_of(w)
        nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
        runs.append(dict(dev=dev, rows=rows, dims=dims, cache=cache_of(dev, r),
                         ws=torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda"), nbytes=nbytes,
                         p=torch.zeros((B, H, max(r, 1)), dtype=torch.float32, device="cuda"),
                         out=torch.zeros((B, H, d_h), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()

    def step(x, stream):
        zk, zv = (x["rows"]["zk_new"], x["rows"]["zv_new"]) if r else (None, None)
        pp, bk, bv = (x["p"], x["dev"]["B_k"], x["dev"]["B_v"]) if r else (None, None, None)
        lk.lrkv_append_absorb(x["dims"], x["cache"], x["rows"]["k_new"], x["rows"]["v_new"], zk, zv,
                              x["dev"]["q"], bk, pp, stream)
        lk.lrkv_decode_partial(x["dims"], x["cache"], max_len, x["dev"]["q"], pp, x["ws"], x["nbytes"], stream)
        lk.lrkv_decode_merge(x["dims"], x["dev"]["seq_lens"], max_len, bv, x["out"], x["ws"], x["nbytes"], stream)

    warm, direct, graphed = runs
    # a warm-up step on a throwaway copy, on a side stream, loads every kernel before the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(warm, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    # the capture itself runs nothing, so the graphed copy's state is unchanged by it
    with torch.cuda.graph(g):
        step(graphed, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert graphed["dev"]["seq_lens"].cpu().numpy().tolist() == lens.tolist()
    for k in range(steps):
        step(direct, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between replays
        for name in ("seq_lens", "k_shared", "v_shared", "z_k", "z_v"):
            a, b = direct["dev"][name], graphed["dev"][name]
            if a.numel():
                va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
                vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
                assert torch.equal(va, vb), f"{name} differs after replay {k}"
        assert torch.equal(direct["out"].view(torch.int32), graphed["out"].view(torch.int32)), f"replay {k}"
        assert bool(torch.isfinite(graphed["out"]).all())
    assert graphed["dev"]["seq_lens"].cpu().numpy().tolist() == (lens + steps).tolist()
