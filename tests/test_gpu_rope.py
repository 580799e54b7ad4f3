"""GPU parity of the rotary variant (every head's whole key turned at its position, the exact position-wise
contraction) against the fp64 reference oracle.rope, through the C ABI.  Metric and tolerances as in
test_gpu_decode.py; the rotation table is checked against fp64 cos/sin rounded to fp32."""
import numpy as np
import pytest
import torch

import bench
import oracle
import rank_shared_kv_amd as lk
import synth
from oracle import rope
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, say  # noqa: E402

BASE = 10000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _table(d_h, n_pos, base=BASE):
    t = torch.full((max(n_pos, 1), d_h // 2, 2), float("nan"), dtype=torch.float32, device="cuda")
    lk.lrkv_rope_table(d_h, n_pos, base, t)
    return t


@pytest.mark.parametrize("d_h,n_pos,base", [(128, 33000, 10000.0), (16, 300, 10000.0), (64, 5000, 500.0)])
def test_rope_table(d_h, n_pos, base):
    got = _table(d_h, n_pos, base).cpu().numpy().astype(np.float64)
    phi = rope.angles(d_h, np.arange(n_pos), base)
    for j, ref in enumerate((np.cos(phi), np.sin(phi))):
        half_ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) / 2
        err = np.abs(got[:, :, j] - ref)
        # fp32 rounding of the fp64 value, plus fp64 differences in the angle (tens of thousands of radians)
        assert np.all(err <= half_ulp * (1 + 1e-6) + 1e-11), f"max err {err.max():.3e}"


def _run(w, dev, max_len, table):
    dims = dims_of(w)
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_rope_workspace_bytes(dims, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_decode_rope(dims, cache_of(dev, w.r), max_len, dev["q"], dev["B_k"] if w.r else None, table,
                        dev["B_v"] if w.r else None, out, ws, nbytes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [  # (dtype, batch, H, d_h, r, lengths)
    ("bf16", 3, 8, 64, 16, [300, 33, 1]),
    ("bf16", 2, 32, 128, 64, [700, 2]),
    ("bf16", 3, 16, 128, 32, [2500, 0, 64]),
    ("bf16", 2, 8, 64, 0, [100, 31]),
    ("bf16", 2, 20, 128, 48, [300, 65]),    # a partial second head group; six latent chunks per head
    ("bf16", 3, 12, 64, 8, [130, 64, 1]),   # a partial head group; one latent chunk per head
    ("bf16", 3, 32, 128, 64, [128, 129, 192]),  # a whole 128-row tile; one row past it; one and a half tiles
    ("bf16", 2, 4, 64, 16, [200, 129]),       # fewer heads than waves: four waves without a head
    ("bf16", 2, 4, 48, 12, [90, 7]),
    ("f32", 2, 4, 16, 4, [64, 3]),
    ("f32", 2, 8, 128, 0, [129, 31]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
def test_decode_rope_matches_reference(case):
    dtype, B, H, d_h, r, lens = case
    L = max(max(lens), 1)
    w = synth.WORKLOADS["small_bf16"].with_(name="rope", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=(L + 31) // 32 * 32 + 32, ragged_lo=None)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] rotary decode {case}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    host = synth.gen_host(w, 0, lengths=lens)
    got = _run(w, dev, int(lens.max()), _table(d_h, w.cap))
    ref = rope.decode_rope(dtype, host["q"], host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                           host["B_k"], host["B_v"], lens, base=BASE)
    live = lens > 0
    assert np.all(got[~live] == 0.0)
    err = oracle.relative_error(got[live].reshape(-1, d_h), ref[live].reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


@pytest.mark.timeout(900)
def test_rope_long_context_full_size():
    """The long-context workload in the benchmark's launch configuration; the first and last sequence are
    checked against the reference in full (all heads, all 32768 positions)."""
    w0 = synth.WORKLOADS["long_context"]
    L_cap, max_len = bench.launch_config(w0, 50)
    w = w0.with_(L_cap=L_cap)
    lens = synth.seq_lengths(w)
    say(f"[case] rotary long context, L_cap={L_cap}")
    dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
    got = _run(w, dev, max_len, _table(w.d_h, L_cap))
    q, Bk, Bv = synth.gen_small(w, 0, "q"), synth.gen_small(w, 0, "B_k"), synth.gen_small(w, 0, "B_v")
    for b in (0, w.batch - 1):
        n = int(lens[b])
        s = synth.gen_sequence(w, 0, b, n)
        ref = rope.decode_rope("bf16", q[b:b + 1], s["k_shared"][None], s["v_shared"][None], s["z_k"][None],
                               s["z_v"][None], Bk, Bv, [n], base=BASE)[0]
        err = oracle.relative_error(got[b], ref)
        say(f"  seq {b}: max rel err {err:.3e} over {w.H} heads (tol {TOL['bf16']:.0e})")
        assert err <= TOL["bf16"]
