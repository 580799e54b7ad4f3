"""GPU parity of the projections around the attention core (project + append, output projection) and of a
whole layer decode step, against the fp64 layer reference (oracle/layer.py), through the C ABI.

Tolerances, derived from the arithmetic:
  * stored projections (q and the new cache rows): the GPU sums in fp32 and rounds once to the storage
    type, so |g - y| <= half an ulp of the storage type (at most 2^-8 |y| for bf16, 2^-24 |y| for fp32)
    plus the fp32 accumulation error, bounded here by 1e-4 * sum_k |x_k w_k| (K <= 4096 terms, unit
    roundoff 2^-24);
  * output projection: o enters the matrix cores as bf16 high + low parts (about 2^-17 relative per
    term) and the sum is fp32: |g - y| <= 1e-4 * sum_k |o_k w_k|;
  * the whole step: the metric of the decode tests, max over rows of ||g - o||_inf / ||o||_inf, within
    2e-3 (bf16) or 1e-5 (fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from oracle import layer as olayer
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _weights(w, d_model, seed):
    n_in = w.H * w.d_h + 2 * w.d_h + 2 * w.H * w.r
    W_in = synth.normal(seed, 1.0 / math.sqrt(d_model), n_in * d_model, w.dtype).reshape(n_in, d_model)
    W_o = synth.normal(seed + 1, 1.0 / math.sqrt(w.H * w.d_h), d_model * w.H * w.d_h, w.dtype).reshape(
        d_model, w.H * w.d_h)
    x = synth.normal(seed + 2, 1.0, w.batch * d_model, w.dtype).reshape(w.batch, d_model)
    return W_in, W_o, x


def _host_cache(w, lens):
    """Host copies of the device cache in the reference's per-head layout."""
    cap = w.cap
    npdt = np.float32 if w.dtype == "f32" else np.uint16
    c = {"k_shared": np.zeros((w.batch, cap, w.d_h), npdt), "v_shared": np.zeros((w.batch, cap, w.d_h), npdt),
         "z_k": np.zeros((w.batch, w.H, cap, w.r), npdt), "z_v": np.zeros((w.batch, w.H, cap, w.r), npdt)}
    for b in range(w.batch):
        n = int(lens[b])
        if n == 0:
            continue
        s = synth.gen_sequence(w, 0, b, n)
        c["k_shared"][b, :n], c["v_shared"][b, :n] = s["k_shared"], s["v_shared"]
        if w.r:
            c["z_k"][b, :, :n], c["z_v"][b, :, :n] = s["z_k"], s["z_v"]
    return c


def _dev_array(t: torch.Tensor, dtype: str) -> np.ndarray:
    """A device tensor back on the host in storage form (float32, or bf16 bit patterns as uint16)."""
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy()


def _bound(x_dtype, x, w_dtype, W):
    return 1e-4 * (np.abs(olayer.widen(x_dtype, x)) @ np.abs(olayer.widen(w_dtype, W)).T)


def _check_stored(dtype, got, ref64, bound, label):
    # half an ulp relative to the value: 8 significant bits (bf16) give at most 2^-8, 24 (fp32) 2^-24
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    g = olayer.widen(dtype, got)
    err = np.abs(g - ref64) - (half_ulp * np.abs(ref64) + bound)
    say(f"  {label}: worst margin {err.max():.3e} (must be <= 0) over {g.size} values")
    assert np.all(err <= 0), f"{label}: {int((err > 0).sum())} values outside the bound"


CASES = [  # (dtype, batch, H, d_h, r, d_model, L, full sequence index or -1)
    ("bf16", 5, 8, 64, 8, 1024, 300, 2),      # one 16-row tile
    ("bf16", 24, 8, 64, 16, 2048, 200, -1),   # two tiles
    ("bf16", 70, 8, 64, 8, 1024, 100, 69),    # four tiles, two row blocks
    ("f32", 3, 4, 16, 4, 48, 64, 1),          # plain fp32 kernel
    ("bf16", 3, 4, 16, 4, 96, 64, -1),        # bf16 with d_model off the matrix-core grid: plain kernel
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}_dm{c[5]}")
def test_project_append(case):
    dtype, B, H, d_h, r, dm, L, full = case
    w = synth.WORKLOADS["small_bf16"].with_(name="proj", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=L + 32, ragged_lo=None)
    lens = np.array([(L - 7 * b) % L + 1 for b in range(B)], dtype=np.int32)
    if full >= 0:
        lens[full] = w.cap
    say(f"[case] project+append {case}")
    W_in, W_o, x = _weights(w, dm, 7100 + B)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    before = {k: dev[k].clone() for k in ("k_shared", "v_shared", "z_k", "z_v")}
    q_out = torch.empty((B, H, d_h), dtype=sdev.torch_dtype(w), device="cuda")
    lk.lrkv_project_append(dims_of(w), dm, cache_of(dev, w.r), sdev.to_device(x), sdev.to_device(W_in), q_out)
    torch.cuda.synchronize()
    y64 = olayer.linear(dtype, x, dtype, W_in)
    bound = _bound(dtype, x, dtype, W_in)
    parts, bparts = olayer.split_projection(y64, H, d_h, r), olayer.split_projection(bound, H, d_h, r)
    _check_stored(dtype, _dev_array(q_out, dtype).reshape(B, H, d_h), parts["q"], bparts["q"], "q")
    new_lens = dev["seq_lens"].cpu().numpy()
    live = [b for b in range(B) if lens[b] < w.cap]
    assert new_lens.tolist() == [int(n) + 1 if b in live else int(n) for b, n in enumerate(lens)]
    for name, key, dv in (("k_new", "k_shared", None), ("v_new", "v_shared", None), ("zk_new", "z_k", 1),
                          ("zv_new", "z_v", 1)):
        if dv and r == 0:
            continue
        got = _dev_array(dev[key], dtype)
        rows = np.stack([got[b, lens[b]] for b in live])  # token-major: z rows are [H][r]
        _check_stored(dtype, rows.reshape(len(live), -1), parts[name][live].reshape(len(live), -1),
                      bparts[name][live].reshape(len(live), -1), name)
        # every other row is untouched
        mask = torch.ones(dev[key].shape[:2], dtype=torch.bool)
        for b in live:
            mask[b, int(lens[b])] = False
        assert torch.equal(dev[key][mask.cuda()], before[key][mask.cuda()]), key


@pytest.mark.parametrize("case", [("bf16", 5, 8, 64, 1024), ("bf16", 40, 16, 64, 2048), ("f32", 3, 4, 16, 48),
                                  ("bf16", 2, 4, 16, 64)], ids=str)
def test_output_project(case):
    dtype, B, H, d_h, dm = case
    say(f"[case] output projection {case}")
    o = synth.normal(7300 + B, 0.3, B * H * d_h, "f32").reshape(B, H * d_h)
    W_o = synth.normal(7301 + B, 1.0 / math.sqrt(H * d_h), dm * H * d_h, dtype).reshape(dm, H * d_h)
    y = torch.empty((B, dm), dtype=torch.float32, device="cuda")
    dims = lk.make_dims(B, H, d_h, 0, 64, lk.LRKV_F32 if dtype == "f32" else lk.LRKV_BF16)
    lk.lrkv_output_project(dims, dm, sdev.to_device(o), sdev.to_device(W_o), y)
    torch.cuda.synchronize()
    ref = olayer.linear("f32", o, dtype, W_o)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref) - _bound("f32", o, dtype, W_o)
    say(f"  worst margin {err.max():.3e} (must be <= 0)")
    assert np.all(err <= 0)


def _layer_step_gpu(w, dm, dev, x, W_in, W_o, max_len):
    dims = dims_of(w)
    cache = cache_of(dev, w.r)
    B = w.batch
    q = torch.empty((B, w.H, w.d_h), dtype=sdev.torch_dtype(w), device="cuda")
    p = torch.empty((B, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    o = torch.empty((B, w.H, w.d_h), dtype=torch.float32, device="cuda")
    y = torch.empty((B, dm), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_project_append(dims, dm, cache, sdev.to_device(x), sdev.to_device(W_in), q)
    if w.r:
        lk.lrkv_absorb_query(dims, q, dev["B_k"], p)
    lk.lrkv_decode(dims, cache, max_len, q, p if w.r else None, dev["B_v"] if w.r else None, o, ws, nbytes)
    lk.lrkv_output_project(dims, dm, o, sdev.to_device(W_o), y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("case", [("bf16", 4, 8, 64, 8, 1024, 700), ("bf16", 3, 16, 64, 32, 1024, 333),
                                  ("f32", 2, 4, 16, 4, 48, 64), ("f32", 3, 8, 64, 0, 512, 200)], ids=str)
def test_layer_step(case):
    dtype, B, H, d_h, r, dm, L = case
    w = synth.WORKLOADS["small_bf16"].with_(name="layer", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=L + 32, ragged_lo=None)
    lens = np.array([L - 5 * b for b in range(B)], dtype=np.int32)
    say(f"[case] layer step {case}")
    W_in, W_o, x = _weights(w, dm, 7500 + B)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    got = _layer_step_gpu(w, dm, dev, x, W_in, W_o, L + 1).cpu().numpy()
    host = _host_cache(w, lens)
    Bk = synth.gen_small(w, 0, "B_k") if r else np.zeros((H, d_h, 0), host["k_shared"].dtype)
    Bv = synth.gen_small(w, 0, "B_v") if r else np.zeros((H, d_h, 0), host["k_shared"].dtype)
    ref = olayer.layer_step(dtype, x, W_in, W_o, Bk, Bv, host, lens, H, d_h, r)
    err = oracle.relative_error(got, ref["y"])
    say(f"  layer step max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


def test_project_append_long_context_full_size():
    """The long-context shape with d_model = H*d_h = 4096 (the matrix-core path), full-size weights."""
    w = synth.WORKLOADS["long_context"].with_(L=2048, L_cap=2048 + 64)
    dm, B, H, d_h, r = 4096, w.batch, w.H, w.d_h, w.r
    lens = np.array([2048 - 3 * b for b in range(B)], dtype=np.int32)
    say(f"[case] project+append long-context shape d_model={dm}")
    W_in, W_o, x = _weights(w, dm, 7700)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    q_out = torch.empty((B, H, d_h), dtype=torch.bfloat16, device="cuda")
    lk.lrkv_project_append(dims_of(w), dm, cache_of(dev, r), sdev.to_device(x), sdev.to_device(W_in), q_out)
    y_o = torch.empty((B, dm), dtype=torch.float32, device="cuda")
    o = synth.normal(7710, 0.3, B * H * d_h, "f32").reshape(B, H * d_h)
    lk.lrkv_output_project(dims_of(w), dm, sdev.to_device(o), sdev.to_device(W_o), y_o)
    torch.cuda.synchronize()
    y64 = olayer.linear("bf16", x, "bf16", W_in)
    bound = _bound("bf16", x, "bf16", W_in)
    parts, bparts = olayer.split_projection(y64, H, d_h, r), olayer.split_projection(bound, H, d_h, r)
    _check_stored("bf16", _dev_array(q_out, "bf16"), parts["q"], bparts["q"], "q")
    zk = _dev_array(dev["z_k"], "bf16")
    _check_stored("bf16", np.stack([zk[b, lens[b]] for b in range(B)]), parts["zk_new"], bparts["zk_new"], "z_k")
    ref = olayer.linear("f32", o, "bf16", W_o)
    err = np.abs(y_o.cpu().numpy().astype(np.float64) - ref) - _bound("f32", o, "bf16", W_o)
    assert np.all(err <= 0)


MAT_CASES = [  # (dtype, batch, H, d_h, r, lengths)
    ("bf16", 3, 8, 64, 8, [100, 17, 0]),
    ("bf16", 2, 32, 128, 64, [300, 65]),
    ("bf16", 2, 16, 128, 48, [129, 1]),
    ("f32", 2, 4, 16, 4, [40, 9]),
    ("bf16", 2, 8, 64, 0, [50, 3]),
    ("bf16", 2, 8, 128, 32, [700, 257]),  # several 256-row workgroups, one row past a 64-row wave
    ("bf16", 2, 8, 96, 16, [70, 33]),     # d_h off the 64 / 128 kernels: a wave per 16 rows
    ("bf16", 2, 6, 64, 16, [100, 70]),    # heads not a multiple of a workgroup's four
]


@pytest.mark.parametrize("case", MAT_CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
def test_materialize(case):
    """Rebuilt per-head keys and values against the reference (oracle.layer.materialize): within half an ulp
    of the storage type plus 1e-5 * (|k_s| + sum_i |z_i b_i|) of its exact value, equal to its stored
    (rounded) value wherever that bound cannot reach a rounding midpoint; rows past each length untouched."""
    dtype, B, H, d_h, r, lens = case
    L = max(lens)
    w = synth.WORKLOADS["small_bf16"].with_(name="mat", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=L + 16, ragged_lo=None)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] materialize {case}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    # sentinels exactly representable in bf16 and fp32
    K = torch.full((B, H, w.cap, d_h), 1024.0, dtype=sdev.torch_dtype(w), device="cuda")
    V = torch.full_like(K, -512.0)
    lk.lrkv_materialize(dims_of(w), cache_of(dev, r), L, dev["B_k"] if r else None, dev["B_v"] if r else None, K, V)
    torch.cuda.synchronize()
    host = _host_cache(w, lens)
    npdt = host["k_shared"].dtype
    Bk = synth.gen_small(w, 0, "B_k") if r else np.zeros((H, d_h, 0), npdt)
    Bv = synth.gen_small(w, 0, "B_v") if r else np.zeros((H, d_h, 0), npdt)
    args = (dtype, host["k_shared"], host["v_shared"], host["z_k"], host["z_v"], Bk, Bv, lens)
    exact = olayer.materialize(*args, rounded=False)   # fp64 before the one rounding
    stored = olayer.materialize(*args)                 # the reference's stored values
    half_ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    for i, (out, shared, z, basis, fill, name) in enumerate(((K, "k_shared", "z_k", Bk, 1024.0, "K"),
                                                             (V, "v_shared", "z_v", Bv, -512.0, "V"))):
        ks = olayer.widen(dtype, host[shared])
        zz = olayer.widen(dtype, host[z])
        bb = olayer.widen(dtype, basis)
        got = _dev_array(out, dtype)
        for b in range(B):
            n = int(lens[b])
            for h in range(H):
                ref = exact[i][b, h, :n]
                bound = 1e-5 * (np.abs(ks[b, :n]) + np.abs(zz[b, h, :n]) @ np.abs(bb[h]).T)
                if (b, h) == (0, 0):
                    _check_stored(dtype, got[b, h, :n], ref, bound, f"{name}[{b},{h}]")
                g = olayer.widen(dtype, got[b, h, :n])
                assert np.all(np.abs(g - ref) <= half_ulp * np.abs(ref) + bound)
                # the one rounding: the GPU rounds a value within `bound` of the exact one, so where its stored
                # value differs from the reference's it can be no farther from the exact value than the
                # reference's plus twice the bound (a tie broken the other way), never a worse rounding
                st = olayer.widen(dtype, stored[i][b, h, :n])
                differ = g != st
                worse = np.abs(g - ref) > np.abs(st - ref) + 2.0 * bound
                assert not np.any(differ & worse), f"{name}[{b},{h}]: stored value differs from the reference's"
            assert np.all(olayer.widen(dtype, got[b, :, n:]) == fill), f"{name}: rows past the length written"
