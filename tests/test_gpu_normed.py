"""GPU parity of the normalised variant (cached per-(token, head) key scales, the key gain folded into the query)
against the fp64 reference oracle.normed, through the C ABI.

Stored values (the scales rho and the normalised query q_eff, kept in the cache dtype) are compared with the
exact fp64 value rounded to that dtype: they must be that rounding, except where the exact value lies within
the fp32 arithmetic's error of a rounding midpoint, where the neighbour is accepted.  The decode is compared on
the reference's own stored rho and q_eff (fed to both sides), with the metric and tolerances of
test_gpu_decode.py; the chained tests run every step on each side from the same raw inputs.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import rank_shared_kv_amd as lk
import synth
from oracle import normed
from oracle.layer import widen
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, say  # noqa: E402

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _workload(dtype, B, H, d_h, r, lens, L_cap=None):
    L = max(max(lens), 1)
    cap = L_cap or ((L + 31) // 32 * 32 + 32)
    return synth.WORKLOADS["small_bf16"].with_(name="normed", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                               L_cap=cap, ragged_lo=None)


def _host_cache(w, lens):
    c = synth.gen_host(w, 0, lengths=np.asarray(lens, dtype=np.int32))
    return c


def _nan_bits(dtype):
    return 0x7FC0 if dtype == "bf16" else np.float32("nan")


def _check_stored(got, exact64, dtype, what):
    """got (stored dtype) is exact64 rounded to nearest even, or its neighbour where exact64 sits at a midpoint
    to within the fp32 arithmetic's error."""
    if dtype == "f32":
        rel = np.abs(got.astype(np.float64) - exact64) / np.maximum(np.abs(exact64), 1e-300)
        say(f"  {what}: max rel err {rel.max():.2e} over {got.size} values")
        assert rel.max() <= 4e-6, f"{what}: fp32 error {rel.max():.3e}"
        return
    want = normed.stored("bf16", exact64)
    mism = got != want
    n = int(mism.sum())
    say(f"  {what}: {n} of {got.size} stored values differ from the exact value rounded (midpoint ties allowed)")
    if n:
        g, w_, e = widen("bf16", got[mism]), widen("bf16", want[mism]), exact64[mism]
        assert np.all(np.abs(got[mism].astype(np.int64) - want[mism].astype(np.int64)) == 1), f"{what}: off by > 1 ulp"
        mid = (g + w_) / 2
        assert np.all(np.abs(e - mid) <= 2.0 ** -18 * np.abs(e)), f"{what}: a value off its rounding, not at a tie"
        assert n <= max(2, got.size // 1000), f"{what}: {n} ties is too many"


def _host_array(t, dtype):
    """A device tensor in the stored dtype as a host array (bf16 as uint16 bit patterns)."""
    t = t.cpu()
    return t.numpy() if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def _rho_device(rho_st, dtype, lens, L_cap):
    """[B][H][L_cap] (reference layout) -> device [B][L_cap][H]; rows at or past L_b hold NaN (never read)."""
    arr = np.array(rho_st, copy=True)
    for b, n in enumerate(lens):
        arr[b, :, int(n):] = _nan_bits(dtype)
    return sdev.to_device(np.ascontiguousarray(arr.transpose(0, 2, 1)))


def _run_normed_decode(w, dev, rho_dev, q_eff_dev, max_len, L_cap=None):
    dims = dims_of(w, L_cap)
    p = torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    if w.r:
        lk.lrkv_absorb_query(dims, q_eff_dev, dev["B_k"], p)
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, max_len)
    ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
    lk.lrkv_decode_normed(dims, cache_of(dev, w.r), rho_dev, max_len, q_eff_dev, p if w.r else None,
                          dev["B_v"] if w.r else None, out, ws, nbytes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SCALE_CASES = [  # (dtype, batch, H, d_h, r, lengths): matrix-core path (bf16, d_h % 16, r % 8, r <= 64) and plain
    ("bf16", 3, 8, 64, 16, [300, 33, 1]),
    ("bf16", 2, 32, 128, 64, [200, 77]),
    ("bf16", 2, 16, 128, 48, [65, 130]),
    ("bf16", 2, 8, 64, 0, [50, 9]),
    ("bf16", 2, 4, 48, 12, [40, 3]),
    ("bf16", 2, 6, 64, 8, [100, 70]),     # heads not a multiple of a workgroup's four
    ("bf16", 2, 8, 96, 16, [70, 33]),     # d_h off the 64 / 128 kernel: a wave per 16 rows
    ("bf16", 2, 16, 128, 64, [2500, 1100]),  # whole history of 1024..4095 rows: four chunks per workgroup
    ("bf16", 1, 8, 128, 32, [5000]),         # 4096 rows and more: sixteen chunks, the last workgroup partial
    ("f32", 2, 4, 16, 4, [64, 3]),
    ("f32", 2, 32, 128, 0, [70, 1]),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
@pytest.mark.parametrize("n_last", [None, 1, 5])
def test_key_scales_match_reference(case, n_last):
    dtype, B, H, d_h, r, lens = case
    w = _workload(dtype, B, H, d_h, r, lens)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] key scales {case} n_last={n_last}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    host = _host_cache(w, lens)
    max_len = int(lens.max())
    nl = max_len if n_last is None else n_last
    rho = torch.full((B, w.cap, H), float("nan"), dtype=sdev.torch_dtype(w), device="cuda")
    lk.lrkv_key_scales(dims_of(w), cache_of(dev, r), max_len, nl, dev["B_k"] if r else None, EPS, rho)
    torch.cuda.synchronize()
    got = _host_array(rho, dtype)
    exact = normed.key_scales(dtype, host["k_shared"], host["z_k"], host["B_k"], lens, EPS)  # [B][H][L_cap]
    for b in range(B):
        n = int(lens[b])
        lo = max(0, n - nl)
        g = got[b].T  # [H][L_cap]
        _check_stored(g[:, lo:n], exact[b, :, lo:n], dtype, f"rho seq {b} rows {lo}..{n - 1}")
        untouched = np.concatenate([g[:, :lo], g[:, n:]], axis=1)
        assert np.all(np.isnan(widen(dtype, untouched))), f"seq {b}: a row outside the range was written"


@pytest.mark.parametrize("dtype,H,d_h", [("bf16", 8, 64), ("bf16", 32, 128), ("f32", 4, 16), ("bf16", 3, 200)])
def test_norm_query_matches_reference(dtype, H, d_h):
    B = 5
    q = synth.normal(7300 + H, 1.5, B * H * d_h, dtype).reshape(B, H, d_h)
    gq, gk = synth.gain(7310 + H, (H, d_h), dtype), synth.gain(7320 + H, (H, d_h), dtype)
    dims = lk.make_dims(B, H, d_h, 0, 32, lk.LRKV_F32 if dtype == "f32" else lk.LRKV_BF16)
    out = torch.full((B, H, d_h), float("nan"), dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                     device="cuda")
    lk.lrkv_norm_query(dims, sdev.to_device(q), sdev.to_device(gq), sdev.to_device(gk), EPS, out)
    torch.cuda.synchronize()
    got = _host_array(out, dtype)
    _check_stored(got, normed.norm_query(dtype, q, gq, gk, EPS), dtype, "q_eff")


DECODE_CASES = [  # (dtype, batch, H, d_h, r, lengths)
    ("bf16", 3, 8, 64, 16, [300, 33, 1]),
    ("bf16", 2, 32, 128, 64, [700, 2]),
    ("bf16", 3, 16, 128, 32, [129, 0, 64]),
    ("bf16", 2, 8, 64, 0, [100, 31]),
    ("bf16", 2, 4, 48, 12, [90, 7]),
    ("f32", 2, 4, 16, 4, [64, 3]),
    ("f32", 2, 32, 128, 0, [129, 31]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
def test_decode_normed_matches_reference(case):
    dtype, B, H, d_h, r, lens = case
    w = _workload(dtype, B, H, d_h, r, lens)
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] normalised decode {case}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    host = _host_cache(w, lens)
    gq, gk = synth.gain(7400, (H, d_h), dtype), synth.gain(7401, (H, d_h), dtype)
    rho_st = normed.stored(dtype, normed.key_scales(dtype, host["k_shared"], host["z_k"], host["B_k"], lens, EPS))
    q_st = normed.stored(dtype, normed.norm_query(dtype, host["q"], gq, gk, EPS))
    ref = normed.decode_normed(dtype, q_st, host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                               host["B_k"], host["B_v"], rho_st, lens)
    got = _run_normed_decode(w, dev, _rho_device(rho_st, dtype, lens, w.cap), sdev.to_device(q_st), int(lens.max()))
    live = lens > 0
    assert np.all(got[~live] == 0.0), "a sequence with no rows must give 0"
    err = oracle.relative_error(got[live].reshape(-1, d_h), ref[live].reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,H,d_h,r,lens", [("f32", 4, 64, 8, [200, 45]), ("bf16", 16, 128, 32, [1500, 900]),
                                                ("bf16", 8, 64, 0, [1200, 1])])
def test_normed_chain_matches_reference(dtype, H, d_h, r, lens):
    """Every step on each side from the same raw inputs: scales of the whole history, then one appended token
    (append + scale of the new row), query normalisation, absorption, decode."""
    B = len(lens)
    w = _workload(dtype, B, H, d_h, r, [n + 1 for n in lens])
    lens = np.array(lens, dtype=np.int32)
    say(f"[case] normalised chain {dtype} H={H} d_h={d_h} r={r} lens={lens.tolist()}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    host = _host_cache(w, lens)
    rows = synth.gen_new_rows(w, 0)
    gq, gk = synth.gain(7500, (H, d_h), dtype), synth.gain(7501, (H, d_h), dtype)
    dims, cache = dims_of(w), cache_of(dev, r)
    max_len = int(lens.max()) + 1
    rho = torch.zeros((B, w.cap, H), dtype=sdev.torch_dtype(w), device="cuda")
    lk.lrkv_key_scales(dims, cache, max_len, max_len, dev["B_k"] if r else None, EPS, rho)
    nd = {k: sdev.to_device(v) for k, v in rows.items()}
    lk.lrkv_cache_append(dims, cache, nd["k_new"], nd["v_new"], nd["zk_new"] if r else None,
                         nd["zv_new"] if r else None)
    lk.lrkv_key_scales(dims, cache, max_len, 1, dev["B_k"] if r else None, EPS, rho)
    q_eff = torch.empty_like(dev["q"])
    lk.lrkv_norm_query(dims, dev["q"], sdev.to_device(gq), sdev.to_device(gk), EPS, q_eff)
    got = _run_normed_decode(w, dev, rho, q_eff, max_len)

    # the reference from the same raw inputs
    for b in range(B):
        j = int(lens[b])
        host["k_shared"][b, j], host["v_shared"][b, j] = rows["k_new"][b], rows["v_new"][b]
        if r:
            host["z_k"][b, :, j], host["z_v"][b, :, j] = rows["zk_new"][b], rows["zv_new"][b]
    lens1 = lens + 1
    rho_st = normed.stored(dtype, normed.key_scales(dtype, host["k_shared"], host["z_k"], host["B_k"], lens1, EPS))
    q_st = normed.stored(dtype, normed.norm_query(dtype, host["q"], gq, gk, EPS))
    ref = normed.decode_normed(dtype, q_st, host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                               host["B_k"], host["B_v"], rho_st, lens1)
    err = oracle.relative_error(got.reshape(-1, d_h), ref.reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


@pytest.mark.timeout(900)
def test_normed_long_context_full_size():
    """The long-context workload (batch 4, H 32, d_h 128, r 64, L 32768, bf16) in the benchmark's launch
    configuration: the scales of every row on the matrix-core path checked on sampled sequences, and the
    normalised decode against the reference on two whole sequences (all heads)."""
    w0 = synth.WORKLOADS["long_context"]
    L_cap, max_len = bench.launch_config(w0, 50)
    w = w0.with_(L_cap=L_cap)
    lens = synth.seq_lengths(w)
    say(f"[case] normalised long context, L_cap={L_cap} max_len={max_len}")
    dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
    dims, cache = dims_of(w, L_cap), cache_of(dev, w.r)
    rho = torch.full((w.batch, L_cap, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    lk.lrkv_key_scales(dims, cache, max_len, max_len, dev["B_k"], EPS, rho)
    torch.cuda.synchronize()
    got_rho = _host_array(rho, "bf16")
    gq, gk = synth.gain(7600, (w.H, w.d_h), "bf16"), synth.gain(7601, (w.H, w.d_h), "bf16")
    q_host = synth.gen_small(w, 0, "q")
    q_st = normed.stored("bf16", normed.norm_query("bf16", q_host, gq, gk, EPS))
    Bk, Bv = synth.gen_small(w, 0, "B_k"), synth.gen_small(w, 0, "B_v")
    rho_ref = np.zeros((w.batch, w.H, L_cap), dtype=np.uint16)
    refs = {}
    for b in range(w.batch):
        n = int(lens[b])
        s = synth.gen_sequence(w, 0, b, n)
        ex = normed.key_scales("bf16", s["k_shared"][None], s["z_k"][None], Bk, [n], EPS)[0]  # [H][n]
        _check_stored(got_rho[b, :n].T, ex, "bf16", f"rho seq {b}")
        rho_ref[b, :, :n] = normed.stored("bf16", ex)
        if b in (0, w.batch - 1):
            refs[b] = normed.decode_normed("bf16", q_st[b:b + 1], s["k_shared"][None], s["v_shared"][None],
                                           s["z_k"][None], s["z_v"][None], Bk, Bv, rho_ref[b:b + 1, :, :n], [n])[0]
    got = _run_normed_decode(w, dev, _rho_device(rho_ref, "bf16", lens, L_cap), sdev.to_device(q_st), max_len,
                             L_cap)
    for b, ref in refs.items():
        err = oracle.relative_error(got[b], ref)
        say(f"  seq {b}: max rel err {err:.3e} over {w.H} heads (tol {TOL['bf16']:.0e})")
        assert err <= TOL["bf16"]
