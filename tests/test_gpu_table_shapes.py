"""GPU parity at the pages' own model shapes on the bf16 matrix-core kernel.

The reading notes' model table (sec. 2.5, the ranks of Table 7 recomputed with Eq. (9)) lists d_h = 128 with
(H, r) = (6, 46), (12, 51), (18, 55) and (32, 54).  Their head counts fill the kernel's 8-head octets only
partly, and their ranks leave a head's last latent lanes with fewer coordinates (odd ranks start most lanes on
an odd element).  Each shape is checked against the fp64 reference at tile-edge lengths, at a batch large
enough for two waves per SIMD, with NaN in every row past the lengths, paged, and with several query tokens.
Metric and tolerances as in test_gpu_decode.py.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, compare, dims_of, gpu_decode, oracle_pairs, say  # noqa: E402

SHAPES = [(6, 46), (12, 51), (18, 55), (32, 54)]  # (H, r) at d_h = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _w(H, r, batch, L, L_cap, name="table"):
    return synth.WORKLOADS["ragged"].with_(name=f"{name}_{H}_{r}", batch=batch, H=H, d_h=128, r=r, dtype="bf16",
                                           L=L, L_cap=L_cap, ragged_lo=None)


def _granule(w, L_cap, max_len):
    return lk.lrkv_decode_num_splits(dims_of(w, L_cap), max_len)[1]


@pytest.mark.parametrize("H,r", SHAPES, ids=[f"H{h}_r{r}" for h, r in SHAPES])
def test_table_shape_edges(H, r):
    """Lengths 0, 1, block edges and a few blocks; every head of every sequence against the reference."""
    lens = np.array([0, 1, 31, 32, 33, 127, 129, 700], dtype=np.int32)
    w = _w(H, r, 8, 700, 704)
    assert _granule(w, 704, 700) in (64, 128), "not on the matrix-core kernel"
    say(f"[case] table shape H={H} r={r} edges, granule {_granule(w, 704, 700)}")
    dev = sdev.fill_layer(w, 0, L_cap=704, lengths=lens)
    got = gpu_decode(w, dev, 700, L_cap=704)
    assert torch.equal(got[0], torch.zeros_like(got[0]))
    pairs = [(b, h) for b in range(1, 8) for h in range(H)]
    compare(w, got, oracle_pairs(w, 0, lens, pairs), pairs, f"table H={H} r={r}")


@pytest.mark.parametrize("H,r", SHAPES, ids=[f"H{h}_r{r}" for h, r in SHAPES])
def test_table_shape_two_waves_per_simd(H, r):
    """A batch of 40 ragged sequences (two waves per SIMD), sampled pairs including every head of two."""
    rng = np.random.default_rng(1000 + H)
    lens = rng.integers(1, 2500, size=40).astype(np.int32)
    w = _w(H, r, 40, int(lens.max()), 2528)
    say(f"[case] table shape H={H} r={r}, batch 40, lengths {lens.min()}..{lens.max()}")
    dev = sdev.fill_layer(w, 0, L_cap=2528, lengths=lens)
    got = gpu_decode(w, dev, int(lens.max()), L_cap=2528)
    bs = sorted({0, int(np.argmax(lens)), int(np.argmin(lens)), 17, 39})
    pairs = [(b, h) for b in bs for h in range(H)]
    compare(w, got, oracle_pairs(w, 0, lens, pairs), pairs, f"table H={H} r={r} batch 40")


@pytest.mark.parametrize("H,r", SHAPES, ids=[f"H{h}_r{r}" for h, r in SHAPES])
def test_table_shape_rows_past_the_end_are_never_used(H, r):
    """NaN in every row at or past each length: finite outputs, equal to the clean run bit for bit (the lanes'
    coordinates past a head's rank, and padding head slots, read the next head's or the next row's values)."""
    lens = np.array([300, 33, 1, 95], dtype=np.int32)
    w = _w(H, r, 4, 300, 320)
    say(f"[case] table shape H={H} r={r}, NaN past the end")
    dev = sdev.fill_layer(w, 0, L_cap=320, lengths=lens)
    clean = gpu_decode(w, dev, 300, L_cap=320)
    for b in range(4):
        n = int(lens[b])
        for k in ("k_shared", "v_shared", "z_k", "z_v"):
            dev[k][b, n:] = float("nan")
    dirty = gpu_decode(w, dev, 300, L_cap=320)
    assert bool(torch.isfinite(dirty).all())
    assert torch.equal(clean, dirty)


def test_table_shape_matches_general_kernel(monkeypatch):
    """H = 18, r = 55: the matrix-core kernel against the general kernel (LRKV_FORCE_GENERAL) on the same
    inputs, within the bf16 tolerance, and both against the reference."""
    lens = np.array([2048, 1500, 77, 2000], dtype=np.int32)
    w = _w(18, 55, 4, 2048, 2048)
    dev = sdev.fill_layer(w, 0, L_cap=2048, lengths=lens)
    mfma = gpu_decode(w, dev, 2048, L_cap=2048)
    monkeypatch.setenv("LRKV_FORCE_GENERAL", "1")
    assert _granule(w, 2048, 2048) == 32
    gen = gpu_decode(w, dev, 2048, L_cap=2048)
    monkeypatch.delenv("LRKV_FORCE_GENERAL")
    pairs = [(b, h) for b in range(4) for h in range(18)]
    ref = oracle_pairs(w, 0, lens, pairs)
    compare(w, mfma, ref, pairs, "H=18 r=55 matrix-core")
    compare(w, gen, ref, pairs, "H=18 r=55 general")


def test_table_shape_paged_equals_contiguous():
    """H = 18, r = 55 in a shuffled pool of 64-row pages: the same kernel with block-table addressing gives the
    contiguous result bit for bit."""
    lens = np.array([1000, 64, 65, 513], dtype=np.int32)
    w = _w(18, 55, 4, 1024, 1024)
    dev = sdev.fill_layer(w, 0, L_cap=1024, lengths=lens)
    want = gpu_decode(w, dev, 1000, L_cap=1024)
    P, maxp = 64, 1024 // 64
    n_pages = 4 * maxp + 5
    perm = np.random.default_rng(18).permutation(n_pages)[:4 * maxp].astype(np.int32)
    table = torch.from_numpy(perm.reshape(4, maxp).copy()).cuda()
    pools = {}
    for name in ("k_shared", "v_shared", "z_k", "z_v"):
        src = dev[name]
        pool = torch.full((n_pages, P) + tuple(src.shape[2:]), float("nan"), dtype=src.dtype, device="cuda")
        pool[table.reshape(-1).long()] = src.reshape((4 * maxp, P) + tuple(src.shape[2:]))
        pools[name] = pool
    seq_lens = dev["seq_lens"].clone()
    pc = lk.make_paged_cache(pools["k_shared"], pools["v_shared"], pools["z_k"], pools["z_v"], table, seq_lens, P,
                             maxp, n_pages)
    dims = dims_of(w, 1024)
    p = torch.empty((4, 18, 55), dtype=torch.float32, device="cuda")
    lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p)
    out = torch.full((4, 18, 128), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_workspace_bytes(dims, 1000)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    say("[case] table shape H=18 r=55 paged")
    lk.lrkv_decode_paged(dims, pc, 1000, dev["q"], p, dev["B_v"], out, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(out, want)


def test_table_shape_several_queries():
    """H = 12, r = 51 with Q = 3 query tokens per sequence (one virtual sequence per token on the matrix-core
    kernel) against the reference at each token's causal length."""
    lens = np.array([400, 3, 130], dtype=np.int32)
    Q = 3
    w = _w(12, 51, 3, 400, 416)
    dev = sdev.fill_layer(w, 0, L_cap=416, lengths=lens)
    qh = synth.normal(9300, 1.0, 3 * Q * 12 * 128, "bf16").reshape(3, Q, 12, 128)
    dims = dims_of(w, 416)
    q = sdev.to_device(qh)
    p = torch.empty((3, Q, 12, 51), dtype=torch.float32, device="cuda")
    lk.lrkv_absorb_query(lk.make_dims(3 * Q, 12, 128, 51, 416, lk.LRKV_BF16), q, dev["B_k"], p)
    out = torch.full((3, Q, 12, 128), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_multi_workspace_bytes(dims, Q, 400)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    say("[case] table shape H=12 r=51, three query tokens")
    lk.lrkv_decode_multi(dims, Q, lk.make_cache(dev["k_shared"], dev["v_shared"], dev["z_k"], dev["z_v"],
                                                dev["seq_lens"]), 400, q, p, dev["B_v"], out, ws, nbytes)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    host = {b: synth.gen_sequence(w, 0, b, int(lens[b])) for b in range(3)}
    k = np.zeros((3, 416, 128), np.uint16)
    v = np.zeros_like(k)
    zk = np.zeros((3, 12, 416, 51), np.uint16)
    zv = np.zeros_like(zk)
    for b in range(3):
        n = int(lens[b])
        k[b, :n], v[b, :n] = host[b]["k_shared"], host[b]["v_shared"]
        zk[b, :, :n], zv[b, :, :n] = host[b]["z_k"], host[b]["z_v"]
    ref = oracle.lrkv_decode_multi("bf16", qh, k, v, zk, zv, synth.gen_small(w, 0, "B_k"), synth.gen_small(w, 0, "B_v"),
                                   lens)
    seen = (lens[:, None] - Q + np.arange(Q)[None, :] + 1) > 0
    assert np.all(got[~seen] == 0.0)
    err = oracle.relative_error(got[seen].reshape(-1, 128), ref[seen].reshape(-1, 128))
    say(f"  max rel err {err:.3e} (tol {TOL['bf16']:.0e})")
    assert err <= TOL["bf16"]


def test_table_shape_2p5b_layout_at_8k():
    """The 2.5B model's layer layout (H = 18, r = 55) at an 8K context, batch 16: sampled pairs."""
    w = _w(18, 55, 16, 8192, 8192, name="t7_8k")
    lens = np.full(16, 8192, dtype=np.int32)
    say("[case] H=18 r=55, 16 x 8192 rows")
    dev = sdev.fill_layer(w, 0, L_cap=8192, lengths=lens)
    got = gpu_decode(w, dev, 8192, L_cap=8192)
    pairs = [(b, h) for b in (0, 7, 15) for h in (0, 5, 16, 17)]
    compare(w, got, oracle_pairs(w, 0, lens, pairs), pairs, "H=18 r=55 8K")
