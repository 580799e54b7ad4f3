"""GPU parity of the LRKV decode library against the CPU reference.

All calls go through the C ABI (rank_shared_kv_amd -> liblrkv.so).  Outputs
are compared element by element with the fp64 reference on the same seeded
inputs, with the metric max over (b, h) of ||gpu - ref||_inf / ||ref||_inf:
1e-5 for fp32 inputs, 2e-3 for bf16 caches with fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, compare, dims_of, gpu_decode, oracle_pairs, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _all_pairs(w):
    return [(b, h) for b in range(w.batch) for h in range(w.H)]


def _run_and_check(w, lengths=None, L_cap=None, pairs=None, label=None, split_calls=False):
    lens = synth.seq_lengths(w) if lengths is None else np.asarray(lengths, dtype=np.int32)
    cap = L_cap or w.cap
    label = label or w.name
    say(f"[case] {label}: B={w.batch} H={w.H} d_h={w.d_h} r={w.r} {w.dtype} L_cap={cap} lens[:8]={lens[:8].tolist()}")
    dev = sdev.fill_layer(w, 0, L_cap=cap, lengths=lens)
    max_len = int(lens.max(initial=0))
    got = gpu_decode(w, dev, max_len, L_cap=cap, split_calls=split_calls)
    pairs = pairs or _all_pairs(w)
    ref = oracle_pairs(w, 0, lens, pairs)
    compare(w, got, ref, pairs, label)
    return got, dev


def test_tiny_fp32_all_pairs():
    _run_and_check(synth.WORKLOADS["tiny_fp32"])


def test_small_bf16_all_pairs():
    _run_and_check(synth.WORKLOADS["small_bf16"])


@pytest.mark.parametrize("splits", [None, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(8, 64, 16), (16, 128, 48), (32, 128, 64), (8, 64, 8), (32, 128, 32)])
def test_ragged_edges(dtype, shape, splits, monkeypatch):
    """Lengths 0, 1, tile boundaries +-1 and a few tiles, with the default split plan and with the plan forced
    to three splits per sequence (LRKV_SPLITS, read at every call)."""
    H, d_h, r = shape
    if splits:
        monkeypatch.setenv("LRKV_SPLITS", str(splits))
    w = synth.WORKLOADS["ragged"].with_(name=f"edges_{dtype}_{H}_{d_h}_{r}_s{splits}", batch=8, H=H, d_h=d_h, r=r,
                                        dtype=dtype, L=700, L_cap=704, ragged_lo=None)
    lens = [0, 1, 31, 32, 33, 127, 129, 700]
    G, _ = lk.lrkv_decode_num_splits(dims_of(w, 704), 700)
    if splits:
        assert G == splits * 8
    pairs = [(b, h) for b in range(8) for h in sorted({0, H // 2, H - 1})]
    _run_and_check(w, lengths=lens, L_cap=704, pairs=pairs)


def test_r0_fp32_matches_mqa_reference():
    w = synth.WORKLOADS["ragged_mqa_fp32"].with_(batch=4)
    lens = np.array([512, 1000, 3001, 777], dtype=np.int32)
    say(f"[case] r=0 fp32 vs MQA reference, lens={lens.tolist()}")
    dev = sdev.fill_layer(w, 0, L_cap=w.cap, lengths=lens)
    got = gpu_decode(w, dev, int(lens.max()))
    pairs = [(b, h) for b in range(4) for h in (0, 7, 31)]
    ref = oracle_pairs(w, 0, lens, pairs, mqa=True)
    compare(w, got, ref, pairs, "r0_fp32_vs_mqa")


def _r0_and_zero_latents(dtype, H, d_h, r):
    """Outputs of the same problem with r = 0 and with rank r but all latents zero."""
    w0 = synth.WORKLOADS["ragged"].with_(name="r0", batch=3, H=H, d_h=d_h, r=0, dtype=dtype, L=600, L_cap=608,
                                         ragged_lo=None)
    lens = np.array([600, 45, 257], dtype=np.int32)
    dev0 = sdev.fill_layer(w0, 0, L_cap=608, lengths=lens)
    out0 = gpu_decode(w0, dev0, 600, L_cap=608)
    wr = w0.with_(r=r)
    devr = dict(dev0)
    devr["z_k"] = torch.zeros((3, 608, H, r), dtype=dev0["k_shared"].dtype, device="cuda")
    devr["z_v"] = torch.zeros_like(devr["z_k"])
    devr["B_k"] = sdev.to_device(synth.gen_small(wr, 0, "B_k"))
    devr["B_v"] = sdev.to_device(synth.gen_small(wr, 0, "B_v"))
    outr = gpu_decode(wr, devr, 600, L_cap=608)
    return out0, outr


@pytest.mark.parametrize("dtype,H,d_h,r", [("bf16", 32, 128, 32), ("bf16", 16, 64, 8), ("f32", 4, 16, 4),
                                           ("f32", 8, 32, 16)])
def test_r0_equals_zero_latents_bitwise(dtype, H, d_h, r):
    """The private branch adds exact zeros: r = 0 and r > 0 with zero latents agree bit for bit when the same
    kernel runs both (bf16 matrix-core kernel; general kernel for these fp32 shapes)."""
    say(f"[case] r=0 vs zero latents, {dtype} H={H} d_h={d_h} r={r}")
    out0, outr = _r0_and_zero_latents(dtype, H, d_h, r)
    assert torch.equal(out0, outr)


def test_r0_fp32_matrix_kernel_matches_zero_latents():
    """fp32 with r = 0 runs on the fp32 matrix-core kernel, r > 0 on the general kernel: same result within
    the fp32 tolerance."""
    say("[case] r=0 fp32 (matrix cores) vs r=32 zero latents (general kernel)")
    out0, outr = _r0_and_zero_latents("f32", 32, 128, 32)
    g, o = out0.double().cpu().numpy(), outr.double().cpu().numpy()
    err = max(np.abs(g[b, h] - o[b, h]).max() / np.abs(o[b, h]).max() for b in range(3) for h in range(32))
    say(f"  max rel diff {err:.3e}")
    assert err <= TOL["f32"]


@pytest.mark.parametrize("H,d_h", [(8, 64), (16, 128), (32, 128), (32, 64)])
def test_r0_fp32_edges_match_mqa_reference(H, d_h):
    """fp32 r = 0 (matrix-core kernel): lengths 0, 1, tile boundaries +-1 and a few tiles, against the
    reference's MQA path."""
    w = synth.WORKLOADS["ragged_mqa_fp32"].with_(name=f"r0_edges_{H}_{d_h}", batch=8, H=H, d_h=d_h, L=700,
                                                 L_cap=704, ragged_lo=None)
    lens = np.array([0, 1, 31, 32, 33, 127, 129, 700], dtype=np.int32)
    say(f"[case] r=0 fp32 edges H={H} d_h={d_h} lens={lens.tolist()}")
    dev = sdev.fill_layer(w, 0, L_cap=704, lengths=lens)
    got = gpu_decode(w, dev, 700, L_cap=704)
    pairs = [(b, h) for b in range(1, 8) for h in sorted({0, H // 2, H - 1})]
    ref = oracle_pairs(w, 0, lens, pairs, mqa=True)
    compare(w, got, ref, pairs, f"r0_fp32_edges_{H}_{d_h}")
    assert torch.equal(got[0], torch.zeros_like(got[0]))  # empty sequence


@pytest.mark.parametrize("occ", [1, 2])
@pytest.mark.parametrize("dtype,H,d_h,r", [("f32", 32, 128, 0), ("f32", 16, 64, 0), ("bf16", 32, 128, 64),
                                           ("bf16", 16, 128, 48)])
def test_occupancy_override(occ, dtype, H, d_h, r, monkeypatch):
    """LRKV_OCCUPANCY (a tuning override) selects the matrix-core kernels built for one or two waves per SIMD,
    with their own register rings and a grid of 256 x occupancy workgroups: both against the reference."""
    monkeypatch.setenv("LRKV_OCCUPANCY", str(occ))
    w = synth.WORKLOADS["ragged"].with_(name=f"occ{occ}_{dtype}_{H}_{r}", batch=5, H=H, d_h=d_h, r=r, dtype=dtype,
                                        L=2600, L_cap=2624, ragged_lo=None)
    lens = np.array([2600, 31, 1200, 0, 777], dtype=np.int32)
    G, chunk = lk.lrkv_decode_num_splits(dims_of(w, 2624), 2600)
    assert G == min(256 * occ, 5 * ((2600 + chunk - 1) // chunk)) and chunk > 32, (G, chunk)
    say(f"[case] occupancy {occ}: {dtype} H={H} d_h={d_h} r={r}, G={G}")
    dev = sdev.fill_layer(w, 0, L_cap=2624, lengths=lens)
    got = gpu_decode(w, dev, 2600, L_cap=2624)
    assert torch.equal(got[3], torch.zeros_like(got[3]))
    pairs = [(b, h) for b in (0, 1, 2, 4) for h in sorted({0, H // 2, H - 1})]
    compare(w, got, oracle_pairs(w, 0, lens, pairs, mqa=(r == 0)), pairs, f"occupancy {occ}")


def test_partial_plus_merge_equals_decode_and_is_deterministic():
    w = synth.WORKLOADS["small_bf16"]
    lens = synth.seq_lengths(w)
    dev = sdev.fill_layer(w, 0)
    a = gpu_decode(w, dev, int(lens.max()))
    b = gpu_decode(w, dev, int(lens.max()), split_calls=True)
    c = gpu_decode(w, dev, int(lens.max()))
    assert torch.equal(a, b) and torch.equal(a, c)


def test_batch_independence():
    """Changing one sequence's cache leaves the other sequences' outputs bit for bit unchanged."""
    w = synth.WORKLOADS["small_bf16"].with_(batch=4, L=300)
    lens = np.array([300, 120, 300, 7], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    a = gpu_decode(w, dev, 300)
    dev["k_shared"][1].mul_(-1.5)
    dev["z_v"][1].add_(1.0)
    b = gpu_decode(w, dev, 300)
    for s in (0, 2, 3):
        assert torch.equal(a[s], b[s])
    assert not torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,H,d_h,r", [("bf16", 32, 128, 64), ("bf16", 2, 64, 2048), ("bf16", 2, 64, 2056),
                                           ("f32", 2, 32, 1024), ("f32", 2, 32, 1028), ("bf16", 3, 24, 55)])
def test_absorb_matches_reference(dtype, H, d_h, r):
    """p = q B^K against the reference's fp64 product (oracle.absorb_query), on the vector path and on ranks past
    it (r > 2048 for bf16, r > 1024 for fp32, r not a multiple of a 16-byte vector), where the scalar kernel
    runs: every rank gets a complete p."""
    w = synth.WORKLOADS["long_context"].with_(name=f"absorb_{dtype}_{H}_{d_h}_{r}", batch=2, H=H, d_h=d_h, r=r,
                                              dtype=dtype)
    say(f"[case] absorb {dtype} H={H} d_h={d_h} r={r}")
    q = synth.gen_small(w, 0, "q")
    Bk = synth.gen_small(w, 0, "B_k")
    dims = dims_of(w)
    p = torch.full((2, w.H, w.r), float("nan"), dtype=torch.float32, device="cuda")
    lk.lrkv_absorb_query(dims, sdev.to_device(q), sdev.to_device(Bk), p)
    torch.cuda.synchronize()
    ref = oracle.absorb_query(dtype, q, Bk)
    got = p.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    say(f"  max rel err {err:.3e}")
    assert err < 1e-6, err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_then_decode(dtype):
    """Append one token after a prefill of L-1 rows: rows land at seq_lens[b], lengths advance, decode agrees."""
    w = synth.WORKLOADS["ragged"].with_(name=f"append_{dtype}", batch=3, H=16, d_h=128, r=48, dtype=dtype, L=260,
                                        L_cap=264, ragged_lo=None)
    full = np.array([260, 33, 1], dtype=np.int32)
    say(f"[case] append after prefill {dtype}")
    dev = sdev.fill_layer(w, 0, L_cap=264, lengths=full)
    ref_dev = {k: v.clone() for k, v in dev.items()}
    # remove the last row of each sequence, then append it back through the library
    host = {b: synth.gen_sequence(w, 0, b, int(full[b])) for b in range(3)}
    k_new = np.stack([host[b]["k_shared"][-1] for b in range(3)])
    v_new = np.stack([host[b]["v_shared"][-1] for b in range(3)])
    zk_new = np.stack([host[b]["z_k"][:, -1] for b in range(3)])
    zv_new = np.stack([host[b]["z_v"][:, -1] for b in range(3)])
    for b in range(3):
        n = int(full[b]) - 1
        dev["k_shared"][b, n:].zero_()
        dev["v_shared"][b, n:].zero_()
        dev["z_k"][b, n:].zero_()
        dev["z_v"][b, n:].zero_()
    dev["seq_lens"] = torch.from_numpy(full - 1).cuda()
    dims = dims_of(w, 264)
    lk.lrkv_cache_append(dims, cache_of(dev, w.r), sdev.to_device(k_new), sdev.to_device(v_new),
                         sdev.to_device(zk_new), sdev.to_device(zv_new))
    torch.cuda.synchronize()
    assert dev["seq_lens"].cpu().numpy().tolist() == full.tolist()
    for k in ("k_shared", "v_shared", "z_k", "z_v"):
        assert torch.equal(dev[k], ref_dev[k]), k
    got = gpu_decode(w, dev, 260, L_cap=264)
    pairs = [(b, h) for b in range(3) for h in range(0, 16, 5)]
    compare(w, got, oracle_pairs(w, 0, full, pairs), pairs, f"append_{dtype}")


def test_append_to_full_sequence_is_dropped():
    w = synth.WORKLOADS["small_bf16"].with_(batch=2, L=16)
    lens = np.array([16, 15], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    before = {k: v.clone() for k, v in dev.items()}
    rows = sdev.new_rows(w)
    lk.lrkv_cache_append(dims_of(w), cache_of(dev, w.r), rows["k_new"], rows["v_new"], rows["zk_new"],
                         rows["zv_new"])
    torch.cuda.synchronize()
    assert dev["seq_lens"].cpu().tolist() == [16, 16]
    assert torch.equal(dev["k_shared"][0], before["k_shared"][0])   # full: untouched
    assert torch.equal(dev["k_shared"][1, 15], rows["k_new"][1])     # appended at row 15
    assert torch.equal(dev["z_v"][1, 15], rows["zv_new"][1])


def test_empty_and_zero_max_len():
    w = synth.WORKLOADS["small_bf16"].with_(batch=3, L=64)
    lens = np.array([0, 0, 0], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    out = gpu_decode(w, dev, 0)
    assert torch.count_nonzero(out) == 0
    lens = np.array([0, 64, 0], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    out = gpu_decode(w, dev, 64)
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
    assert torch.count_nonzero(out[1]) > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(32, 128, 64), (16, 128, 48), (8, 64, 8), (32, 128, 0), (8, 64, 0)])
def test_rows_past_the_end_are_never_used(dtype, shape):
    """Rows at or past seq_lens[b] hold NaN: outputs must stay finite and equal the clean run bit for bit."""
    H, d_h, r = shape
    w = synth.WORKLOADS["ragged"].with_(name=f"poison_{dtype}_{H}_{r}", batch=4, H=H, d_h=d_h, r=r, dtype=dtype,
                                        L=300, L_cap=320, ragged_lo=None)
    lens = np.array([300, 33, 1, 95], dtype=np.int32)
    say(f"[case] NaN past the end, {dtype} H={H} d_h={d_h} r={r}")
    dev = sdev.fill_layer(w, 0, L_cap=320, lengths=lens)
    clean = gpu_decode(w, dev, 300, L_cap=320)
    nan = float("nan")
    for b in range(4):
        n = int(lens[b])
        dev["k_shared"][b, n:] = nan
        dev["v_shared"][b, n:] = nan
        if r > 0:
            dev["z_k"][b, n:] = nan
            dev["z_v"][b, n:] = nan
    dirty = gpu_decode(w, dev, 300, L_cap=320)
    assert bool(torch.isfinite(dirty).all())
    assert torch.equal(clean, dirty)


@pytest.mark.parametrize("dtype,H,d_h,r", [("bf16", 32, 128, 64), ("f32", 32, 128, 0), ("f32", 8, 64, 16)])
@pytest.mark.parametrize("mix", ["one_long", "skewed", "all_empty"])
def test_length_proportional_splits(dtype, H, d_h, r, mix):
    """Splits are dealt to sequences by length on the device: one long sequence among empty ones, a skewed
    mix, and an all-empty batch (bf16 and fp32 matrix-core kernels, general kernel)."""
    lens = {"one_long": [0] * 15 + [5000],
            "skewed": [1, 2, 3000, 33, 0, 700, 64, 65, 4999, 31, 32, 5000, 128, 0, 1, 96],
            "all_empty": [0] * 16}[mix]
    lens = np.array(lens, dtype=np.int32)
    w = synth.WORKLOADS["ragged"].with_(name=f"lp_{mix}_{dtype}_{H}_{d_h}_{r}", batch=16, H=H, d_h=d_h, r=r,
                                        dtype=dtype, L=5000, L_cap=5024, ragged_lo=None)
    G, chunk = lk.lrkv_decode_num_splits(dims_of(w, 5024), 5000)
    say(f"[case] length-proportional splits {mix} {dtype} H={H} d_h={d_h} r={r}: G={G} granule={chunk}")
    dev = sdev.fill_layer(w, 0, L_cap=5024, lengths=lens)
    got = gpu_decode(w, dev, 5000, L_cap=5024)
    live = [b for b in range(16) if lens[b] > 0]
    for b in range(16):
        if lens[b] == 0:
            assert torch.equal(got[b], torch.zeros_like(got[b]))
    if live:
        pairs = [(b, h) for b in live for h in sorted({0, H - 1})]
        ref = oracle_pairs(w, 0, lens, pairs, mqa=(r == 0))
        compare(w, got, ref, pairs, f"lp_{mix}")


@pytest.mark.parametrize("dtype,H,r", [("bf16", 32, 64), ("f32", 6, 5), ("bf16", 18, 55)])
def test_latents_from_head_major(dtype, H, r):
    """lrkv_latents_to_token_major: per-head latents [batch][H][L_cap][r] become the token-major layout bit
    for bit, and a decode on the converted cache equals the decode of the same cache filled token-major."""
    w = synth.WORKLOADS["ragged"].with_(name=f"layout_{dtype}_{H}_{r}", batch=3, H=H, d_h=64, r=r, dtype=dtype,
                                        L=300, L_cap=320, ragged_lo=None)
    lens = np.array([300, 1, 129], dtype=np.int32)
    say(f"[case] latents from the per-head layout {dtype} H={H} r={r}")
    dev = sdev.fill_layer(w, 0, L_cap=320, lengths=lens)
    want = gpu_decode(w, dev, 300, L_cap=320)
    conv = dict(dev)
    dims = dims_of(w, 320)
    for name in ("z_k", "z_v"):
        head_major = dev[name].permute(0, 2, 1, 3).contiguous()   # [batch][H][L_cap][r]
        dst = torch.full_like(dev[name], float("nan"))
        lk.lrkv_latents_to_token_major(dims, head_major, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst.view(torch.int16 if dtype == "bf16" else torch.int32),
                           dev[name].view(torch.int16 if dtype == "bf16" else torch.int32))
        conv[name] = dst
    assert torch.equal(gpu_decode(w, conv, 300, L_cap=320), want)
