"""lrkv_decode_step (a whole decode step -- append, absorb, split pass, merge -- in one launch) against the
separate calls lrkv_append_absorb then lrkv_decode, through the C ABI: p, the outputs, the cache rows and the
lengths must be bit for bit the same after every step of several in a row, and the step's counter words must be
back at zero after every call (they hand work on between the launch's workgroups and are cleared by its last
workgroup).  On the fp32 rank-0 kernel the split pass appends the token and grows the lengths, and the merge
kernel follows.  The separate calls are checked against the reference in test_gpu_decode.py and its neighbours; one
case here also checks the fused step against the reference directly.  Shapes cover the fused path (bf16
matrix-core shapes: d_h 64 and 128, r 0 to 64, one and two waves per SIMD, one and four merge groups), a full
sequence, an empty one, a negative length, appends past max_len (rows written but not seen), and shapes that run
the two calls (fp32; r = 12; the model-table shape H 18 r 55; a batch with more merge workgroups than one
resident round)."""
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


CASES = [  # (dtype, batch, H, d_h, r, lengths, L_cap, max_len)
    ("bf16", 4, 32, 128, 64, [700, 33, 0, 95], 768, 704),
    ("bf16", 3, 16, 128, 48, [64, 1, 200], 256, 256),
    ("bf16", 3, 8, 64, 8, [61, 10, 64], 64, 64),          # sequence 2 is full: nothing appended
    ("bf16", 2, 8, 64, 0, [5, 40], 64, 64),               # r = 0: no absorb
    ("bf16", 4, 18, 128, 55, [300, 33, 1, 95], 320, 320),  # model-table shape (r = 55: the two calls)
    ("bf16", 3, 32, 128, 32, [100, 500, 64], 512, 128),    # sequence 1 grows past max_len: row written, not seen
    ("bf16", 2, 16, 64, 16, [3000, 2900], 3072, 3072),     # long sequences: four merge groups
    ("f32", 2, 8, 64, 0, [10, 63], 64, 64),                # fp32 rank 0: split pass with the append, merge
    ("bf16", 2, 8, 64, 12, [5, 40], 64, 64),               # r = 12: the two calls
]


def _ragged_case(batch=32, H=16):
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 2500, size=batch).astype(np.int32)
    return ("bf16", batch, H, 128, 32, lens.tolist(), 2528, 2528)  # batch >= 32: two waves per SIMD


def _setup(case, negative=None):
    dtype, B, H, d_h, r, lens, L_cap, max_len = case
    w = synth.WORKLOADS["small_bf16"].with_(name="step", batch=B, H=H, d_h=d_h, r=r, dtype=dtype,
                                            L=max(max(lens), 1), L_cap=L_cap, ragged_lo=None)
    lens = np.array(lens, dtype=np.int32)
    dev = sdev.fill_layer(w, 0, lengths=lens)
    if negative is not None:
        dev["seq_lens"][negative] = -1
    return w, dev, sdev.new_rows(w), max_len


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _run(case, fused, steps, negative=None):
    w, dev, rows, max_len = _setup(case, negative)
    B, H, d_h, r = w.batch, w.H, w.d_h, w.r
    dims = dims_of(w)
    cache = cache_of(dev, r)
    p = torch.full((B, H, max(r, 1)), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((B, H, d_h), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = lk.lrkv_decode_step_workspace_bytes(dims, max_len)
    assert nbytes >= lk.lrkv_decode_workspace_bytes(dims, max_len) > 0
    ws = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")  # the counter words start at zero
    sync_at = lk.lrkv_decode_step_sync_offset(dims, max_len) // 4
    zk, zv = (rows["zk_new"], rows["zv_new"]) if r else (None, None)
    pp, bk, bv = (p, dev["B_k"], dev["B_v"]) if r else (None, None, None)
    per_step = []
    for _ in range(steps):
        if fused:
            lk.lrkv_decode_step(dims, cache, max_len, rows["k_new"], rows["v_new"], zk, zv, dev["q"], bk, bv, pp, out,
                                ws, nbytes)
        else:
            lk.lrkv_append_absorb(dims, cache, rows["k_new"], rows["v_new"], zk, zv, dev["q"], bk, pp)
            lk.lrkv_decode(dims, cache, max_len, dev["q"], pp, bv, out, ws, nbytes)
        torch.cuda.synchronize()
        if fused:
            words = ws[sync_at:].view(torch.int32)
            assert int(words[1]) == 0, "a wait of the fused step ran out of its bound"
            assert int(words.abs().sum()) == 0, "counter words not cleared"
        per_step.append({"out": out.clone(), "p": p.clone(), "seq_lens": dev["seq_lens"].clone()})
    final = {k: dev[k].clone() for k in ("k_shared", "v_shared", "z_k", "z_v")}
    return per_step, final, dev


def _check_equal(case, steps=3, negative=None):
    a_steps, a_final, _ = _run(case, False, steps, negative)
    b_steps, b_final, _ = _run(case, True, steps, negative)
    r = case[4]
    for k, (x, y) in enumerate(zip(a_steps, b_steps)):
        assert torch.equal(x["seq_lens"], y["seq_lens"]), f"step {k}: lengths differ"
        assert torch.equal(_bits(x["out"]), _bits(y["out"])), f"step {k}: outputs differ"
        if r:
            assert torch.equal(_bits(x["p"]), _bits(y["p"])), f"step {k}: p differs"
        assert bool(torch.isfinite(y["out"]).all())
    for name in a_final:
        if a_final[name].numel():
            assert torch.equal(_bits(a_final[name]), _bits(b_final[name])), f"cache {name} differs"
    return a_steps


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}_L{max(c[5])}_m{c[7]}")
def test_step_equals_separate_calls(case):
    say(f"[case] decode step {case[:5]} lengths {case[5]} max_len {case[7]}")
    _check_equal(case)


def test_step_two_waves_per_simd():
    case = _ragged_case()
    w = synth.WORKLOADS["small_bf16"].with_(name="step", batch=case[1], H=case[2], d_h=case[3], r=case[4],
                                            dtype="bf16", L=max(case[5]), L_cap=case[6], ragged_lo=None)
    assert lk.lrkv_decode_step_fused(dims_of(w), case[7]), "expected the fused launch"
    say("[case] decode step, batch 32 x 16 heads ragged (two waves per SIMD, fused)")
    _check_equal(case, steps=2)


def test_step_fewest_splits_plan_with_edge_lengths():
    """Long ragged sequences whose plan gives each sequence the fewest splits under a common lane cap (some
    workgroups of the launch have no split), with an empty sequence, one that grows to L_cap and a full one:
    the fused step equals the two calls bit for bit over three steps."""
    case = ("bf16", 6, 32, 128, 64, [32768, 0, 32799, 32800, 31000, 20000], 32800, 32800)
    w, dev, _, max_len = _setup(case)
    dims = dims_of(w)
    G = lk.lrkv_decode_num_splits(dims, max_len)[0]
    W = torch.empty(6, dtype=torch.int32, device="cuda")
    S = torch.empty(6, dtype=torch.int32, device="cuda")
    lk.lrkv_decode_split_plan(dims, max_len, dev["seq_lens"], 1, W, S)
    torch.cuda.synchronize()
    S = S.cpu().tolist()
    say(f"[case] decode step, fewest-splits plan: G={G}, splits {S}")
    assert sum(S) < G and S[1] == 1
    _check_equal(case)


def test_step_many_merges_runs_the_calls():
    """A batch whose merge workgroups would not fit one resident round runs the two calls; same results."""
    case = _ragged_case(batch=40, H=32)
    say("[case] decode step, batch 40 x 32 heads (the two calls)")
    _check_equal(case, steps=2)


F32_FUSED = [  # (dtype, batch, H, d_h, r, lengths, L_cap, max_len): fp32 rank 0, fused on its matrix-core kernel
    ("f32", 16, 8, 64, 0, [0, 1, 31, 32, 33, 255, 256, 100, 64, 63, 65, 200, 2, 128, 129, 17], 256, 256),
    ("f32", 20, 32, 128, 0, [700, 33, 0, 95, 1000, 1023, 1024, 5, 640, 641, 639, 300, 1, 2, 900, 960, 961, 31,
                             32, 699], 1024, 700),   # max_len below L_cap: rows written past it, not seen
    ("f32", 17, 16, 128, 0, [2048 - k for k in range(17)], 2048, 2048),  # full and nearly full sequences
    ("f32", 3, 32, 128, 0, [4000, 4095, 17], 4096, 4096),  # many splits a sequence: four merge groups
]


@pytest.mark.parametrize("case", F32_FUSED, ids=lambda c: f"f32_B{c[1]}_H{c[2]}_d{c[3]}_cap{c[6]}_m{c[7]}")
def test_step_fp32_rank0_fused(case):
    w, _, _, max_len = _setup(case)
    assert lk.lrkv_decode_step_fused(dims_of(w), max_len), "expected the fused launch"
    say(f"[case] fp32 rank-0 fused step {case[:5]} L_cap {case[6]} max_len {case[7]}")
    _check_equal(case)


def test_step_fp32_rank0_ragged_batch():
    """64 ragged sequences, 32 heads (the fp32 rank-0 workload's shape at shorter lengths), and one negative
    length: fused, bit for bit the two calls."""
    rng = np.random.default_rng(78)
    lens = rng.integers(1, 2500, size=64).astype(np.int32).tolist()
    case = ("f32", 64, 32, 128, 0, lens, 2528, 2528)
    w, _, _, max_len = _setup(case)
    assert lk.lrkv_decode_step_fused(dims_of(w), max_len), "expected the fused launch"
    say("[case] fp32 rank-0 fused step, 64 ragged sequences, sequence 5 negative")
    steps = _check_equal(case, steps=2, negative=5)
    assert steps[-1]["seq_lens"].cpu().tolist()[5] == -1
    assert float(steps[-1]["out"][5].abs().max()) == 0.0


def test_step_negative_length():
    case = ("bf16", 3, 8, 64, 16, [20, 7, 33], 64, 64)
    say("[case] decode step with a negative length")
    steps = _check_equal(case, steps=2, negative=1)
    assert steps[-1]["seq_lens"].cpu().tolist() == [22, -1, 35]
    assert float(steps[-1]["out"][1].abs().max()) == 0.0


def test_step_against_reference():
    """One fused step against the reference on the cache with the appended token."""
    case = CASES[0]
    say("[case] decode step against the reference")
    steps, _, dev = _run(case, True, 1)
    w, _, rows, _ = _setup(case)
    lens = np.array(case[5], dtype=np.int32)
    grown = np.minimum(lens + 1, case[6])
    assert steps[0]["seq_lens"].cpu().numpy().tolist() == grown.tolist()
    new = synth.gen_new_rows(w, 0)
    B, H, r, cap = w.batch, w.H, w.r, int(grown.max())
    k = np.zeros((B, cap, w.d_h), np.uint16)
    v = np.zeros_like(k)
    zk = np.zeros((B, H, cap, r), np.uint16)
    zv = np.zeros_like(zk)
    for b in range(B):
        n = int(lens[b])
        if n:
            s = synth.gen_sequence(w, 0, b, n)
            k[b, :n], v[b, :n], zk[b, :, :n], zv[b, :, :n] = s["k_shared"], s["v_shared"], s["z_k"], s["z_v"]
        k[b, n], v[b, n] = new["k_new"][b], new["v_new"][b]
        zk[b, :, n], zv[b, :, n] = new["zk_new"][b], new["zv_new"][b]
    ref = oracle.lrkv_decode("bf16", synth.gen_small(w, 0, "q"), k, v, zk, zv, synth.gen_small(w, 0, "B_k"),
                             synth.gen_small(w, 0, "B_v"), grown)
    err = oracle.relative_error(steps[0]["out"].cpu().numpy().reshape(-1, w.d_h).astype(np.float64),
                                ref.reshape(-1, w.d_h))
    say(f"  max rel err {err:.3e} (tol {TOL['bf16']:.0e})")
    assert err <= TOL["bf16"]


def test_step_graph_replays():
    """The fused step captured as a HIP graph: replays with eager work between them match direct launches bit for
    bit, step after step (the counters clear themselves, so every replay starts from zero)."""
    case = ("bf16", 3, 32, 128, 64, [300, 397, 494], 544, 500)
    say("[case] decode step graph replays")
    runs = []
    for _ in range(3):
        w, dev, rows, max_len = _setup(case)
        dims = dims_of(w)
        nbytes = lk.lrkv_decode_step_workspace_bytes(dims, max_len)
        runs.append(dict(dev=dev, rows=rows, dims=dims, cache=cache_of(dev, w.r),
                         ws=torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda"), nbytes=nbytes,
                         p=torch.zeros((w.batch, w.H, w.r), dtype=torch.float32, device="cuda"),
                         out=torch.zeros((w.batch, w.H, w.d_h), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()

    def step(x, stream):
        lk.lrkv_decode_step(x["dims"], x["cache"], max_len, x["rows"]["k_new"], x["rows"]["v_new"], x["rows"]["zk_new"],
                            x["rows"]["zv_new"], x["dev"]["q"], x["dev"]["B_k"], x["dev"]["B_v"], x["p"], x["out"],
                            x["ws"], x["nbytes"], stream)

    warm, direct, graphed = runs
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(warm, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graphed, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for k in range(4):
        step(direct, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.ones(1024, device="cuda").sum().item()  # eager work between replays
        for name in ("seq_lens", "k_shared", "v_shared", "z_k", "z_v"):
            assert torch.equal(_bits(direct["dev"][name]), _bits(graphed["dev"][name])), f"{name}, replay {k}"
        assert torch.equal(_bits(direct["out"]), _bits(graphed["out"])), f"out, replay {k}"
        assert torch.equal(_bits(direct["p"]), _bits(graphed["p"])), f"p, replay {k}"
        sync_at = lk.lrkv_decode_step_sync_offset(graphed["dims"], max_len) // 4
        assert int(graphed["ws"][sync_at:].view(torch.int32).abs().sum()) == 0
