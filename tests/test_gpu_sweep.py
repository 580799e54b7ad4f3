"""GPU parity over seeded random shapes and lengths: single-token decode, multi-token decode and the rotary
variant, bf16 and fp32, against the fp64 reference through the C ABI; and the fused decode step on random
shapes, bit for bit against the separate calls (append and absorb, then decode) over two steps in a row (and a set
of fp32 rank-0 steps, whose split pass appends the token and grows the lengths before the merge); the
paged cache (random page sizes, pool permutations with NaN spare pages) and the normalised variant on random
shapes, checked as in test_gpu_paged.py and test_gpu_normed.py.  Lengths mix random values with the tile and block edges (0, 1, 31-33, 63-65, 127-129, 255-257).  Metric and
tolerances as in test_gpu_decode.py.  LRKV_SWEEP_CASES and LRKV_SWEEP_SEED (read when the module is collected)
widen the sweep or draw another one; the defaults are the committed cases."""
import os

import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from oracle import rope
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, gpu_decode, say  # noqa: E402

EDGE = [0, 1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 255, 256, 257]
N_CASES = int(os.environ.get("LRKV_SWEEP_CASES", "36"))
SEED = int(os.environ.get("LRKV_SWEEP_SEED", "20261202"))


def _cases(seed=SEED, n=N_CASES):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ("decode", "multi", "rope")[i % 3]
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        H = int(rng.choice([8, 16, 24, 32] if dtype == "bf16" else [4, 8, 32]))
        d_h = int(rng.choice([64, 128]))
        r = int(rng.choice([0, 8, 16, 32, 48, 64]))
        if dtype == "f32" and kind == "rope":
            r = int(rng.choice([0, 4]))  # the general kernel's rotary mode keeps its tile in LDS
        B = int(rng.integers(1, 5))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 1600)) for _ in range(B)]
        if max(lens) == 0:
            lens[0] = 1
        Q = int(rng.integers(2, 7)) if kind == "multi" else 1
        out.append((kind, dtype, B, H, d_h, r, Q, tuple(lens)))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}_{c[1]}_B{c[2]}_H{c[3]}_d{c[4]}_r{c[5]}_Q{c[6]}")
def test_random_shape_matches_reference(case):
    kind, dtype, B, H, d_h, r, Q, lens = case
    L = max(lens)
    w = synth.WORKLOADS["small_bf16"].with_(name="sweep", batch=B, H=H, d_h=d_h, r=r, dtype=dtype, L=L,
                                            L_cap=(L + 31) // 32 * 32 + 32, ragged_lo=None)
    la = np.array(lens, dtype=np.int32)
    say(f"[case] {case}")
    dev = sdev.fill_layer(w, 0, lengths=la)
    host = synth.gen_host(w, 0, lengths=la)
    if kind == "decode":
        got = gpu_decode(w, dev, L).cpu().numpy()
        ref = oracle.lrkv_decode(dtype, host["q"], host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                                 host["B_k"], host["B_v"], la).reshape(B, H, d_h)
        seen = la > 0
    elif kind == "rope":
        dims = dims_of(w)
        table = torch.empty((w.cap, d_h // 2, 2), dtype=torch.float32, device="cuda")
        lk.lrkv_rope_table(d_h, w.cap, 10000.0, table)
        out = torch.full((B, H, d_h), float("nan"), dtype=torch.float32, device="cuda")
        nbytes = lk.lrkv_decode_rope_workspace_bytes(dims, L)
        ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
        lk.lrkv_decode_rope(dims, cache_of(dev, r), L, dev["q"], dev["B_k"] if r else None, table,
                            dev["B_v"] if r else None, out, ws, nbytes)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = rope.decode_rope(dtype, host["q"], host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                               host["B_k"], host["B_v"], la, base=10000.0)
        seen = la > 0
    else:
        qh = synth.normal(9400 + B * 7 + H, 1.0, B * Q * H * d_h, dtype).reshape(B, Q, H, d_h)
        q = sdev.to_device(qh)
        dims = dims_of(w)
        p = torch.empty((B, Q, H, max(r, 1)), dtype=torch.float32, device="cuda")
        if r:
            lk.lrkv_absorb_query(lk.make_dims(B * Q, H, d_h, r, w.cap, dims.dtype), q, dev["B_k"], p)
        out = torch.full((B, Q, H, d_h), float("nan"), dtype=torch.float32, device="cuda")
        nbytes = lk.lrkv_decode_multi_workspace_bytes(dims, Q, L)
        ws = torch.empty(max(nbytes, 256) // 4 + 64, dtype=torch.float32, device="cuda")
        lk.lrkv_decode_multi(dims, Q, cache_of(dev, r), L, q, p if r else None, dev["B_v"] if r else None, out, ws,
                             nbytes)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.lrkv_decode_multi(dtype, qh, host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                                       host["B_k"], host["B_v"], la)
        seen = (la[:, None] - Q + np.arange(Q)[None, :] + 1) > 0  # [B][Q]: queries that see a row
    assert np.all(got[~seen] == 0.0), "a query that sees no row must give 0"
    err = oracle.relative_error(got[seen].reshape(-1, d_h), ref[seen].reshape(-1, d_h))
    say(f"  max rel err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


def _step_cases(seed=SEED + 1, n=max(1, N_CASES // 3)):
    """(dtype, batch, H, d_h, r, lengths, L_cap, max_len): mostly the fused path's shapes (bf16 matrix-core
    kernel), some that run the two calls (fp32, r off the kernel's set); lengths include 0, full sequences
    (L = L_cap, nothing appended) and sequences that grow past max_len (the row written but not seen)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = "bf16" if rng.random() < 0.8 else "f32"
        H = int(rng.choice([8, 16, 32]))
        d_h = int(rng.choice([64, 128]))
        r = int(rng.choice([0, 8, 16, 32, 48, 64] if rng.random() < 0.85 else [4, 12, 20]))
        B = int(rng.integers(1, 6))
        L_cap = int(rng.choice([64, 256, 1024, 2048]))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(1, L_cap + 1)) for _ in range(B)]
        lens = [min(x, L_cap) for x in lens]
        max_len = L_cap if rng.random() < 0.7 else int(rng.integers(1, L_cap + 1))
        out.append((dtype, B, H, d_h, r, tuple(lens), L_cap, max_len))
    return out


@pytest.mark.parametrize("case", _step_cases(),
                         ids=lambda c: f"step_{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}_cap{c[6]}_max{c[7]}")
def test_random_step_matches_separate_calls(case):
    from test_gpu_step import _check_equal
    say(f"[case] step {case}")
    dtype, B, H, d_h, r, lens, L_cap, max_len = case
    _check_equal((dtype, B, H, d_h, r, list(lens), L_cap, max_len), steps=2)


def _shape(rng, dtype):
    """(H, d_h, r): the matrix-core kernels' shapes mostly, the general kernel's now and then."""
    if rng.random() < 0.2:
        return (4, 48, 12) if dtype == "bf16" else (4, 16, 4)
    if dtype == "f32":
        return (int(rng.choice([8, 32])), int(rng.choice([64, 128])), int(rng.choice([0, 8])))
    return int(rng.choice([8, 16, 32])), int(rng.choice([64, 128])), int(rng.choice([0, 8, 16, 32, 48, 64]))


def _paged_cases(seed=SEED + 2, n=max(1, N_CASES // 6)):
    """(dtype, batch, H, d_h, r, L_cap, page_rows, lengths) as in test_gpu_paged.py."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        H, d_h, r = _shape(rng, dtype)
        P = int(rng.choice([32, 64, 128, 256]))
        L_cap = P * int(rng.integers(1, 9))
        B = int(rng.integers(1, 5))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(0, L_cap + 1)) for _ in range(B)]
        lens = [min(x, L_cap) for x in lens]
        if max(lens) == 0:
            lens[0] = 1
        out.append((dtype, B, H, d_h, r, L_cap, P, lens))
    return out


def _normed_cases(seed=SEED + 3, n=max(1, N_CASES // 6)):
    """(dtype, batch, H, d_h, r, lengths) as in test_gpu_normed.py."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        H, d_h, r = _shape(rng, dtype)
        B = int(rng.integers(1, 5))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(1, 1200)) for _ in range(B)]
        if max(lens) == 0:
            lens[0] = 1
        out.append((dtype, B, H, d_h, r, lens))
    return out


@pytest.mark.parametrize("case", _paged_cases(), ids=lambda c: f"paged_{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}_P{c[6]}")
def test_random_paged_decode(case):
    from test_gpu_paged import test_paged_decode
    test_paged_decode(case)


@pytest.mark.parametrize("case", _normed_cases(), ids=lambda c: f"normed_{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
def test_random_normed_decode(case):
    from test_gpu_normed import test_decode_normed_matches_reference
    test_decode_normed_matches_reference(case)


def _f32_step_cases(seed=SEED + 4, n=max(1, N_CASES // 6)):
    """fp32 rank-0 decode steps on the fp32 matrix-core kernel: (dtype, batch, H, d_h, r, lengths, L_cap,
    max_len) with batches from one sequence to 70, lengths at the block and tile edges, empty and full."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(rng.choice([8, 16, 32]))
        d_h = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 71))
        L_cap = 32 * int(rng.integers(2, 129))
        lens = [int(rng.choice(EDGE)) if rng.random() < 0.4 else int(rng.integers(0, L_cap + 1)) for _ in range(B)]
        lens = [min(x, L_cap) for x in lens]
        max_len = L_cap if rng.random() < 0.7 else int(rng.integers(1, L_cap + 1))
        out.append(("f32", B, H, d_h, 0, tuple(lens), L_cap, max_len))
    return out


@pytest.mark.parametrize("case", _f32_step_cases(),
                         ids=lambda c: f"f32step_B{c[1]}_H{c[2]}_d{c[3]}_cap{c[6]}_max{c[7]}")
def test_random_fp32_rank0_step(case):
    from test_gpu_step import _check_equal
    dtype, B, H, d_h, r, lens, L_cap, max_len = case
    dims = lk.make_dims(B, H, d_h, r, L_cap, lk.LRKV_F32)
    assert lk.lrkv_decode_step_fused(dims, max_len), "the fp32 rank-0 step folds the append into its split pass"
    say(f"[case] fp32 rank-0 step B={B} H={H} d_h={d_h} L_cap={L_cap} max_len={max_len}")
    _check_equal((dtype, B, H, d_h, r, list(lens), L_cap, max_len), steps=2)
