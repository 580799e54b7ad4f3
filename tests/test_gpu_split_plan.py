"""The device split plan (lrkv_decode_split_plan) against the plan as documented in include/lrkv.h, written out
here in plain integer arithmetic: for every sequence its first workgroup W_b and split count S_b, exactly.

With n_b the 32-row blocks of sequence b (its length clamped to [0, max_len], grown by one for the fused step's
append when 0 <= L < L_cap), ntl = granule / 32 and G the launch's workgroups:
  - fewest splits, when the batch holds at most 64 sequences and the least M with
    sum_b max(1, ceil(n_b / (M ntl))) <= G is at least 8: S_b = max(1, ceil(n_b / (M ntl))), W_b their prefix sums;
  - otherwise in proportion to the blocks: W_b = b + floor((G - batch) C_{b-1} / T), S_b = W_{b+1} - W_b, with C
    the running block count and T the total (W_b = b when T = 0).
Cases cover both plans, the limit between them, the 64-sequence boundary (the larger batch plans from memory
rather than from registers), empty, negative, clamped and full lengths, and three kernels' granules.
"""
import numpy as np
import pytest
import torch

import rank_shared_kv_amd as lk

pytestmark = pytest.mark.gpu

from gpu_harness import say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _blocks(lens, max_len, L_cap, append):
    out = []
    for L in lens:
        L = int(L)
        if append and 0 <= L < L_cap:
            L += 1
        out.append((min(max(L, 0), max_len) + 31) // 32)
    return out


def _expected(lens, max_len, L_cap, append, G, granule):
    nb = _blocks(lens, max_len, L_cap, append)
    B, ntl = len(nb), max(1, granule // 32)
    splits = lambda per: [max(1, -(-n // per)) for n in nb]
    M = 1
    while sum(splits(M * ntl)) > G:
        M += 1
    if B <= 64 and M >= 8:
        S = splits(M * ntl)
        W = [sum(S[:b]) for b in range(B)]
        return W, S, "fewest"
    T, extra = sum(nb), G - B
    first = lambda b: b + (extra * sum(nb[:b])) // T if T else b
    W = [first(b) for b in range(B)]
    S = [first(b + 1) - first(b) for b in range(B)]
    return W, S, "proportional"


def _device_plan(dims, lens, max_len, append):
    sl = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    W = torch.full((len(lens),), -7, dtype=torch.int32, device="cuda")
    S = torch.full((len(lens),), -7, dtype=torch.int32, device="cuda")
    lk.lrkv_decode_split_plan(dims, max_len, sl, append, W, S)
    torch.cuda.synchronize()
    return W.cpu().tolist(), S.cpu().tolist()


def _check(dims, lens, max_len, append, want_kind=None):
    G, granule = lk.lrkv_decode_num_splits(dims, max_len)
    W, S = _device_plan(dims, lens, max_len, append)
    eW, eS, kind = _expected(lens, max_len, dims.L_cap, append, G, granule)
    say(f"  batch {len(lens)} G {G} granule {granule} append {append}: {kind}, {sum(S)} workgroups with splits")
    assert W == eW and S == eS
    assert W[0] == 0 and all(s >= 1 for s in S) and sum(S) <= G
    assert all(W[b + 1] == W[b] + S[b] for b in range(len(lens) - 1))
    if want_kind is not None:
        assert kind == want_kind
    return kind


SHAPES = {  # (batch-independent) H, d_h, r, dtype: the bf16 and fp32 matrix-core kernels and the general kernel
    "bf16_h32_r64": (32, 128, 64, lk.LRKV_BF16),
    "bf16_h16_r48": (16, 128, 48, lk.LRKV_BF16),
    "f32_h32_r0": (32, 128, 0, lk.LRKV_F32),
    "f32_h8_r16": (8, 64, 16, lk.LRKV_F32),
}


@pytest.mark.parametrize("append", [0, 1])
def test_long_context_plan(append):
    """4 x 32768 rows, 256 workgroups of two row lanes: with the appended row (1025 blocks) the fewest-splits plan
    gives 57 splits of at most 9 blocks a lane; without it, 64 splits of 8 (the proportional plan's split)."""
    H, d_h, r, dt = SHAPES["bf16_h32_r64"]
    dims = lk.make_dims(4, H, d_h, r, 32832, dt)
    say(f"[case] long-context plan, append {append}")
    lens = [32768] * 4
    kind = _check(dims, lens, 32832 if append else 32768, append, want_kind="fewest")
    _, S = _device_plan(dims, lens, 32832 if append else 32768, append)
    assert S == ([57] * 4 if append else [64] * 4), (kind, S)


def test_short_lanes_take_the_proportional_plan():
    """16 x 8192 rows with H = 16 (four row lanes): the least cap is 4 or 5 blocks, so the plan is proportional."""
    H, d_h, r, dt = SHAPES["bf16_h16_r48"]
    dims = lk.make_dims(16, H, d_h, r, 8448, dt)
    say("[case] 16 x 8192 plan")
    for append in (0, 1):
        _check(dims, [8192] * 16, 8448, append, want_kind="proportional")


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("batch", [1, 7, 33, 64, 65, 200])
def test_ragged_plans(shape, batch):
    """Ragged lengths (a few empty, negative, past max_len or at L_cap) at batch sizes around the 64-sequence
    boundary, both plans, both append modes."""
    H, d_h, r, dt = SHAPES[shape]
    L_cap, max_len = 40000, 36000
    rng = np.random.default_rng(batch * 31 + len(shape))
    dims = lk.make_dims(batch, H, d_h, r, L_cap, dt)
    if not lk.lrkv_decode_num_splits(dims, max_len)[0]:
        pytest.skip("no kernel for this shape")
    say(f"[case] ragged plan {shape} batch {batch}")
    for kind_lens in ("long", "mixed", "short"):
        hi = {"long": 36000, "mixed": 20000, "short": 3000}[kind_lens]
        lens = rng.integers(1, hi, size=batch).astype(np.int32)
        if batch >= 7:
            lens[1], lens[3], lens[5] = 0, -1, L_cap
            lens[6] = max_len + 100  # clamped to max_len
        for append in (0, 1):
            _check(dims, lens.tolist(), max_len, append)


def test_all_empty_and_tiny():
    """An all-empty batch (every sequence one workgroup) and single-block sequences."""
    H, d_h, r, dt = SHAPES["bf16_h32_r64"]
    dims = lk.make_dims(16, H, d_h, r, 4096, dt)
    say("[case] empty and one-block plans")
    _check(dims, [0] * 16, 4096, 0, want_kind="proportional")
    _check(dims, [1] * 16, 4096, 0)
    _check(dims, [0] * 16, 4096, 1)


def test_plan_limit_between_the_two():
    """Lengths around the cap of 8 blocks a lane: the device takes the same side as the rule."""
    H, d_h, r, dt = SHAPES["bf16_h32_r64"]
    dims = lk.make_dims(4, H, d_h, r, 48000, dt)
    G, granule = lk.lrkv_decode_num_splits(dims, 45000)
    ntl = granule // 32
    say(f"[case] plan limit, G {G}, {ntl} lanes")
    kinds = set()
    for n_blocks in range(G * ntl * 6 // 4, G * ntl * 10 // 4, 7):  # about 6 to 10 blocks a lane
        kinds.add(_check(dims, [n_blocks * 32] * 4, 45000, 0))
    assert kinds == {"fewest", "proportional"}
