"""lrkv_decode_noalloc (the decode entry point that allocates nothing) against lrkv_decode.

Two calls in a row through the C ABI on one device, the second with a smaller problem, so the second reads
only records its own split pass wrote into the shared device scratch.  Each output must equal lrkv_decode's
on the same inputs bit for bit (same kernels, same plan; lrkv_decode is itself held to the reference within
2e-3 for bf16 and 1e-5 for fp32 by the other GPU tests), and the first call's output is also compared with
the fp64 reference on sampled (sequence, head) pairs.
"""
import numpy as np
import pytest
import torch

import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import cache_of, compare, dims_of, gpu_decode, oracle_pairs, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _noalloc(w, dev, max_len, L_cap, stream=None):
    dims = dims_of(w, L_cap)
    p = torch.empty((w.batch, w.H, max(w.r, 1)), dtype=torch.float32, device="cuda")
    out = torch.full((w.batch, w.H, w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    if w.r > 0:
        lk.lrkv_absorb_query(dims, dev["q"], dev["B_k"], p, stream)
    lk.lrkv_decode_noalloc(dims, cache_of(dev, w.r), max_len, dev["q"], p if w.r > 0 else None,
                           dev["B_v"] if w.r > 0 else None, out, stream)
    torch.cuda.synchronize()
    return out


CASES = [
    # (label, workload, first (batch, lengths, L_cap), second (batch, lengths, L_cap))
    ("long_context_bf16", "long_context", (4, [32768, 32768, 32768, 32768], 32768), (2, [3000, 17], 3072)),
    ("ragged_bf16", "ragged", (16, list(range(700, 16700, 1000)), 16704), (3, [1, 33, 640], 640)),
    ("mqa_fp32", "ragged_mqa_fp32", (8, [9000, 512, 4096, 1, 0, 7777, 300, 64], 9024), (2, [100, 31], 128)),
    ("tiny_fp32", "tiny_fp32", (1, [64], 64), (1, [5], 64)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_decode_twice(case):
    label, name, first, second = case
    base = synth.WORKLOADS[name]
    for call, (batch, lens, L_cap) in enumerate((first, second)):
        w = base.with_(name=f"{label}_{call}", batch=batch, L=max(lens), L_cap=L_cap, ragged_lo=None)
        lens = np.array(lens, dtype=np.int32)
        max_len = int(lens.max())
        G, chunk = lk.lrkv_decode_num_splits(dims_of(w, L_cap), max_len)
        need = lk.lrkv_decode_workspace_bytes(dims_of(w, L_cap), max_len)
        say(f"[case] noalloc {label} call {call}: B={batch} H={w.H} d_h={w.d_h} r={w.r} {w.dtype} "
            f"lens[:6]={lens[:6].tolist()} G={G} records {need} B (scratch {lk.lrkv_decode_noalloc_max_bytes()} B)")
        assert 0 < need <= lk.lrkv_decode_noalloc_max_bytes()
        dev = sdev.fill_layer(w, 0, L_cap=L_cap, lengths=lens)
        got = _noalloc(w, dev, max_len, L_cap)
        ref_gpu = gpu_decode(w, dev, max_len, L_cap=L_cap)
        assert torch.equal(got, ref_gpu), f"{label} call {call}: differs from lrkv_decode"
        if call == 0:
            bs = sorted({0, batch // 2, batch - 1})
            pairs = [(b, h) for b in bs if lens[b] > 0 for h in sorted({0, w.H // 2, w.H - 1})]
            compare(w, got, oracle_pairs(w, 0, lens, pairs, mqa=(w.r == 0)), pairs, f"noalloc {label}")
        del dev


def test_noalloc_on_a_side_stream_and_empty_batch():
    """A non-default stream (the scratch of the stream's device), then a batch with no live rows (out = 0)."""
    w = synth.WORKLOADS["small_bf16"].with_(batch=3, L=500, L_cap=512)
    lens = np.array([500, 0, 77], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=512, lengths=lens)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = _noalloc(w, dev, 500, 512, stream=s)
    assert torch.equal(got, gpu_decode(w, dev, 500, L_cap=512))
    assert torch.count_nonzero(got[1]) == 0
    dev["seq_lens"].zero_()
    got0 = _noalloc(w, dev, 0, 512)
    assert torch.count_nonzero(got0) == 0
