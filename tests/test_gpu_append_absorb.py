"""lrkv_append_absorb (a decode step's append and query absorption in one launch) against the two separate
calls, lrkv_cache_append then lrkv_absorb_query, through the C ABI: the cache rows, the lengths and p must be
bit for bit the same.  The separate calls are themselves checked against the reference in test_gpu_decode.py
and test_gpu_layer.py; here the fused launch must not change a bit.  Shapes cover the fused vector path (bf16
and fp32), a shape outside it that runs the two kernels (r = 12 in bf16), r = 0 (the append alone) and a
sequence that is already full."""
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


CASES = [  # (dtype, batch, H, d_h, r, lengths, L_cap)
    ("bf16", 4, 32, 128, 64, [700, 33, 0, 95], 768),
    ("bf16", 3, 16, 128, 48, [64, 1, 200], 256),
    ("f32", 2, 4, 16, 4, [10, 63], 64),
    ("bf16", 2, 8, 64, 12, [5, 40], 64),        # r = 12: outside the vector path, two launches
    ("bf16", 2, 8, 64, 0, [5, 40], 64),         # r = 0: the append alone
    ("bf16", 3, 8, 64, 16, [64, 10, 63], 64),   # sequence 0 is full: nothing written, length unchanged
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_B{c[1]}_H{c[2]}_d{c[3]}_r{c[4]}")
def test_append_absorb_equals_separate_calls(case):
    dtype, B, H, d_h, r, lens, L_cap = case
    say(f"[case] append+absorb {case}")
    w = synth.WORKLOADS["small_bf16"].with_(name="append_absorb", batch=B, H=H, d_h=d_h, r=r, dtype=dtype,
                                            L=max(lens), L_cap=L_cap, ragged_lo=None)
    lens = np.array(lens, dtype=np.int32)
    runs = []
    for fused in (False, True):
        dev = sdev.fill_layer(w, 0, lengths=lens)
        rows = sdev.new_rows(w)
        dims = dims_of(w)
        cache = cache_of(dev, r)
        p = torch.full((B, H, max(r, 1)), float("nan"), dtype=torch.float32, device="cuda")
        zk, zv = (rows["zk_new"], rows["zv_new"]) if r else (None, None)
        bk = dev["B_k"] if r else None
        pp = p if r else None
        for _ in range(2):  # two steps in a row
            if fused:
                lk.lrkv_append_absorb(dims, cache, rows["k_new"], rows["v_new"], zk, zv, dev["q"], bk, pp)
            else:
                lk.lrkv_cache_append(dims, cache, rows["k_new"], rows["v_new"], zk, zv)
                lk.lrkv_absorb_query(dims, dev["q"], bk, pp)
        torch.cuda.synchronize()
        runs.append({k: dev[k].clone() for k in ("k_shared", "v_shared", "z_k", "z_v", "seq_lens") if k in dev}
                    | {"p": p.clone()})
    want = np.minimum(lens + 2, L_cap)
    want[lens >= L_cap] = lens[lens >= L_cap]
    assert runs[1]["seq_lens"].cpu().numpy().tolist() == want.tolist()
    for k in runs[0]:
        a, b = runs[0][k], runs[1][k]
        same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
        assert same, f"{k} differs between the fused launch and the separate calls"
