"""Rank padded to an aligned width on the GPU ("Low-Rank Key Value Attention | What a shared cache can preserve",
sec. 4: a rank of 55 padded to a physical width of 64 for an alignment-constrained kernel, which moves the
payload fraction to 55.56%; that figure is pinned in test_abi_host.py).  Padding appends zero latent
coordinates and zero basis columns, so the padded cache decodes to the unpadded result: the padded problem
(r = 64) runs on the matrix-core kernel, the unpadded one (r = 55) on the general kernel, and both are compared
with the reference at r = 55.  Metric and tolerances as in test_gpu_decode.py."""
import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, cache_of, dims_of, gpu_decode, say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


def _pad_last(t, width):
    out = torch.zeros(tuple(t.shape[:-1]) + (width,), dtype=t.dtype, device=t.device)
    out[..., :t.shape[-1]] = t
    return out


@pytest.mark.parametrize("r,r_pad,H,d_h", [(55, 64, 32, 128), (12, 16, 8, 64), (40, 48, 16, 128)])
def test_padded_rank_decodes_to_unpadded_result(r, r_pad, H, d_h):
    lens = np.array([700, 300, 1], dtype=np.int32)
    w = synth.WORKLOADS["small_bf16"].with_(name="padding", batch=3, H=H, d_h=d_h, r=r, dtype="bf16", L=700,
                                            L_cap=768, ragged_lo=None)
    say(f"[case] rank {r} padded to {r_pad}, H={H} d_h={d_h}")
    dev = sdev.fill_layer(w, 0, lengths=lens)
    got = gpu_decode(w, dev, 700).cpu().numpy()  # r = 55: general kernel

    wp = w.with_(r=r_pad)
    devp = dict(dev)
    for name in ("z_k", "z_v", "B_k", "B_v"):
        devp[name] = _pad_last(dev[name], r_pad)
    # the unpadded shape runs the general kernel (32-row granule), the padded one a matrix-core kernel
    assert lk.lrkv_decode_num_splits(dims_of(w), 700)[1] == 32
    assert lk.lrkv_decode_num_splits(dims_of(wp), 700)[1] in (64, 128)
    got_p = gpu_decode(wp, devp, 700).cpu().numpy()

    host = synth.gen_host(w, 0, lengths=lens)
    ref = oracle.lrkv_decode("bf16", host["q"], host["k_shared"], host["v_shared"], host["z_k"], host["z_v"],
                             host["B_k"], host["B_v"], lens).reshape(3, H, d_h)
    for label, g in (("unpadded", got), ("padded", got_p)):
        err = oracle.relative_error(g.reshape(-1, d_h), ref.reshape(-1, d_h))
        say(f"  {label}: max rel err {err:.3e} (tol {TOL['bf16']:.0e})")
        assert err <= TOL["bf16"]
    # the physical payload of the padded layout, counted as the pages count it
    ratio = lk.lrkv_cache_bytes(dims_of(wp), lens.tolist()) / lk.lrkv_cache_bytes(dims_of(w), lens.tolist())
    assert abs(ratio - (d_h + H * r_pad) / (d_h + H * r)) < 1e-12
