"""Host-side checks of the C ABI (no GPU needed; no kernel is launched).

* the shared library loads and exports every function include/lrkv.h declares;
* lrkv_cache_bytes reproduces the cache accounting printed on the pages;
* argument checks reject bad calls before any HIP call;
* the split plan and workspace size are consistent host arithmetic.
"""
import json
import math
import os
import re

import pytest

import rank_shared_kv_amd as lk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "lrkv.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*[A-Za-z_][\w \*]*?[\s\*](lrkv_\w+)\s*\(", header, re.M))
    assert declared, "no declarations parsed from include/lrkv.h"
    L = lk.lib()
    for name in sorted(declared):
        assert hasattr(L, name), f"{name} declared in lrkv.h but not exported"
    assert declared == set(lk.EXPORTED)


def _bytes(H, d_h, r, L, dtype=lk.LRKV_BF16, batch=1, lens=None):
    dims = lk.make_dims(batch, H, d_h, r, max(1, L), dtype)
    return lk.lrkv_cache_bytes(dims, lens)


def _mha_bytes(H, d_h, L, s=2, batch=1):
    # MHA payload per token and layer is 2 H d_h elements (reading notes, sec. 1 cache table)
    return 2 * s * batch * L * H * d_h


def test_cache_fraction_table():
    g = _golden("cache_accounting.json")
    for row in g["table7_fractions_percent"]:
        frac = _bytes(row["H"], row["d_h"], row["r"], 2048) / _mha_bytes(row["H"], row["d_h"], 2048)
        assert abs(100 * frac - row["percent"]) < 0.005 + 1e-9, row
    for row in g["rank_sweep_percent"]:
        frac = _bytes(6, 128, row["r"], 2048) / _mha_bytes(6, 128, 2048)
        assert abs(100 * frac - row["percent"]) < 0.05 + 1e-9, row


def test_elements_per_token_example():
    e = _golden("cache_accounting.json")["elements_example"]
    lrkv_elems = _bytes(e["H"], e["d_h"], e["r"], 1) // 2  # bf16: 2 bytes per element
    assert lrkv_elems == e["lrkv"]
    assert 2 * e["H"] * e["d_h"] == e["mha"]
    assert abs(100 * lrkv_elems / e["mha"] - e["kept_percent"]) < 0.005
    assert abs(100 - 100 * lrkv_elems / e["mha"] - e["saved_percent"]) < 0.005


def test_layout_example_bytes():
    x = _golden("cache_accounting.json")["layout_example"]
    per_layer = _bytes(x["H"], x["d_h"], x["r"], x["tokens"])
    total = x["layers"] * per_layer
    assert x["layers"] * _mha_bytes(x["H"], x["d_h"], x["tokens"]) == x["mha_bytes"]
    assert x["mha_bytes"] / 2**20 == x["mha_mib"]
    assert total / 2**20 == x["lrkv_mib"]
    assert x["layers"] * _bytes(x["H"], x["d_h"], x["r"], x["tokens_long"]) / 2**20 == x["lrkv_mib_long"]
    assert x["layers"] * _mha_bytes(x["H"], x["d_h"], x["tokens_long"]) / 2**20 == x["mha_mib_long"]


def test_rank_ceiling_and_padding():
    g = _golden("cache_accounting.json")
    for key in ("rank_ceiling", "gqa6_parity"):
        c = g[key]
        H, d_h, cap = c["H"], c["d_h"], c["c"]
        frac = lambda r: _bytes(H, d_h, r, 64) / _mha_bytes(H, d_h, 64)
        assert frac(c["r_max"]) <= cap + 1e-12 < frac(c["r_max"] + 1), key
    p = g["padded"]
    assert abs(100 * _bytes(p["H"], p["d_h"], p["r"], 64) / _mha_bytes(p["H"], p["d_h"], 64) - p["percent"]) < 0.005


def test_tensor_parallel_replication():
    t = _golden("cache_accounting.json")["tp_replicated"]
    H, d_h, r, P = t["H"], t["d_h"], t["r"], t["P"]
    single = _bytes(H, d_h, r, 64)
    shared_only = _bytes(H, d_h, 0, 64)  # r = 0 leaves only the shared block
    replicated = single + (P - 1) * shared_only
    mha = _mha_bytes(H, d_h, 64)
    assert abs(100 * single / mha - t["single_percent"]) < 0.05
    assert abs(100 * replicated / mha - t["replicated_percent"]) < 0.05


def test_full_rank_and_break_even():
    for H in (4, 6, 18, 32):
        d_h = 128
        assert _bytes(H, d_h, d_h, 64) / _mha_bytes(H, d_h, 64) == pytest.approx(1 + 1 / H, rel=1e-12)
        r_star = d_h * (1 - 1 / H)
        for r in range(0, d_h + 1):
            saves = _bytes(H, d_h, r, 64) < _mha_bytes(H, d_h, 64)
            assert saves == (r < r_star), (H, r)


def test_cache_bytes_ragged_and_dtype():
    dims = lk.make_dims(3, 4, 16, 2, 100, lk.LRKV_F32)
    assert lk.lrkv_cache_bytes(dims, [10, 0, 50]) == 2 * 4 * 60 * (16 + 4 * 2)
    assert lk.lrkv_cache_bytes(dims, [-5, 200, 1]) == 2 * 4 * (0 + 100 + 1) * (16 + 8)
    assert lk.lrkv_cache_bytes(dims) == 2 * 4 * 300 * 24
    bad = lk.make_dims(0, 4, 16, 2, 100, lk.LRKV_F32)
    assert lk.lrkv_cache_bytes(bad) == 0


# ---- argument checks: each call must fail on the host before any HIP call ----

A = 1 << 20  # a fake 16-byte-aligned device address; never dereferenced on these paths


def _dims():
    return lk.make_dims(2, 8, 64, 8, 256, lk.LRKV_BF16)


def _status(fn, *args):
    try:
        fn(*args)
    except lk.LrkvError as e:
        return e.status
    return lk.LRKV_OK


def test_invalid_dims_rejected():
    for bad in [lk.make_dims(0, 8, 64, 8, 256, 1), lk.make_dims(2, 0, 64, 8, 256, 1), lk.make_dims(2, 8, 0, 8, 256, 1),
                lk.make_dims(2, 8, 64, -1, 256, 1), lk.make_dims(2, 8, 64, 8, 0, 1), lk.make_dims(2, 8, 64, 8, 256, 7)]:
        cache = lk.Cache(A, A, A, A, A)
        assert _status(lk.lrkv_absorb_query, bad, A, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
        assert _status(lk.lrkv_cache_append, bad, cache, A, A, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
        assert _status(lk.lrkv_decode, bad, cache, 10, A, A, A, A, A, 1 << 30, 0) == lk.LRKV_ERR_INVALID_ARG
        assert lk.lrkv_decode_workspace_bytes(bad, 10) == 0


def test_null_and_misaligned_pointers_rejected():
    d = _dims()
    ws = lk.lrkv_decode_workspace_bytes(d, 256)
    good = lk.Cache(A, A, A, A, A)
    for field in ("k_shared", "v_shared", "z_k", "z_v", "seq_lens"):
        for badval in (None, A + 2):
            c = lk.Cache(A, A, A, A, A)
            setattr(c, field, badval)
            assert _status(lk.lrkv_decode, d, c, 256, A, A, A, A, 1 << 12, ws, 0) == lk.LRKV_ERR_INVALID_ARG, field
            assert _status(lk.lrkv_cache_append, d, c, A, A, A, A, 0) == lk.LRKV_ERR_INVALID_ARG, field
    for i in range(4):  # q, p, B_v, out
        args = [A, A, A, A]
        args[i] = None
        assert _status(lk.lrkv_decode, d, good, 256, *args, 1 << 12, ws, 0) == lk.LRKV_ERR_INVALID_ARG, i
    assert _status(lk.lrkv_absorb_query, d, None, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_absorb_query, d, A, A, A + 4, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_cache_append, d, good, A, None, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_merge, d, None, 256, A, A, 1 << 12, ws, 0) == lk.LRKV_ERR_INVALID_ARG
    for i in range(7):  # k_new, v_new, zk_new, zv_new, q, B_k, p of the fused append + absorb
        args = [A] * 7
        args[i] = None
        assert _status(lk.lrkv_append_absorb, d, good, *args, 0) == lk.LRKV_ERR_INVALID_ARG, i


def test_max_len_and_workspace_rejected():
    d = _dims()
    c = lk.Cache(A, A, A, A, A)
    need = lk.lrkv_decode_workspace_bytes(d, 256)
    assert need > 0
    assert _status(lk.lrkv_decode, d, c, 257, A, A, A, A, 1 << 12, need, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode, d, c, -1, A, A, A, A, 1 << 12, need, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode, d, c, 256, A, A, A, A, 1 << 12, need - 1, 0) == lk.LRKV_ERR_WORKSPACE
    assert _status(lk.lrkv_decode, d, c, 256, A, A, A, A, None, need, 0) == lk.LRKV_ERR_WORKSPACE
    assert _status(lk.lrkv_decode, d, c, 256, A, A, A, A, (1 << 12) + 16, need, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_partial, d, c, 256, A, A, 1 << 12, need - 4, 0) == lk.LRKV_ERR_WORKSPACE


def test_split_plan_entry_checks_before_any_launch():
    """lrkv_decode_split_plan rejects invalid dims, max_len outside [0, L_cap], an append flag other than 0 or 1
    and NULL pointers before anything is enqueued; with max_len 0 there is nothing to plan (no launch)."""
    d = _dims()
    bad = lk.make_dims(0, 8, 64, 8, 256, 1)
    assert _status(lk.lrkv_decode_split_plan, bad, 10, A, 0, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_split_plan, d, 257, A, 0, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_split_plan, d, -1, A, 0, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_split_plan, d, 256, A, 2, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    for i in range(3):  # seq_lens, first_wg, splits
        args = [A, A, A]
        args[i] = None
        assert _status(lk.lrkv_decode_split_plan, d, 256, args[0], 1, args[1], args[2], 0) == lk.LRKV_ERR_INVALID_ARG, i
    assert _status(lk.lrkv_decode_split_plan, d, 0, A, 0, A, A, 0) == lk.LRKV_OK


def test_noalloc_checks_before_any_launch():
    """lrkv_decode_noalloc: the same argument checks as lrkv_decode, and a problem whose split records exceed
    its device scratch is rejected with LRKV_ERR_WORKSPACE before anything is enqueued."""
    cap = lk.lrkv_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    d = _dims()
    c = lk.Cache(A, A, A, A, A)
    assert _status(lk.lrkv_decode_noalloc, d, c, 257, A, A, A, A, 0) == lk.LRKV_ERR_INVALID_ARG
    for i in range(4):  # q, p, B_v, out
        args = [A, A, A, A]
        args[i] = None
        assert _status(lk.lrkv_decode_noalloc, d, c, 256, *args, 0) == lk.LRKV_ERR_INVALID_ARG, i
    big = lk.make_dims(8, 32, 128, 128, 65536, lk.LRKV_F32)  # general kernel, 1024 splits of 260-float records
    need = lk.lrkv_decode_workspace_bytes(big, 65536)
    assert need > cap
    assert _status(lk.lrkv_decode_noalloc, big, c, 65536, A, A, A, A, 0) == lk.LRKV_ERR_WORKSPACE
    assert "scratch" in lk.lib().lrkv_last_error().decode()


def test_decode_step_layout_and_fusion():
    """lrkv_decode_step: the workspace holds the split records (lrkv_decode_workspace_bytes, rounded up to 256
    bytes), then the counter words (4 header words and two per sequence); the step runs as one launch on the bf16
    matrix-core shapes whose merge workgroups fit one resident round, as a split pass that appends plus the merge
    on the fp32 rank-0 shapes, as the two calls elsewhere; its argument checks run before any launch."""
    for (B, H, d_h, r, L, dt, fused) in [(4, 32, 128, 64, 32768, 1, True), (16, 16, 128, 48, 8192, 1, True),
                                         (4, 18, 128, 55, 8192, 1, False),   # r = 55: the absorb's scalar path
                                         (64, 32, 128, 32, 32768, 1, False),  # 2048 merge workgroups
                                         (32, 16, 128, 32, 2528, 1, True), (2, 8, 64, 0, 64, 1, True),
                                         (64, 32, 128, 0, 32768, 0, True), (4, 32, 128, 0, 32768, 0, True),
                                         (64, 32, 128, 8, 32768, 0, False),  # fp32, r > 0: the general kernel
                                         (2, 8, 64, 12, 64, 1, False)]:
        d = lk.make_dims(B, H, d_h, r, L, dt)
        rec = lk.lrkv_decode_workspace_bytes(d, L)
        off = lk.lrkv_decode_step_sync_offset(d, L)
        total = lk.lrkv_decode_step_workspace_bytes(d, L)
        assert off == (rec + 255) // 256 * 256
        assert total == off + ((4 + 2 * B) * 4 + 255) // 256 * 256
        assert lk.lrkv_decode_step_fused(d, L) == fused, (B, H, d_h, r, dt)
    d = _dims()
    c = lk.Cache(A, A, A, A, A)
    need = lk.lrkv_decode_step_workspace_bytes(d, 256)
    good = [A] * 10
    assert _status(lk.lrkv_decode_step, d, c, 257, *good, need, 0) == lk.LRKV_ERR_INVALID_ARG  # max_len > L_cap
    for i in range(9):  # k_new, v_new, zk_new, zv_new, q, B_k, B_v, p, out
        args = list(good)
        args[i] = None
        assert _status(lk.lrkv_decode_step, d, c, 256, *args, need, 0) == lk.LRKV_ERR_INVALID_ARG, i
    assert _status(lk.lrkv_decode_step, d, c, 256, *good[:9], None, need, 0) == lk.LRKV_ERR_WORKSPACE
    assert _status(lk.lrkv_decode_step, d, c, 256, *good[:9], A + 64, need, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_decode_step, d, c, 256, *good, need - 4, 0) == lk.LRKV_ERR_WORKSPACE


def test_latent_layout_conversion_checks():
    d = _dims()
    n = 2 * 8 * 256 * 8 * 2  # bytes of one latent tensor
    assert _status(lk.lrkv_latents_to_token_major, d, None, A, 0) == lk.LRKV_ERR_INVALID_ARG
    assert _status(lk.lrkv_latents_to_token_major, d, A, A + n - 16, 0) == lk.LRKV_ERR_INVALID_ARG  # overlap
    assert _status(lk.lrkv_latents_to_token_major, d, A, A + 8, 0) == lk.LRKV_ERR_INVALID_ARG       # misaligned
    lk.lrkv_latents_to_token_major(lk.make_dims(2, 8, 64, 0, 256, lk.LRKV_BF16), None, None, 0)   # r = 0: no-op


def test_unsupported_shape_rejected():
    d = lk.make_dims(1, 4, 300, 4, 64, lk.LRKV_F32)  # d_h beyond every kernel
    c = lk.Cache(A, A, A, A, A)
    assert _status(lk.lrkv_decode, d, c, 64, A, A, A, A, 1 << 12, 1 << 20, 0) == lk.LRKV_ERR_UNSUPPORTED
    assert lk.lrkv_decode_workspace_bytes(d, 64) == 0


def test_r0_needs_no_latents():
    d = lk.make_dims(2, 8, 64, 0, 256, lk.LRKV_F32)
    # absorb is a no-op for r == 0 and touches nothing
    lk.lrkv_absorb_query(d, None, None, None, 0)


def test_split_plan_arithmetic():
    for (B, H, d_h, r, L, dt) in [(1, 4, 16, 4, 64, 0), (8, 8, 64, 8, 2048, 1), (16, 16, 128, 48, 8192, 1),
                                  (4, 32, 128, 64, 32768, 1), (64, 32, 128, 32, 32768, 1), (64, 32, 128, 0, 32768, 0)]:
        d = lk.make_dims(B, H, d_h, r, L, dt)
        G, chunk = lk.lrkv_decode_num_splits(d, L)
        # G workgroups for the whole batch: at least one per sequence, at most one per tile of every sequence
        assert B <= G <= B * math.ceil(L / chunk) and chunk % 32 == 0 and G <= B + 8192
        rec = ((d_h + r + 2) + 3) // 4 * 4
        assert lk.lrkv_decode_workspace_bytes(d, L) == 4 * G * H * rec
        # within a kernel the plan depends on the shape and max_len, not on the rank
        if dt == 1 or r == 0:
            assert lk.lrkv_decode_num_splits(lk.make_dims(B, H, d_h, 0, L, dt), L) == (G, chunk)
    # one resident round of workgroups on the 256 CUs for the long-context shape
    assert lk.lrkv_decode_num_splits(lk.make_dims(4, 32, 128, 64, 33024, 1), 32818) == (256, 64)
    # short contexts: never more workgroups than tiles
    assert lk.lrkv_decode_num_splits(lk.make_dims(4, 32, 128, 64, 256, 1), 64) == (4, 64)
    d = lk.make_dims(2, 8, 64, 8, 256, 1)
    assert lk.lrkv_decode_num_splits(d, 0) == (0, 0)
    assert lk.lrkv_decode_workspace_bytes(d, 0) == 0


def test_multi_query_plan_arithmetic(monkeypatch):
    """Multi-token decode plans virtual sequences of qw query tokens each (ceil(Q / qw) per sequence): qw = 2
    (Q = 2) or 4 (Q >= 3, but 2 at d_h = 128 and r = 64) on the bf16 matrix-core shapes, one workgroup per SIMD,
    so G is the single-token plan's G of the virtual batch capped at 256; qw = 1 elsewhere (the single-token
    plan of batch * Q virtual sequences).  Workspace: G * qw * H records, then the virtual lengths, each part
    256-byte aligned."""
    al = lambda n: (n + 255) // 256 * 256
    rec = lambda d_h, r: 4 * ((d_h + r + 2 + 3) // 4 * 4)
    monkeypatch.delenv("LRKV_MULTI_QW", raising=False)
    for (B, H, d_h, r, L, dt, Q, qw) in [(4, 32, 128, 64, 33024, 1, 4, 2), (4, 32, 128, 64, 33024, 1, 16, 2),
                                         (4, 16, 128, 48, 8192, 1, 4, 4), (4, 32, 64, 64, 4096, 1, 7, 4),
                                         (2, 16, 128, 32, 4096, 1, 2, 2), (64, 32, 128, 32, 33024, 1, 3, 4),
                                         (2, 8, 64, 16, 256, 1, 5, 4), (2, 4, 16, 4, 128, 0, 3, 1),
                                         (3, 8, 64, 16, 512, 1, 1, 1)]:
        d = lk.make_dims(B, H, d_h, r, L, dt)
        nv = B * -(-Q // qw)
        dq = lk.make_dims(nv, H, d_h, r, L, dt)
        if qw == 1:
            want = al(lk.lrkv_decode_workspace_bytes(dq, L)) + al(4 * nv)
        else:
            G = min(lk.lrkv_decode_num_splits(dq, L)[0], 256)
            want = al(G * qw * H * rec(d_h, r)) + al(4 * nv)
        assert lk.lrkv_decode_multi_workspace_bytes(d, Q, L) == want, (B, H, d_h, r, Q)
    # the override selects one token per workgroup (the single-token plan of batch * Q sequences); four tokens
    # are capped at two where they do not fit
    monkeypatch.setenv("LRKV_MULTI_QW", "1")
    d, dq = lk.make_dims(4, 32, 128, 64, 33024, 1), lk.make_dims(16, 32, 128, 64, 33024, 1)
    assert lk.lrkv_decode_multi_workspace_bytes(d, 4, 33024) == al(lk.lrkv_decode_workspace_bytes(dq, 33024)) + 256
    monkeypatch.setenv("LRKV_MULTI_QW", "4")
    assert lk.lrkv_decode_multi_workspace_bytes(d, 4, 33024) == al(256 * 2 * 32 * rec(128, 64)) + 256
    monkeypatch.delenv("LRKV_MULTI_QW")
    assert lk.lrkv_decode_multi_workspace_bytes(d, 0, 100) == 0
    assert lk.lrkv_decode_multi_workspace_bytes(d, 65, 100) == 0
    assert lk.lrkv_decode_multi_workspace_bytes(lk.make_dims(2048, 8, 64, 8, 256, 1), 64, 100) == 0  # > 65535


def test_rope_plan_arithmetic():
    """The rotary decode plans on its own: up to 256 workgroups (one eight-wave workgroup per CU) on the bf16
    matrix-core shapes, the general kernel's 1024 elsewhere; workspace = G * H * record floats."""
    d = lk.make_dims(4, 32, 128, 64, 33024, 1)
    rec = (128 + 64 + 2 + 3) // 4 * 4
    assert lk.lrkv_decode_rope_workspace_bytes(d, 32818) == 4 * 256 * 32 * rec
    # a short batch: at most one workgroup per 128-row tile of each sequence
    assert lk.lrkv_decode_rope_workspace_bytes(lk.make_dims(3, 8, 64, 16, 256, 1), 100) == 4 * 3 * 1 * 8 * 84
    assert lk.lrkv_decode_rope_workspace_bytes(lk.make_dims(3, 8, 64, 16, 256, 1), 129) == 4 * 3 * 2 * 8 * 84
    small = lk.make_dims(2, 4, 16, 4, 128, 0)
    G = lk.lrkv_decode_rope_workspace_bytes(small, 100) // (4 * 4 * ((16 + 4 + 2 + 3) // 4 * 4))
    assert G == 2 * math.ceil(100 / 32)  # one workgroup per 32-row tile of each sequence, the general kernel
    assert lk.lrkv_decode_rope_workspace_bytes(lk.make_dims(2, 4, 18, 4, 128, 0), 100) == 0  # d_h % 4 != 0
