"""Pins for the CPU reference: each check ties it to something other than itself.

Sources of truth used here:
  * worked examples printed on the pages (fixtures under tests/golden/, each cited);
  * the weight-space definition W_h = W_shared + U_h B_h^T evaluated by a
    different route (full per-head projections, then torch's
    scaled_dot_product_attention in float64);
  * special cases that reduce to textbook attention (r = 0 -> MQA, r = d_h with
    identity bases and zero shared part -> MHA), a single visible row, and
    invariances (token order, gauge of the factors);
  * the associativity identity (factored evaluation == rebuilt keys/values).

Every pin is a plain function taking the library path, so the last test can
run all of them against copies of the reference with a planted mistake and
check that each planted mistake is caught.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _rand(seed, shape, std=1.0):
    n = int(np.prod(shape))
    return synth.normal(seed, std, n, "f64").reshape(shape)


def _sdpa(q, k, v):
    """Textbook attention via torch (float64): q [B,H,d], k/v [B,H,L,d] -> [B,H,d]."""
    qt = torch.from_numpy(q)[:, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, torch.from_numpy(k), torch.from_numpy(v))
    return out[:, :, 0, :].numpy()


# ---------------------------------------------------------------------------------------------
# pins (each returns None on success and raises AssertionError on failure)
# ---------------------------------------------------------------------------------------------

def pin_worked_logits(lib_path=None):
    g = _golden("worked_logits.json")
    d, r = g["d_h"], g["r"]
    q = _f64(g["q"]).reshape(1, 1, d)
    k = _f64(g["k_shared"]).reshape(1, 2, d)
    v = _f64(np.eye(2, d)).reshape(1, 2, d)
    zk = _f64(g["z_k"]).reshape(1, 1, 2, r)
    zv = np.zeros((1, 1, 2, r))
    Bk = _f64(g["B_k"]).reshape(1, d, r)
    Bv = np.zeros((1, d, r))
    lens = np.array([2], dtype=np.int32)
    out, w = oracle.lrkv_decode("f64", q, k, v, zk, zv, Bk, Bv, lens, want_weights=True, lib_path=lib_path)
    np.testing.assert_allclose(w[0], g["summed_weights"], rtol=0, atol=1e-15)
    # the shared branch alone (private latents zero) puts weight softmax(2, 0) on the first row
    _, w_sh = oracle.lrkv_decode("f64", q, k, v, np.zeros_like(zk), zv, Bk, Bv, lens, want_weights=True,
                                 lib_path=lib_path)
    a0 = 1.0 / (1.0 + math.exp(-g["shared_scaled_logits"][0] + g["shared_scaled_logits"][1]))
    np.testing.assert_allclose(w_sh[0], [a0, 1.0 - a0], rtol=0, atol=1e-15)


def pin_hand_score(lib_path=None):
    g = _golden("hand_calc_score.json")
    d, r = g["d_h"], g["r"]
    q = _f64(g["q"]).reshape(1, 1, d)
    k = _f64(g["k_shared"]).reshape(1, 2, d)
    zk = _f64(g["z_k"]).reshape(1, 1, 2, r)
    Bk = _f64(g["B_k"]).reshape(1, d, r)
    v = _f64([[1, 0], [0, 0]]).reshape(1, 2, d)
    zv = np.zeros((1, 1, 2, r))
    Bv = np.zeros((1, d, r))
    lens = np.array([2], dtype=np.int32)
    # the page's decomposition: materialised key and the two score parts
    key0 = k[0, 0] + zk[0, 0, 0] @ Bk[0].T
    np.testing.assert_array_equal(key0, g["materialised_key_row0"])
    assert float(q[0, 0] @ k[0, 0]) == g["shared_part_row0"]
    assert float((q[0, 0] @ Bk[0]) @ zk[0, 0, 0]) == g["private_part_row0"]
    raw = g["raw_score_row0"]
    a0 = 1.0 / (1.0 + math.exp(-raw / math.sqrt(d)))
    a1 = 1.0 / (1.0 + math.exp(raw / math.sqrt(d)))
    out, w = oracle.lrkv_decode("f64", q, k, v, zk, zv, Bk, Bv, lens, want_weights=True, lib_path=lib_path)
    np.testing.assert_allclose(w[0], [a0, a1], rtol=1e-13, atol=0)
    np.testing.assert_allclose(out[0], [a0, 0.0], rtol=1e-14, atol=1e-300)


def pin_hand_value(lib_path=None):
    g = _golden("hand_calc_value.json")
    d, r = g["d_h"], g["r"]
    q = _f64([math.sqrt(2.0) * math.log(3.0), 0.0]).reshape(1, 1, d)
    k = _f64([[0, 0], [1, 0]]).reshape(1, 2, d)
    v = np.zeros((1, 2, d))
    zk = np.zeros((1, 1, 2, r))
    Bk = np.zeros((1, d, r))
    zv = _f64(g["z_v"]).reshape(1, 1, 2, r)
    Bv = _f64(g["B_v"]).reshape(1, d, r)
    lens = np.array([2], dtype=np.int32)
    out, w = oracle.lrkv_decode("f64", q, k, v, zk, zv, Bk, Bv, lens, want_weights=True, lib_path=lib_path)
    np.testing.assert_allclose(w[0], g["weights"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(out[0], g["out"], rtol=1e-13, atol=0)


def _weight_space_case(seed, B, H, d_h, r, L, lens):
    """Random weights and activations; cache rows from them; reference by the full per-head projection."""
    d = H * d_h
    X = _rand(seed + 1, (B, L, d), 1.0 / math.sqrt(d))
    Wsk, Wsv = _rand(seed + 2, (d, d_h)), _rand(seed + 3, (d, d_h))
    Uk, Uv = _rand(seed + 4, (H, d, r)), _rand(seed + 5, (H, d, r))
    Bk, Bv = _rand(seed + 6, (H, d_h, r), 0.5), _rand(seed + 7, (H, d_h, r), 0.5)
    q = _rand(seed + 8, (B, H, d_h))
    # cache rows (reading notes sec. 2.3): shared rows x W_shared, latents x U_h
    k_s = X @ Wsk
    v_s = X @ Wsv
    z_k = np.einsum("bld,hdr->bhlr", X, Uk)
    z_v = np.einsum("bld,hdr->bhlr", X, Uv)
    # full per-head projections (Eqs. (2)-(5)): W_h = W_shared + U_h B_h^T
    Wk = Wsk[None] + np.einsum("hdr,hcr->hdc", Uk, Bk)
    Wv = Wsv[None] + np.einsum("hdr,hcr->hdc", Uv, Bv)
    K = np.einsum("bld,hdc->bhlc", X, Wk)
    V = np.einsum("bld,hdc->bhlc", X, Wv)
    ref = np.zeros((B, H, d_h))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        ref[b:b + 1] = _sdpa(q[b:b + 1], np.ascontiguousarray(K[b:b + 1, :, :n]),
                             np.ascontiguousarray(V[b:b + 1, :, :n]))
    return dict(q=q, k=k_s, v=v_s, zk=z_k, zv=z_v, Bk=Bk, Bv=Bv, lens=np.asarray(lens, np.int32)), ref


def pin_weight_space_route(lib_path=None):
    grid = [(1, 1, 2, 1, 3), (2, 3, 4, 2, 5), (1, 4, 8, 4, 8), (3, 2, 8, 3, 7), (2, 4, 6, 6, 4)]
    for i, (B, H, d_h, r, L) in enumerate(grid):
        lens = [L - (b % 2) for b in range(B)]
        case, ref = _weight_space_case(1000 + 17 * i, B, H, d_h, r, L, lens)
        got = oracle.lrkv_decode("f64", case["q"], case["k"], case["v"], case["zk"], case["zv"], case["Bk"],
                                 case["Bv"], case["lens"], lib_path=lib_path).reshape(B, H, d_h)
        err = oracle.relative_error(got, ref)
        assert err < 1e-12, (B, H, d_h, r, L, err)


def pin_mqa_special_case(lib_path=None):
    B, H, d_h, L = 2, 3, 8, 9
    q = _rand(201, (B, H, d_h))
    k = _rand(202, (B, L, d_h))
    v = _rand(203, (B, L, d_h))
    lens = np.array([L, L], dtype=np.int32)
    ref = _sdpa(q, np.ascontiguousarray(np.broadcast_to(k[:, None], (B, H, L, d_h))),
                np.ascontiguousarray(np.broadcast_to(v[:, None], (B, H, L, d_h))))
    got = oracle.mqa_decode("f64", q, k, v, lens, lib_path=lib_path).reshape(B, H, d_h)
    assert oracle.relative_error(got, ref) < 1e-13
    empty = np.zeros((B, H, L, 0))
    got0 = oracle.lrkv_decode("f64", q, k, v, empty, empty, np.zeros((H, d_h, 0)), np.zeros((H, d_h, 0)), lens,
                              lib_path=lib_path).reshape(B, H, d_h)
    assert oracle.relative_error(got0, ref) < 1e-13


def pin_mha_special_case(lib_path=None):
    # r = d_h, B^K_h = B^V_h = I, zero shared part: each head has its own keys z^K_h and values z^V_h
    B, H, d_h, L = 2, 3, 6, 7
    q = _rand(301, (B, H, d_h))
    zk = _rand(302, (B, H, L, d_h))
    zv = _rand(303, (B, H, L, d_h))
    eye = np.ascontiguousarray(np.broadcast_to(np.eye(d_h), (H, d_h, d_h)))
    zero = np.zeros((B, L, d_h))
    lens = np.array([L, L], dtype=np.int32)
    ref = _sdpa(q, zk, zv)
    got = oracle.lrkv_decode("f64", q, zero, zero, zk, zv, eye, eye, lens, lib_path=lib_path).reshape(B, H, d_h)
    assert oracle.relative_error(got, ref) < 1e-13


def pin_single_row(lib_path=None):
    # one visible row: softmax weight 1, so o_h = v_s0 + z^V_0 (B^V_h)^T for every head
    B, H, d_h, r, L_cap = 2, 3, 5, 2, 4
    q = _rand(401, (B, H, d_h))
    k, v = _rand(402, (B, L_cap, d_h)), _rand(403, (B, L_cap, d_h))
    zk, zv = _rand(404, (B, H, L_cap, r)), _rand(405, (B, H, L_cap, r))
    Bk, Bv = _rand(406, (H, d_h, r)), _rand(407, (H, d_h, r))
    lens = np.array([1, 1], dtype=np.int32)
    got = oracle.lrkv_decode("f64", q, k, v, zk, zv, Bk, Bv, lens, lib_path=lib_path).reshape(B, H, d_h)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(got[b, h], v[b, 0] + Bv[h] @ zv[b, h, 0], rtol=1e-14, atol=1e-14)


def _random_case(seed, B, H, d_h, r, L_cap, lens):
    return dict(q=_rand(seed, (B, H, d_h)), k=_rand(seed + 1, (B, L_cap, d_h)), v=_rand(seed + 2, (B, L_cap, d_h)),
                zk=_rand(seed + 3, (B, H, L_cap, r)), zv=_rand(seed + 4, (B, H, L_cap, r)),
                Bk=_rand(seed + 5, (H, d_h, r), 1 / math.sqrt(r)), Bv=_rand(seed + 6, (H, d_h, r), 1 / math.sqrt(r)),
                lens=np.asarray(lens, dtype=np.int32))


def _run(c, lib_path=None):
    return oracle.lrkv_decode("f64", c["q"], c["k"], c["v"], c["zk"], c["zv"], c["Bk"], c["Bv"], c["lens"],
                              lib_path=lib_path)


def pin_token_permutation(lib_path=None):
    B, H, d_h, r, L = 2, 3, 8, 3, 11
    c = _random_case(501, B, H, d_h, r, L, [L, L])
    base = _run(c, lib_path)
    perm = np.random.default_rng(5).permutation(L)
    c2 = dict(c, k=c["k"][:, perm], v=c["v"][:, perm], zk=c["zk"][:, :, perm], zv=c["zv"][:, :, perm])
    assert oracle.relative_error(_run(c2, lib_path), base.reshape(-1, d_h)) < 1e-13


def pin_gauge(lib_path=None):
    # U_h -> U_h C and B_h -> B_h C^{-T} leave U_h B_h^T unchanged (reading notes sec. 4.6);
    # on cached latents this is z -> z C, B -> B C^{-T}.
    B, H, d_h, r, L = 2, 2, 8, 3, 9
    c = _random_case(601, B, H, d_h, r, L, [L, L - 2])
    base = _run(c, lib_path)
    C = np.eye(r) + 0.3 * _rand(607, (r, r))
    CinvT = np.linalg.inv(C).T
    c2 = dict(c, zk=c["zk"] @ C, zv=c["zv"] @ C, Bk=c["Bk"] @ CinvT, Bv=c["Bv"] @ CinvT)
    assert oracle.relative_error(_run(c2, lib_path), base) < 1e-12


def pin_associativity(lib_path=None):
    for i, (B, H, d_h, r, L) in enumerate([(2, 3, 8, 3, 13), (1, 4, 16, 4, 64), (3, 2, 32, 8, 40)]):
        lens = [L - 3 * b for b in range(B)]
        c = _random_case(701 + 10 * i, B, H, d_h, r, L, lens)
        rec = _run(c, lib_path)
        fac = oracle.factored_decode("f64", c["q"], c["k"], c["v"], c["zk"], c["zv"], c["Bk"], c["Bv"], c["lens"],
                                     lib_path=lib_path)
        assert oracle.relative_error(fac, rec) < 1e-12


def pin_ragged_rows_ignored(lib_path=None):
    # rows at or beyond seq_lens[b] are never read; a sequence with no live rows gives 0
    B, H, d_h, r, L = 3, 2, 8, 2, 10
    c = _random_case(801, B, H, d_h, r, L, [10, 4, 0])
    base = _run(c, lib_path).reshape(B, H, d_h)
    assert np.all(base[2] == 0.0)
    c2 = dict(c)
    for key in ("k", "v"):
        a = c[key].copy()
        a[1, 4:] = 1e6
        c2[key] = a
    for key in ("zk", "zv"):
        a = c[key].copy()
        a[1, :, 4:] = -1e6
        c2[key] = a
    np.testing.assert_array_equal(_run(c2, lib_path).reshape(B, H, d_h), base)
    # and the live prefix alone, as its own cache, gives the same output
    c3 = _random_case(801, B, H, d_h, r, L, [10, 4, 0])
    c3 = dict(c3, k=c3["k"][1:2, :4], v=c3["v"][1:2, :4], zk=c3["zk"][1:2, :, :4], zv=c3["zv"][1:2, :, :4],
              q=c3["q"][1:2], lens=np.array([4], np.int32))
    np.testing.assert_allclose(_run(c3, lib_path).reshape(1, H, d_h)[0], base[1], rtol=1e-15, atol=0)


ALL_PINS = [pin_worked_logits, pin_hand_score, pin_hand_value, pin_weight_space_route, pin_mqa_special_case,
            pin_mha_special_case, pin_single_row, pin_token_permutation, pin_gauge, pin_associativity,
            pin_ragged_rows_ignored]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_absorb_query_pins():
    """The projected query: the review's hand calculation (q = (2, 1), reconstruction column (1, -1) give the
    projected coordinate 1), a one-hot query picks one row of the basis exactly, and the associativity step of
    Eq. (6): (q B^K) . z equals q . (z B^K^T) for random inputs."""
    g = _golden("hand_calc_score.json")
    p = oracle.absorb_query("f64", _f64(g["q"]).reshape(1, 1, 2), _f64(g["B_k"]).reshape(1, 2, 1))
    assert p.reshape(-1).tolist() == g["projected_query"]
    Bk = _rand(71, (3, 8, 5), 0.5)
    q = np.zeros((1, 3, 8))
    q[0, 1, 6] = 1.0
    np.testing.assert_array_equal(oracle.absorb_query("f64", q, Bk)[0, 1], Bk[1, 6])
    q = _rand(72, (2, 3, 8))
    z = _rand(73, (2, 3, 5))
    lhs = np.einsum("bhi,bhi->bh", oracle.absorb_query("f64", q, Bk), z)
    rhs = np.einsum("bhc,bhc->bh", q, np.einsum("bhi,hci->bhc", z, Bk))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    # bf16 inputs are widened exactly: a power-of-two basis times an integer query is exact
    qb = np.array([[[0x4000, 0x3F80]]], dtype=np.uint16)          # (2, 1) in bf16
    bb = np.array([[[0x3F80], [0xBF80]]], dtype=np.uint16)        # (1, -1) in bf16
    assert oracle.absorb_query("bf16", qb, bb).reshape(-1).tolist() == [1.0]


def test_r0_lrkv_equals_mqa_bitwise():
    """r = 0 reduces the rebuilt keys and values to the shared ones exactly (empty private sums)."""
    for dtype in ("f32", "bf16", "f64"):
        B, H, d_h, L = 2, 4, 16, 33
        gen = lambda s, shape: synth.normal(s, 1.0, int(np.prod(shape)), dtype).reshape(shape)
        q, k, v = gen(901, (B, H, d_h)), gen(902, (B, L, d_h)), gen(903, (B, L, d_h))
        empty = np.zeros((B, H, L, 0), dtype=q.dtype)
        eb = np.zeros((H, d_h, 0), dtype=q.dtype)
        lens = np.array([L, 17], dtype=np.int32)
        a = oracle.lrkv_decode(dtype, q, k, v, empty, empty, eb, eb, lens)
        m = oracle.mqa_decode(dtype, q, k, v, lens)
        assert np.array_equal(a.view(np.uint64), m.view(np.uint64))


def test_bf16_inputs_widen_exactly():
    """bf16 inputs are read as their exact fp32 values: same answer as passing the widened fp32 arrays."""
    w = synth.WORKLOADS["small_bf16"].with_(batch=2, L=40)
    x = synth.gen_host(w)
    pairs = [(0, 0), (1, 7)]
    a = oracle.lrkv_decode("bf16", x["q"], x["k_shared"], x["v_shared"], x["z_k"], x["z_v"], x["B_k"], x["B_v"],
                           x["seq_lens"], pairs=pairs)
    f = {k: synth.bf16_bits_to_f32(v) for k, v in x.items() if k != "seq_lens"}
    b = oracle.lrkv_decode("f32", f["q"], f["k_shared"], f["v_shared"], f["z_k"], f["z_v"], f["B_k"], f["B_v"],
                           x["seq_lens"], pairs=pairs)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("plant", [1, 2, 3, 4])
def test_planted_mistake_is_caught(plant, tmp_path):
    """A copy of the reference with one planted mistake must fail at least one pin."""
    path = str(tmp_path / f"liboracle_plant{plant}.so")
    oracle.build(force=True, plant=plant, out_path=path)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib_path=path)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {plant} slipped through every pin"


# ---------------------------------------------------------------------------------------------
# layer step around the attention core: projections in, output projection out
# ---------------------------------------------------------------------------------------------
from oracle import layer as olayer  # noqa: E402


def _layer_case(seed, B, H, d_h, r, dm, L_hist):
    g = lambda s, shape, std=1.0: _rand(seed + s, shape, std)
    n_in = H * d_h + 2 * d_h + 2 * H * r
    return {"B": B, "H": H, "d_h": d_h, "r": r, "dm": dm,
            "W_in": g(1, (n_in, dm), 1 / math.sqrt(dm)), "W_o": g(2, (dm, H * d_h), 1 / math.sqrt(H * d_h)),
            "B_k": g(3, (H, d_h, r), 1 / math.sqrt(max(r, 1))), "B_v": g(4, (H, d_h, r), 1 / math.sqrt(max(r, 1))),
            "X": g(5, (B, L_hist, dm)), "x": g(6, (B, dm))}


def _layer_oracle(c, lens, plant=0, lib_path=None):
    L_cap = c["X"].shape[1] + 2
    cache = olayer.project_history("f64", c["X"], c["W_in"], c["H"], c["d_h"], c["r"], L_cap, lens)
    return olayer.layer_step("f64", c["x"], c["W_in"], c["W_o"], c["B_k"], c["B_v"], cache, lens, c["H"], c["d_h"],
                             c["r"], plant=plant, lib_path=lib_path)["y"]


def pin_layer_materialized_weights(lib_path=None, plant=0):
    """The factored step (project into the cache, LRKV decode, W_o) equals attention with every head's
    weights materialised, W_h = W_S + U_h B_h^T (reading notes sec. 2.1 Eqs. (2)-(5)), computed by a
    different route: torch fp64, keys and values of all tokens from the materialised weights."""
    for i, (B, H, d_h, r, dm, L) in enumerate([(2, 3, 4, 2, 7, 6), (1, 2, 8, 3, 5, 9), (2, 4, 4, 4, 16, 5)]):
        c = _layer_case(1100 + 10 * i, B, H, d_h, r, dm, L)
        lens = np.array([L - b for b in range(B)], dtype=np.int32)
        got = _layer_oracle(c, lens, plant, lib_path)
        t = {k: torch.from_numpy(np.asarray(v)) for k, v in c.items() if isinstance(v, np.ndarray)}
        o_rows = 0
        Wq = t["W_in"][0:H * d_h]; o_rows = H * d_h
        WSK = t["W_in"][o_rows:o_rows + d_h]; o_rows += d_h
        WSV = t["W_in"][o_rows:o_rows + d_h]; o_rows += d_h
        UK = t["W_in"][o_rows:o_rows + H * r]; o_rows += H * r
        UV = t["W_in"][o_rows:o_rows + H * r]
        ref = torch.zeros((B, dm), dtype=torch.float64)
        for b in range(B):
            n = int(lens[b])
            X_all = torch.cat([t["X"][b, :n], t["x"][b:b + 1]], dim=0)  # history then the new token
            heads = []
            for h in range(H):
                WK_h = WSK.T + UK[h * r:(h + 1) * r].T @ t["B_k"][h].T   # [dm][d_h]
                WV_h = WSV.T + UV[h * r:(h + 1) * r].T @ t["B_v"][h].T
                q_h = t["x"][b] @ Wq[h * d_h:(h + 1) * d_h].T
                K_h, V_h = X_all @ WK_h, X_all @ WV_h
                a = torch.softmax(K_h @ q_h / math.sqrt(d_h), dim=0)
                heads.append(a @ V_h)
            ref[b] = torch.cat(heads) @ t["W_o"].T
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def pin_layer_mha_special_case(lib_path=None, plant=0):
    """r = d_h, B_h = I, zero shared projections and d_model = H*d_h: the layer step is textbook multi-head
    attention, checked against torch's own implementation (fp64)."""
    B, H, d_h, L = 2, 3, 4, 6
    dm, r = H * d_h, d_h
    c = _layer_case(1200, B, H, d_h, r, dm, L)
    c["W_in"][H * d_h:H * d_h + 2 * d_h] = 0.0
    c["B_k"] = np.broadcast_to(np.eye(d_h), (H, d_h, d_h)).copy()
    c["B_v"] = c["B_k"].copy()
    lens = np.array([L, L - 2], dtype=np.int32)
    got = _layer_oracle(c, lens, plant, lib_path)
    W = torch.from_numpy(c["W_in"])
    in_proj = torch.cat([W[:H * d_h], W[H * d_h + 2 * d_h:H * d_h + 2 * d_h + H * r],
                         W[H * d_h + 2 * d_h + H * r:]], dim=0)
    for b in range(B):
        n = int(lens[b])
        X_all = torch.cat([torch.from_numpy(c["X"][b, :n]), torch.from_numpy(c["x"][b:b + 1])], dim=0)
        ref, _ = torch.nn.functional.multi_head_attention_forward(
            torch.from_numpy(c["x"][b:b + 1])[:, None, :], X_all[:, None, :], X_all[:, None, :], dm, H,
            in_proj, None, None, None, False, 0.0, torch.from_numpy(c["W_o"]), None, training=False,
            need_weights=False)
        np.testing.assert_allclose(got[b], ref[0, 0].numpy(), rtol=1e-10, atol=1e-12)


def pin_layer_rounding(lib_path=None, plant=0):
    """Stored rows are the fp64 projections rounded to the cache dtype: fp32 values are the nearest fp32,
    bf16 values the nearest bf16 of that (both round half to even); bf16 of an exact bf16 value is itself."""
    # bf16 keeps 7 fraction bits: the spacing just above 1 is 2^-7
    y = np.array([1.0, 1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9, -2.5, 1.0 + 2.0 ** -30,
                  1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])  # the last two are exact ties
    b = olayer.round_to("bf16", y)
    np.testing.assert_array_equal(olayer.widen("bf16", b),
                                  [1.0, 1.0, 1.0 + 2.0 ** -7, -2.5, 1.0, 1.0, 1.0 + 2.0 ** -6])
    np.testing.assert_array_equal(olayer.widen("f32", olayer.round_to("f32", y)), y.astype(np.float32))


LAYER_PINS = [pin_layer_materialized_weights, pin_layer_mha_special_case, pin_layer_rounding]


@pytest.mark.parametrize("pin", LAYER_PINS, ids=lambda f: f.__name__)
def test_layer_pin(pin):
    pin()


@pytest.mark.parametrize("plant", [1, 2, 3, 4])
def test_layer_planted_mistake_is_caught(plant):
    """The layer reference with one planted mistake (K/V projections swapped, W_o transposed, heads of the
    value latents reversed, new token not appended) must fail at least one layer pin."""
    failed = []
    for pin in LAYER_PINS:
        try:
            pin(plant=plant)
        except (AssertionError, ValueError, RuntimeError):
            failed.append(pin.__name__)
    assert failed, f"planted layer mistake {plant} slipped through every pin"


# ---------------------------------------------------------------------------------------------
# several query tokens per sequence with a causal mask inside the chunk
# ---------------------------------------------------------------------------------------------
def pin_multi_query_causal(lib_path=None):
    """Q trailing query tokens with the causal mask inside the chunk, checked against torch's
    scaled_dot_product_attention (fp64) on materialised per-head keys and values with an explicit mask."""
    for i, (B, Q, H, d_h, r, L) in enumerate([(2, 3, 2, 8, 3, 9), (1, 4, 3, 4, 2, 4), (3, 2, 1, 6, 6, 7)]):
        c = _random_case(1300 + 10 * i, B, H, d_h, r, L, [L - b for b in range(B)])
        q = _rand(1305 + 10 * i, (B, Q, H, d_h))
        lens = np.array([L - b for b in range(B)], dtype=np.int32)
        got = oracle.lrkv_decode_multi("f64", q, c["k"], c["v"], c["zk"], c["zv"], c["Bk"], c["Bv"], lens,
                                       lib_path=lib_path)
        for b in range(B):
            n = int(lens[b])
            for h in range(H):
                K = torch.from_numpy(c["k"][b, :n] + c["zk"][b, h, :n] @ c["Bk"][h].T)
                V = torch.from_numpy(c["v"][b, :n] + c["zv"][b, h, :n] @ c["Bv"][h].T)
                pos = torch.arange(n - Q, n)[:, None]           # query positions (may be negative)
                mask = torch.arange(n)[None, :] <= pos           # [Q][n]
                qq = torch.from_numpy(q[b, :, h])
                ref = torch.nn.functional.scaled_dot_product_attention(qq[None], K[None], V[None],
                                                                       attn_mask=mask[None])[0]
                seen = mask.any(dim=1)
                ref = torch.where(seen[:, None], ref, torch.zeros_like(ref))  # a query that sees nothing: 0
                np.testing.assert_allclose(got[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-13)


ALL_PINS.append(pin_multi_query_causal)


def pin_materialize_weight_space(lib_path=None, plant=0):
    """Keys and values rebuilt from the factored cache equal the projections through materialised weights
    W_h = W_S + U_h B_h^T (torch fp64 route), and attending over them reproduces the decode reference."""
    B, H, d_h, r, dm, L = 2, 3, 4, 2, 7, 6
    c = _layer_case(1400, B, H, d_h, r, dm, L)
    lens = np.array([L, L - 2], dtype=np.int32)
    cache = olayer.project_history("f64", c["X"], c["W_in"], H, d_h, r, L, lens)
    K, V = olayer.materialize("f64", cache["k_shared"], cache["v_shared"], cache["z_k"], cache["z_v"], c["B_k"],
                              c["B_v"], lens)
    W = torch.from_numpy(c["W_in"])
    o = H * d_h
    WSK, WSV = W[o:o + d_h], W[o + d_h:o + 2 * d_h]
    UK, UV = W[o + 2 * d_h:o + 2 * d_h + H * r], W[o + 2 * d_h + H * r:]
    for b in range(B):
        n = int(lens[b])
        X = torch.from_numpy(c["X"][b, :n])
        for h in range(H):
            WK_h = WSK.T + UK[h * r:(h + 1) * r].T @ torch.from_numpy(c["B_k"][h]).T
            WV_h = WSV.T + UV[h * r:(h + 1) * r].T @ torch.from_numpy(c["B_v"][h]).T
            np.testing.assert_allclose(K[b, h, :n], (X @ WK_h).numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(V[b, h, :n], (X @ WV_h).numpy(), rtol=1e-12, atol=1e-12)
        assert not K[b, :, n:].any() and not V[b, :, n:].any()
    q = _rand(1410, (B, H, d_h))
    ref = oracle.lrkv_decode("f64", q, cache["k_shared"], cache["v_shared"], cache["z_k"], cache["z_v"], c["B_k"],
                             c["B_v"], lens, lib_path=lib_path).reshape(B, H, d_h)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            a = torch.softmax(torch.from_numpy(K[b, h, :n] @ q[b, h]) / math.sqrt(d_h), dim=0)
            np.testing.assert_allclose(ref[b, h], (a @ torch.from_numpy(V[b, h, :n])).numpy(), rtol=1e-12,
                                       atol=1e-13)


LAYER_PINS.append(pin_materialize_weight_space)
