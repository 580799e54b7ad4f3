"""Pins for the rotary-position reference (oracle.rope): each check ties it to something other than itself.

  * the textbook route: per-head keys rebuilt in full, rotated as complex numbers (coordinate pair k of a row
    read as x_2k + i x_2k+1 and multiplied by exp(i phi)), the query likewise, then torch's
    scaled_dot_product_attention in float64;
  * rotary scores depend on relative positions only: shifting every position by the same amount leaves the
    output unchanged;
  * the pages' rank-one example (a residual basis along the first axis, review sec. 8 / reading notes
    sec. 2.7) in closed form: the private key turns off its axis, so the score is sin of the position gap.
Each pin takes ``plant``; the last test checks that every planted mistake fails at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import rope


def _rand(seed, shape, std=1.0):
    return synth.normal(seed, std, int(np.prod(shape)), "f64").reshape(shape)


def _case(seed, B, H, d_h, r, L_cap, lens):
    return {"q": _rand(seed, (B, H, d_h)), "ks": _rand(seed + 1, (B, L_cap, d_h)),
            "vs": _rand(seed + 2, (B, L_cap, d_h)), "zk": _rand(seed + 3, (B, H, L_cap, r)),
            "zv": _rand(seed + 4, (B, H, L_cap, r)), "bk": _rand(seed + 5, (H, d_h, r), 1 / math.sqrt(max(r, 1))),
            "bv": _rand(seed + 6, (H, d_h, r), 1 / math.sqrt(max(r, 1))), "lens": np.array(lens, dtype=np.int32)}


def _oracle(c, plant=0, pos0=0, base=10000.0):
    return rope.decode_rope("f64", c["q"], c["ks"], c["vs"], c["zk"], c["zv"], c["bk"], c["bv"], c["lens"],
                            base=base, pos0=pos0, plant=plant)


def _complex_turn(x, pos, base):
    """x [n][d] (torch float64) turned at positions pos [n] as complex pairs."""
    d = x.shape[-1]
    theta = base ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    phi = torch.as_tensor(pos, dtype=torch.float64)[:, None] * theta[None, :]
    xc = torch.view_as_complex(x.reshape(x.shape[0], d // 2, 2).contiguous())
    return torch.view_as_real(xc * torch.polar(torch.ones_like(phi), phi)).reshape(x.shape[0], d)


def _textbook(c, base=10000.0):
    q, ks, vs = (torch.from_numpy(c[k]) for k in ("q", "ks", "vs"))
    zk, zv, bk, bv = (torch.from_numpy(c[k]) for k in ("zk", "zv", "bk", "bv"))
    B, H, _, r = zk.shape
    d_h = q.shape[-1]
    out = torch.zeros(B, H, d_h, dtype=torch.float64)
    for b in range(B):
        n = int(c["lens"][b])
        for h in range(H):
            K = ks[b, :n] + torch.matmul(zk[b, h, :n], bk[h].T.contiguous())
            V = vs[b, :n] + torch.matmul(zv[b, h, :n], bv[h].T.contiguous())
            Kt = _complex_turn(K, np.arange(n), base)
            qt = _complex_turn(q[b, h][None, :], [n - 1], base)
            out[b, h] = torch.nn.functional.scaled_dot_product_attention(qt[None, None], Kt[None, None],
                                                                         V[None, None])[0, 0, 0]
    return out.numpy()


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------------------------------------

def pin_textbook_route(plant=0):
    for seed, (B, H, d_h, r, L_cap, lens), base in [(600, (2, 3, 8, 3, 9, [9, 4]), 10000.0),
                                                    (610, (1, 2, 16, 0, 12, [12]), 10000.0),
                                                    (620, (2, 2, 8, 8, 40, [40, 17]), 50.0)]:
        c = _case(seed, B, H, d_h, r, L_cap, lens)
        err = _rel(_oracle(c, plant, base=base), _textbook(c, base))
        assert err < 1e-12, f"textbook route differs by {err:.3e} (seed {seed})"


def pin_relative_positions(plant=0):
    c = _case(630, 2, 3, 8, 4, 20, [20, 7])
    err = _rel(_oracle(c, plant, pos0=1000), _oracle(c, plant, pos0=0))
    assert err < 1e-9, f"a common position shift moved the output by {err:.3e}"


def pin_rank_one_example(plant=0):
    """d_h 2, r 1, B = e_1, no shared key part: row 0 has latent 1 (key e_1 before rotation), row 1 a zero key;
    values (1, 0) and 0.  Rows at positions 5 and 6, the query (0, 1) at position 6: its score against row 0
    is sin(5 - 6) / sqrt(2), against row 1 zero, so out = (sigmoid(-sin(1) / sqrt(2)), 0)."""
    c = {"q": np.array([[[0.0, 1.0]]]), "ks": np.zeros((1, 2, 2)), "vs": np.array([[[1.0, 0.0], [0.0, 0.0]]]),
         "zk": np.array([[[[1.0], [0.0]]]]), "zv": np.zeros((1, 1, 2, 1)), "bk": np.array([[[1.0], [0.0]]]),
         "bv": np.zeros((1, 2, 1)), "lens": np.array([2], dtype=np.int32)}
    got = _oracle(c, plant, pos0=5, base=10000.0)[0, 0]
    a0 = 1.0 / (1.0 + math.exp(math.sin(1.0) / math.sqrt(2.0)))
    assert abs(got[0] - a0) < 1e-14 and abs(got[1]) < 1e-15, got


ROPE_PINS = [pin_textbook_route, pin_relative_positions, pin_rank_one_example]


@pytest.mark.parametrize("pin", ROPE_PINS, ids=lambda p: p.__name__)
def test_rope_pin(pin):
    pin()


@pytest.mark.parametrize("plant", [1, 2, 3])
def test_rope_planted_mistake_is_caught(plant):
    """Planted mistakes: the private key part left unrotated (1), the rotation turned the other way (2), the
    query left at position 0 (3)."""
    failed = []
    for pin in ROPE_PINS:
        try:
            pin(plant=plant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {plant} slipped through every pin"
