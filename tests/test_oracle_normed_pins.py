"""Pins for the normalised-variant CPU reference (oracle.normed): each check ties it to something other than
itself.

  * the textbook route: per-head keys rebuilt in full, torch's rms_norm on keys and queries (with the gains as
    its weight), torch's scaled_dot_product_attention, all in float64;
  * the review's expansion of the key's squared norm into shared, cross and private terms (sec. 8), evaluated
    without rebuilding a key;
  * with unit gains and eps = 0 the logit is sqrt(d_h) times the cosine of query and key (a closed form);
  * scaling one token's key factors by c > 0 leaves every output unchanged when eps = 0 (RMS normalisation is
    scale-free), which fails as soon as the scale misses a part of the logit.
Each pin takes ``plant``; the last test checks that every planted mistake fails at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import normed


def _rand(seed, shape, std=1.0, mean=0.0):
    n = int(np.prod(shape))
    return mean + synth.normal(seed, std, n, "f64").reshape(shape)


def _case(seed, B, H, d_h, r, L_cap, lens, eps=1e-5):
    return {"q": _rand(seed, (B, H, d_h)), "ks": _rand(seed + 1, (B, L_cap, d_h)),
            "vs": _rand(seed + 2, (B, L_cap, d_h)), "zk": _rand(seed + 3, (B, H, L_cap, r)),
            "zv": _rand(seed + 4, (B, H, L_cap, r)), "bk": _rand(seed + 5, (H, d_h, r), 1 / math.sqrt(max(r, 1))),
            "bv": _rand(seed + 6, (H, d_h, r), 1 / math.sqrt(max(r, 1))),
            "gq": _rand(seed + 7, (H, d_h), 0.3, 1.0), "gk": _rand(seed + 8, (H, d_h), 0.3, 1.0),
            "lens": np.array(lens, dtype=np.int32), "eps": eps}


def _oracle(c, plant=0):
    rho = normed.key_scales("f64", c["ks"], c["zk"], c["bk"], c["lens"], c["eps"], plant=plant)
    qe = normed.norm_query("f64", c["q"], c["gq"], c["gk"], c["eps"], plant=plant)
    return normed.decode_normed("f64", qe, c["ks"], c["vs"], c["zk"], c["zv"], c["bk"], c["bv"], rho, c["lens"],
                                plant=plant)


def _textbook(c):
    """Normalised attention written out with torch library routines (float64)."""
    q, ks, vs = (torch.from_numpy(c[k]) for k in ("q", "ks", "vs"))
    zk, zv, bk, bv = (torch.from_numpy(c[k]) for k in ("zk", "zv", "bk", "bv"))
    gq, gk = torch.from_numpy(c["gq"]), torch.from_numpy(c["gk"])
    B, H, _, r = zk.shape
    d_h = q.shape[-1]
    out = torch.zeros(B, H, d_h, dtype=torch.float64)
    for b in range(B):
        n = int(c["lens"][b])
        for h in range(H):
            K = ks[b, :n] + torch.matmul(zk[b, h, :n], bk[h].T.contiguous())
            V = vs[b, :n] + torch.matmul(zv[b, h, :n], bv[h].T.contiguous())
            kn = torch.nn.functional.rms_norm(K, (d_h,), weight=gk[h], eps=c["eps"])
            qn = torch.nn.functional.rms_norm(q[b, h][None, :], (d_h,), weight=gq[h], eps=c["eps"])
            out[b, h] = torch.nn.functional.scaled_dot_product_attention(qn[None], kn[None], V[None])[0, 0]
    return out.numpy()


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------------------------------------

def pin_textbook_route(plant=0):
    for seed, (B, H, d_h, r, L_cap, lens) in [(500, (2, 3, 8, 3, 9, [7, 4])), (510, (1, 2, 16, 0, 6, [6])),
                                             (520, (2, 4, 8, 8, 5, [1, 5]))]:
        c = _case(seed, B, H, d_h, r, L_cap, lens)
        err = _rel(_oracle(c, plant), _textbook(c))
        assert err < 1e-12, f"textbook route differs by {err:.3e} (seed {seed})"


def pin_expanded_norm(plant=0):
    """d_h n^2 = |s|^2 + 2 (s B).z + z (B^T B) z^T + d_h eps (review sec. 8), with no key rebuilt."""
    c = _case(530, 2, 3, 8, 4, 7, [7, 3], eps=1e-3)
    rho = normed.key_scales("f64", c["ks"], c["zk"], c["bk"], c["lens"], c["eps"], plant=plant)
    d_h = c["ks"].shape[-1]
    for b in range(2):
        n = int(c["lens"][b])
        for h in range(3):
            s, z, Bh = c["ks"][b, :n], c["zk"][b, h, :n], c["bk"][h]
            gram = Bh.T @ Bh
            dn2 = np.einsum("jc,jc->j", s, s) + 2 * np.einsum("jk,jk->j", s @ Bh, z) \
                + np.einsum("jk,kl,jl->j", z, gram, z) + d_h * c["eps"]
            want = 1.0 / np.sqrt(dn2 / d_h)
            assert np.allclose(rho[b, h, :n], want, rtol=1e-12, atol=0), f"expanded norm differs at ({b},{h})"
            assert np.all(rho[b, h, n:] == 0.0)


def pin_cosine_logits(plant=0):
    """Unit gains, eps = 0: logit = sqrt(d_h) cos(q, k).  One-hot values (v_j = e_j, no private value part)
    make the output the softmax weight vector itself."""
    B, H, d_h, r, L = 1, 2, 8, 3, 6
    c = _case(540, B, H, d_h, r, L, [L], eps=0.0)
    c["gq"] = np.ones((H, d_h))
    c["gk"] = np.ones((H, d_h))
    c["vs"] = np.zeros((B, L, d_h))
    c["vs"][0, np.arange(L), np.arange(L)] = 1.0
    c["zv"] = np.zeros((B, H, L, r))
    got = _oracle(c, plant)
    for h in range(H):
        K = c["ks"][0] + c["zk"][0, h] @ c["bk"][h].T
        q = c["q"][0, h]
        cos = np.array([np.dot(q, k) / (np.linalg.norm(q) * np.linalg.norm(k)) for k in K])
        w = np.exp(math.sqrt(d_h) * cos)
        w /= w.sum()
        assert np.allclose(got[0, h, :L], w, rtol=1e-12, atol=1e-15), f"cosine weights differ (head {h})"
        assert np.all(np.abs(got[0, h, L:]) < 1e-300)


def pin_row_scale_invariance(plant=0):
    """eps = 0: multiplying token j's shared key row and all its key latents by c_j > 0 changes nothing."""
    c = _case(550, 2, 3, 8, 4, 7, [7, 5], eps=0.0)
    base = _oracle(c, plant)
    cj = np.exp(_rand(551, (2, 7), 1.0))
    c2 = dict(c)
    c2["ks"] = c["ks"] * cj[:, :, None]
    c2["zk"] = c["zk"] * cj[:, None, :, None]
    err = _rel(_oracle(c2, plant), base)
    assert err < 1e-12, f"per-row key scaling moved the output by {err:.3e}"


NORMED_PINS = [pin_textbook_route, pin_expanded_norm, pin_cosine_logits, pin_row_scale_invariance]


@pytest.mark.parametrize("pin", NORMED_PINS, ids=lambda p: p.__name__)
def test_normed_pin(pin):
    pin()


@pytest.mark.parametrize("plant", [1, 2, 3, 4])
def test_normed_planted_mistake_is_caught(plant):
    """Planted mistakes: the scale taken from the shared key part alone (1), the key gain not folded into the
    query (2), eps added outside the square root (3), the scale applied to the shared logit part only (4)."""
    failed = []
    for pin in NORMED_PINS:
        try:
            pin(plant=plant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {plant} slipped through every pin"


def test_stored_rounding():
    """Stored rho and q_eff are the fp64 values rounded to nearest even, through fp32 for bf16 (1 + 2^-8 is a
    tie and stays at 1; 1 + 3 * 2^-9 is three quarters of an ulp and goes up)."""
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, 3.0e-3])
    got = normed.stored("bf16", x)
    want = np.array([0x3F80, 0x3F80, 0x3F81, 0x3B45], dtype=np.uint16)
    assert np.array_equal(got, want), got
