"""GPU invariances and structured inputs at the long-context shape.

The decode has no positional term and uses the factors only through z B^T, so its output must not depend
on how the split plan cuts a sequence, on the order of the cached rows, or on the gauge of the factors
(z -> z C, B -> B C for an orthogonal C).  Softmax state is merged across splits by rescaling, so the case
where one row carries almost all the weight, and arrives in the last split merged, must come out right;
and the shared and private key terms are added before the softmax, so keys whose two parts nearly cancel
must come out right too ("Low-Rank Key Value Attention | What a shared cache can preserve", sec. 3, the
fused online-softmax paragraph after Algorithm 2, and sec. 9, the verification inputs it asks for;
"Low-Rank Key Value Attention: Chinese reading notes", sec. 2.4, Eqs. (6)-(7)).

Every call goes through the C ABI.  Outputs are compared with the fp64 reference on the inputs as stored on
the device (metric max over (b, h) of ||gpu - ref||_inf / ||ref||_inf), and with each other.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_shared_kv_amd as lk
from oracle import layer as olayer
import synth
from synth import device as sdev

pytestmark = pytest.mark.gpu

from gpu_harness import TOL, dims_of, gpu_decode, say  # noqa: E402

LONG = synth.WORKLOADS["long_context"]  # batch 4, H 32, d_h 128, r 64, L 32768, bf16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lk.lib()
    yield


@pytest.fixture(scope="module")
def long_dev():
    """The long-context inputs on the device (every sequence at its full length)."""
    say(f"[fixture] long-context cache B={LONG.batch} H={LONG.H} d_h={LONG.d_h} r={LONG.r} L={LONG.L}")
    dev = sdev.fill_layer(LONG, 0)
    yield dev
    del dev
    torch.cuda.empty_cache()


def _np_store(t: torch.Tensor) -> np.ndarray:
    """A device tensor as stored (fp32, or bf16 bit patterns as uint16) on the host."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _reference(w, dev, pairs, mqa=False):
    """fp64 reference of the given (b, h) pairs on the inputs exactly as stored on the device."""
    lens = dev["seq_lens"].cpu().numpy()
    q = _np_store(dev["q"])
    out = np.zeros((len(pairs), w.d_h))
    for b in sorted({b for b, _ in pairs}):
        idx = [i for i, (bb, _) in enumerate(pairs) if bb == b]
        n = int(lens[b])
        ks = _np_store(dev["k_shared"][b, :n])[None]
        vs = _np_store(dev["v_shared"][b, :n])[None]
        one = np.array([n], dtype=np.int32)
        sub = [(0, pairs[i][1]) for i in idx]
        if mqa:
            res = oracle.mqa_decode(w.dtype, q[b:b + 1], ks, vs, one, pairs=sub)
        else:
            zk = _np_store(dev["z_k"][b, :n].transpose(0, 1))[None]  # token-major -> [H][n][r]
            zv = _np_store(dev["z_v"][b, :n].transpose(0, 1))[None]
            res = oracle.lrkv_decode(w.dtype, q[b:b + 1], ks, vs, zk, zv, _np_store(dev["B_k"]),
                                     _np_store(dev["B_v"]), one, pairs=sub)
        out[idx] = res
    return out


def _err(got, ref, pairs):
    g = got.detach().cpu().numpy().astype(np.float64)
    sel = np.stack([g[b, h] for (b, h) in pairs])
    assert np.all(np.isfinite(sel))
    return oracle.relative_error(sel, ref)


def _rel_diff(a: torch.Tensor, b: torch.Tensor) -> float:
    """max over (b, h) of ||a - b||_inf / ||b||_inf between two GPU outputs."""
    x, y = a.double().cpu().numpy(), b.double().cpu().numpy()
    num = np.abs(x - y).max(axis=-1)
    den = np.abs(y).max(axis=-1)
    return float((num / np.where(den > 0, den, 1.0)).max())


def _check_vs_reference(w, dev, got, pairs, label, mqa=False):
    err = _err(got, _reference(w, dev, pairs, mqa=mqa), pairs)
    say(f"  {label}: max rel err {err:.3e} against the reference over {len(pairs)} (b,h) pairs "
        f"(tol {TOL[w.dtype]:.0e})")
    assert err <= TOL[w.dtype], (label, err)
    return err


# ---------------------------------------------------------------------------------------------------------
# split count
# ---------------------------------------------------------------------------------------------------------

def test_split_count_invariance_long_context(long_dev, monkeypatch):
    """One split per sequence, seven, and the default plan (64 per sequence): each bitwise reproducible, all
    within the bf16 tolerance of each other and of the reference."""
    w, dev = LONG, long_dev
    outs = {}
    for splits in (None, 1, 7):
        if splits:
            monkeypatch.setenv("LRKV_SPLITS", str(splits))
        else:
            monkeypatch.delenv("LRKV_SPLITS", raising=False)
        G, chunk = lk.lrkv_decode_num_splits(dims_of(w), w.L)
        say(f"[case] long context, LRKV_SPLITS={splits}: G={G} granule={chunk}")
        if splits:
            assert G == splits * w.batch
        a = gpu_decode(w, dev, w.L)
        b = gpu_decode(w, dev, w.L)
        assert torch.equal(a, b), f"splits={splits}: not bitwise reproducible"
        outs[splits] = a
    monkeypatch.delenv("LRKV_SPLITS", raising=False)
    for s in (1, 7):
        d = _rel_diff(outs[s], outs[None])
        say(f"  {s} split(s) vs default plan: max rel diff {d:.3e}")
        assert d <= TOL["bf16"]
    pairs = [(b, h) for b in range(w.batch) for h in (0, 9 + 6 * b, w.H - 1)]
    for s, o in outs.items():
        _check_vs_reference(w, dev, o, pairs, f"splits={s}")


# ---------------------------------------------------------------------------------------------------------
# token order and gauge
# ---------------------------------------------------------------------------------------------------------

def test_token_permutation_long_context(long_dev):
    """Permuting the cached rows of every sequence (shared rows and both latents together) leaves the output
    unchanged within tolerance: there is no positional term, and masking, splits and merge do not depend on
    which row sits where."""
    w, dev = LONG, long_dev
    base = gpu_decode(w, dev, w.L)
    gen = torch.Generator().manual_seed(5150)
    perm_dev = dict(dev)
    for k in ("k_shared", "v_shared", "z_k", "z_v"):
        perm_dev[k] = dev[k].clone()
    for b in range(w.batch):
        n = int(dev["seq_lens"][b])
        perm = torch.randperm(n, generator=gen).cuda()
        for k in ("k_shared", "v_shared", "z_k", "z_v"):
            perm_dev[k][b, :n] = dev[k][b, :n].index_select(0, perm)
    say("[case] long context, rows permuted within every sequence")
    got = gpu_decode(w, perm_dev, w.L)
    d = _rel_diff(got, base)
    say(f"  permuted vs original: max rel diff {d:.3e}")
    assert d <= TOL["bf16"]
    del perm_dev


def test_gauge_signed_permutation_long_context(long_dev):
    """z -> z C and B -> B C with C a signed permutation of the rank coordinates (orthogonal, and exact in
    bf16), separately for keys and values: z B^T is unchanged, so the output is too, within tolerance."""
    w, dev = LONG, long_dev
    base = gpu_decode(w, dev, w.L)
    g_dev = dict(dev)
    rng = np.random.default_rng(77)
    for zname, bname in (("z_k", "B_k"), ("z_v", "B_v")):
        perm = torch.from_numpy(rng.permutation(w.r)).cuda()
        sign = torch.from_numpy(rng.choice([-1.0, 1.0], size=w.r)).to(dev[zname].dtype).cuda()
        g_dev[zname] = dev[zname].index_select(-1, perm) * sign   # (z C)[i] = z[perm[i]] * sign[i]
        g_dev[bname] = dev[bname].index_select(-1, perm) * sign   # (B C)[c][i] = B[c][perm[i]] * sign[i]
    say("[case] long context, gauge z -> zC, B -> BC with a signed permutation C")
    got = gpu_decode(w, g_dev, w.L)
    d = _rel_diff(got, base)
    say(f"  gauged vs original: max rel diff {d:.3e}")
    assert d <= TOL["bf16"]
    pairs = [(b, h) for b in range(w.batch) for h in (3, w.H - 5)]
    _check_vs_reference(w, g_dev, got, pairs, "gauged")
    del g_dev


def test_gauge_orthogonal_fp32():
    """A general orthogonal C (seeded, from a QR factorisation) on fp32 factors: z C and B C are rounded to
    fp32 once, which moves z B^T by about 1e-7 relative, so the output moves by less than the fp32
    tolerance."""
    w = synth.WORKLOADS["ragged"].with_(name="gauge_fp32", batch=3, H=8, d_h=64, r=16, dtype="f32", L=2000,
                                        L_cap=2016, ragged_lo=None)
    lens = np.array([2000, 777, 33], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=2016, lengths=lens)
    base = gpu_decode(w, dev, 2000, L_cap=2016)
    g_dev = dict(dev)
    rng = np.random.default_rng(78)
    for zname, bname in (("z_k", "B_k"), ("z_v", "B_v")):
        C, _ = np.linalg.qr(rng.standard_normal((w.r, w.r)))
        Ct = torch.from_numpy(C).cuda()
        g_dev[zname] = (dev[zname].double() @ Ct).float()
        g_dev[bname] = (dev[bname].double() @ Ct).float()
    say("[case] fp32 gauge with a general orthogonal C")
    got = gpu_decode(w, g_dev, 2000, L_cap=2016)
    d = _rel_diff(got, base)
    say(f"  gauged vs original: max rel diff {d:.3e}")
    assert d <= TOL["f32"]


# ---------------------------------------------------------------------------------------------------------
# structured inputs: near-cancelling keys, one dominant row
# ---------------------------------------------------------------------------------------------------------

def test_near_cancelling_key_terms():
    """For two heads the shared key row is set to minus the head's private key term plus a small remainder
    (k_s ~ -z^K B^K^T + 0.05 n, with z^K of those heads scaled by 8), so the shared and private logits are
    each about 60 and cancel to about 0.5: the sum has to be formed accurately before the softmax."""
    w = LONG.with_(name="cancel", batch=2, L=4096, L_cap=4096)
    lens = np.array([4096, 3001], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=4096, lengths=lens)
    heads = {0: 5, 1: 22}  # the head whose key cancels, per sequence
    rng = np.random.default_rng(99)
    for b, h0 in heads.items():
        n = int(lens[b])
        z = (dev["z_k"][b, :n, h0].double() * 8.0).to(torch.bfloat16)
        dev["z_k"][b, :n, h0] = z
        priv = z.double() @ dev["B_k"][h0].double().T.contiguous()   # z^K_h0 (B^K_h0)^T, [n][d_h]
        noise = torch.from_numpy(rng.standard_normal((n, w.d_h)) * 0.05).cuda()
        dev["k_shared"][b, :n] = (-priv + noise).to(torch.bfloat16)
        kh = dev["k_shared"][b, :n].double() + priv
        ratio = float(kh.abs().max() / priv.abs().max())
        say(f"  sequence {b}, head {h0}: |k_s + z B^T| / |z B^T| = {ratio:.3f}")
        assert ratio < 0.1
    say("[case] near-cancelling shared and private key terms")
    got = gpu_decode(w, dev, 4096, L_cap=4096)
    pairs = [(b, h) for b in range(2) for h in range(w.H)]
    _check_vs_reference(w, dev, got, pairs, "near-cancelling keys")
    hot = [(b, h0) for b, h0 in heads.items()]
    err = _err(got, _reference(w, dev, hot), hot)
    say(f"  cancelling heads alone: max rel err {err:.3e}")


def _splits_of(G, lens, b, ntl):
    """Sequence b's split count (one query set per sequence, at most 64 sequences).  With the least cap M whose
    splits S_i = max(1, ceil(n_i / (M ntl))) add up to at most G (n_i the 32-row block counts): those S_i when
    M >= 8, else the length-proportional plan, where sequence i starts at workgroup i + floor((G - batch) C_{i-1} / T),
    C the running count of blocks and T their total."""
    nbs = [(int(n) + 31) // 32 for n in lens]
    need = lambda per: sum(max(1, -(-n // per)) for n in nbs)
    M = 1
    while need(M * ntl) > G:
        M += 1
    if M >= 8:
        return max(1, -(-nbs[b] // (M * ntl)))
    T, extra = sum(nbs), G - len(lens)
    W = lambda i: i + (extra * sum(nbs[:i])) // T if T else i
    return W(b + 1) - W(b)


def _last_row_of_last_split(G, lens, b, ntl):
    """A row in the block that split S_b - 1 (merged last) reaches last in its last row lane, following the
    split kernels' block deal (block s*NTL + tl + k*S_b*NTL) and their per-sequence rotation."""
    L = int(lens[b])
    nb = (L + 31) // 32
    S = _splits_of(G, lens, b, ntl)
    s, tl = S - 1, ntl - 1
    first, step = s * ntl + tl, S * ntl
    nmine = (nb - first + step - 1) // step if nb > first else 0
    if nmine == 0:
        return L - 1
    rot = (nmine * b) // len(lens)
    itr = (nmine - 1 + rot) % nmine
    blk = first + itr * step
    return min(32 * blk + 31, L - 1)


@pytest.mark.parametrize("where", ["last_row", "last_split"])
@pytest.mark.parametrize("logit", [6.0, 30.0, 200.0])
def test_dominant_row(where, logit):
    """One row per (sequence, head) gets a scaled logit of about 6 (a few percent of the weight), 30 (almost
    all of it) or 200 (every other weight underflows to 0 in fp32), by setting its key latent along the
    head's projected query.  The row is the sequence's last (the query's own token), or a row of the block
    that the last merged split reaches last."""
    w = LONG.with_(name="dominant", batch=2, L=8192, L_cap=8192)
    lens = np.array([8192, 6000], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=8192, lengths=lens)
    G, chunk = lk.lrkv_decode_num_splits(dims_of(w, 8192), 8192)
    ntl = chunk // 32
    q = olayer.widen("bf16", _np_store(dev["q"]))
    Bk = _np_store(dev["B_k"])
    p = oracle.absorb_query("bf16", _np_store(dev["q"]), Bk)  # [batch][H][r] fp64
    for b in range(2):
        n = int(lens[b])
        j = n - 1 if where == "last_row" else _last_row_of_last_split(G, lens, b, ntl)
        # the raw private score p.z = logit * sqrt(d_h) minus the row's shared score
        qk = q[b] @ olayer.widen("bf16", _np_store(dev["k_shared"][b, j]))
        target = logit * np.sqrt(w.d_h) - qk                         # [H]
        z = target[:, None] * p[b] / np.sum(p[b] ** 2, axis=1, keepdims=True)
        dev["z_k"][b, j] = torch.from_numpy(z).to(torch.bfloat16).cuda()
        say(f"  sequence {b}: dominant row {j} of {n} (G={G}, granule {chunk})")
    say(f"[case] dominant row, scaled logit {logit}, {where}")
    got = gpu_decode(w, dev, 8192, L_cap=8192)
    pairs = [(b, h) for b in range(2) for h in range(0, w.H, 3)]
    _check_vs_reference(w, dev, got, pairs, f"dominant {logit} {where}")


def test_dominant_row_mqa_fp32():
    """fp32 with r = 0 (the fp32 matrix-core kernel): the shared key of one row per sequence is set along head
    0's query so that head 0's scaled logit there is 30, in the block the last merged split reaches last."""
    w = synth.WORKLOADS["ragged_mqa_fp32"].with_(name="dominant_mqa", batch=2, L=8192, L_cap=8192, ragged_lo=None)
    lens = np.array([8192, 5000], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=8192, lengths=lens)
    G, chunk = lk.lrkv_decode_num_splits(dims_of(w, 8192), 8192)
    for b in range(2):
        n = int(lens[b])
        j = _last_row_of_last_split(G, lens, b, chunk // 32)
        q0 = dev["q"][b, 0].double()
        dev["k_shared"][b, j] = (30.0 * np.sqrt(w.d_h) * q0 / (q0 @ q0)).float()
        say(f"  sequence {b}: dominant row {j} of {n}")
    say("[case] dominant row, fp32 r = 0")
    got = gpu_decode(w, dev, 8192, L_cap=8192)
    pairs = [(b, h) for b in range(2) for h in range(0, w.H, 5)]
    _check_vs_reference(w, dev, got, pairs, "dominant mqa fp32", mqa=True)


def test_mqa_fp32_keys_of_wide_range():
    """fp32 with r = 0: the score product takes each key and query value as three bf16 parts; keys whose rows
    span 2^-12 to 2^2 in magnitude (every element with a full 24-bit significand) and queries scaled per head
    over 2^-4 to 2^2 exercise all three parts and leave some heads' softmax nearly flat and others peaked on
    a few rows (logits up to about 40).  Against the reference within the fp32 tolerance."""
    w = synth.WORKLOADS["ragged_mqa_fp32"].with_(name="wide_mqa", batch=3, L=3000, L_cap=3008, ragged_lo=None)
    lens = np.array([3000, 1777, 129], dtype=np.int32)
    dev = sdev.fill_layer(w, 0, L_cap=3008, lengths=lens)
    g = torch.Generator(device="cpu").manual_seed(4242)
    row_scale = torch.pow(2.0, torch.empty((3, 3008, 1)).uniform_(-10.0, 3.0, generator=g))
    mant = 1.0 + torch.rand((3, 3008, w.d_h), generator=g)  # significands in [1, 2): low bits set
    sign = torch.where(torch.rand((3, 3008, w.d_h), generator=g) < 0.5, -1.0, 1.0)
    dev["k_shared"].copy_((sign * mant * row_scale / 4.0).float().cuda())
    head_scale = torch.pow(2.0, torch.linspace(-4.0, 2.0, w.H)).view(1, w.H, 1)
    dev["q"].copy_((dev["q"].cpu() * head_scale).float().cuda())
    say("[case] fp32 r = 0, keys over 2^-12..2^2, queries over 2^-4..2^2 per head")
    got = gpu_decode(w, dev, 3000, L_cap=3008)
    pairs = [(b, h) for b in range(3) for h in range(0, w.H, 3)]
    _check_vs_reference(w, dev, got, pairs, "wide-range keys, mqa fp32", mqa=True)


# ---------------------------------------------------------------------------------------------------------
# rank 0 at the ragged fp32 shape on one kernel
# ---------------------------------------------------------------------------------------------------------

def test_r0_equals_zero_latents_bitwise_ragged_fp32_shape(monkeypatch):
    """At the ragged fp32 shape (64 sequences of the seeded lengths in [512, 32768], H 32, d_h 128) rank 0
    and rank 32 with all latents zero agree bit for bit when one kernel runs both: the private branch adds
    exact zeros.  The general kernel serves both (LRKV_FORCE_GENERAL); the fp32 matrix-core kernel, which
    serves rank 0 by default, agrees with it within the fp32 tolerance."""
    w0 = synth.WORKLOADS["ragged_mqa_fp32"]
    lens = synth.seq_lengths(w0)
    max_len = int(lens.max())
    say(f"[case] r=0 vs zero latents, fp32 B={w0.batch} H={w0.H} d_h={w0.d_h} lengths {lens.min()}..{max_len}")
    dev0 = sdev.fill_layer(w0, 0, lengths=lens)
    default = gpu_decode(w0, dev0, max_len)
    monkeypatch.setenv("LRKV_FORCE_GENERAL", "1")
    gen0 = gpu_decode(w0, dev0, max_len)
    wr = w0.with_(r=32)
    devr = dict(dev0)
    devr["z_k"] = torch.zeros((w0.batch, w0.cap, w0.H, 32), dtype=torch.float32, device="cuda")
    devr["z_v"] = torch.zeros_like(devr["z_k"])
    devr["B_k"] = sdev.to_device(synth.gen_small(wr, 0, "B_k"))
    devr["B_v"] = sdev.to_device(synth.gen_small(wr, 0, "B_v"))
    genr = gpu_decode(wr, devr, max_len)
    monkeypatch.delenv("LRKV_FORCE_GENERAL")
    assert torch.equal(gen0, genr), "general kernel: rank 0 and zero latents differ"
    d = _rel_diff(default, gen0)
    say(f"  fp32 matrix-core kernel vs general kernel at rank 0: max rel diff {d:.3e}")
    assert d <= TOL["f32"]
    del devr, dev0
    torch.cuda.empty_cache()
