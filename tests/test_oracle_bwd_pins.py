"""Pins of the oracle's backward (dq, dk, dv of sum(dO * O)).

The gradients are fixed by central finite differences of the oracle's own
forward (the C two-pass routine, which shares no code with the numpy
backward), by torch.autograd through float64 scaled_dot_product_attention
with the equivalent additive mask (a library routine), and by invariants of
softmax: the rows of dS sum to zero, so without a nonlinear score
modification the key gradients of a head sum to zero, and the value
gradients sum to the output gradients of the rows that see any key.  No GPU.
"""
import functools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

assert_close = functools.partial(np.testing.assert_allclose, rtol=0)

MODS = ("vanilla", "alibi", "softcap")
MASKS = (None, "causal", "sliding_window", "prefix_lm", "document")


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def kw_for(mod, mask, B, S, rng):
    kw = dict(variant=mod if mask is None or mod != "vanilla" else mask)
    if mask is not None and mod != "vanilla":
        kw["mask"] = mask
    if mod == "softcap":
        kw["softcap"] = 1.5
    if mod == "alibi":
        kw["alibi_max_bias"] = 4.0
    if mask == "sliding_window":
        kw.update(window=3, window_causal=True)
    if mask == "prefix_lm":
        kw["prefix"] = 3
    if mask == "document":
        offs = []
        for _ in range(B):
            cuts = np.sort(rng.choice(np.arange(1, S), size=2, replace=False))
            offs.append(np.concatenate([[0], cuts, [S]]))
        kw["doc_offsets"] = np.array(offs, np.int32)
    return kw


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
def test_bwd_matches_finite_differences(oracle_mod, mod, mask):
    rng = np.random.default_rng(1000 + 7 * MODS.index(mod) + MASKS.index(mask))
    B, Hq, Hkv, S, D = 2, 4, 2, 9, 5
    q, k, v = rnd(rng, B, Hq, S, D, scale=1.5), rnd(rng, B, Hkv, S, D), rnd(rng, B, Hkv, S, D)
    do = rnd(rng, B, Hq, S, D)
    kw = kw_for(mod, mask, B, S, rng)
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, **kw)

    def loss(q_, k_, v_):
        return float((oracle_mod.attn(q_, k_, v_, **kw)[0] * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(12)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if a is x else a for a in args]
            am = [xm if a is x else a for a in args]
            fd = (loss(*ap) - loss(*am)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


def sdpa_grads(q, k, v, do, attn_mask, scale=None):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = t[1].repeat_interleave(Hq // Hkv, dim=1)
    vv = t[2].repeat_interleave(Hq // Hkv, dim=1)
    o = F.scaled_dot_product_attention(t[0], kk, vv, attn_mask=attn_mask, scale=scale)
    (o * torch.tensor(do)).sum().backward()
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("variant", ["vanilla", "causal", "alibi", "sliding_window", "prefix_lm"])
def test_bwd_matches_autograd_sdpa(oracle_mod, variant):
    rng = np.random.default_rng(1100)
    B, Hq, Hkv, S, D = 2, 4, 2, 33, 8
    q, k, v = rnd(rng, B, Hq, S, D), rnd(rng, B, Hkv, S, D), rnd(rng, B, Hkv, S, 6)
    do = rnd(rng, B, Hq, S, 6)
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    kw = dict(variant=variant)
    if variant == "vanilla":
        bias = np.zeros((1, 1, S, S))
    elif variant == "causal":
        bias = np.where(j <= i, 0.0, -np.inf)[None, None]
    elif variant == "sliding_window":
        kw.update(window=5)
        bias = np.where((j <= i) & (j > i - 5), 0.0, -np.inf)[None, None]
    elif variant == "prefix_lm":
        kw.update(prefix=7)
        bias = np.where((j < 7) | (j <= i), 0.0, -np.inf)[None, None]
    else:
        kw.update(alibi_max_bias=8.0)
        slopes = 2.0 ** (-8.0 * (np.arange(Hq) + 1) / Hq)
        bias = (-slopes[:, None, None] * np.abs(i - j))[None]
    want = sdpa_grads(q, k, v, do, torch.tensor(bias))
    got = oracle_mod.attn_bwd(q, k, v, do, **kw)
    for g, w in zip(got, want):
        assert_close(g, w, atol=1e-11)


@pytest.mark.parametrize("mask", MASKS)
def test_bwd_invariants(oracle_mod, mask):
    rng = np.random.default_rng(1200 + MASKS.index(mask))
    B, H, S, D = 2, 3, 17, 4
    q, k, v, do = (rnd(rng, B, H, S, D) for _ in range(4))
    kw = kw_for("alibi", mask, B, S, rng)
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, **kw)
    # rows of dS sum to zero: an additive modification keeps sum_j dk_j = 0
    assert_close(dk.sum(2), 0.0, atol=1e-12)
    # value gradients collect each row's dO once (its probabilities sum to 1)
    assert_close(dv.sum(2), do.sum(2), atol=1e-12)


def test_bwd_uniform_scores_closed_form(oracle_mod):
    """Q = 0 under the causal mask: P_ij = 1/(i+1) for j <= i, so
    dV_j = sum_{i>=j} dO_i/(i+1), and dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j."""
    rng = np.random.default_rng(1300)
    S, D = 12, 4
    q = np.zeros((1, 1, S, D))
    k, v, do = (rnd(rng, 1, 1, S, D) for _ in range(3))
    dq, dk, dv = oracle_mod.attn_bwd(q, k, v, do, variant="causal")
    for jj in range(S):
        want = sum(do[0, 0, ii] / (ii + 1) for ii in range(jj, S))
        assert_close(dv[0, 0, jj], want, atol=1e-13)
    assert_close(dk, 0.0, atol=1e-14)  # dK = scale dS^T Q with Q = 0
    for ii in (0, 5, S - 1):
        p = np.full(ii + 1, 1.0 / (ii + 1))
        dp = do[0, 0, ii] @ v[0, 0, : ii + 1].T
        ds = p * (dp - (p * dp).sum())
        assert_close(dq[0, 0, ii], 0.5 * ds @ k[0, 0, : ii + 1], atol=1e-13)


def test_bwd_heads_subset(oracle_mod):
    rng = np.random.default_rng(1400)
    q, k, v, do = rnd(rng, 2, 4, 10, 4), rnd(rng, 2, 2, 10, 4), rnd(rng, 2, 2, 10, 4), rnd(rng, 2, 4, 10, 4)
    full = oracle_mod.attn_bwd(q, k, v, do, variant="softcap", softcap=2.0)
    part = oracle_mod.attn_bwd(q, k, v, do, variant="softcap", softcap=2.0, heads=[(1, 0)])
    assert_close(part[0][1, :2], full[0][1, :2], atol=0)
    assert_close(part[1][1, 0], full[1][1, 0], atol=0)
    assert_close(part[2][1, 0], full[2][1, 0], atol=0)
    assert (part[1][0] == 0).all()
