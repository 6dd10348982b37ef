"""Pins of the oracle's decode rows (attention of the newest tokens against a
KV cache holding seqlens[b] tokens) and of its (O, LSE) merge.

Decode is fixed by brute force with its own position vectors, by the prefill
oracle on the same tokens (the last rows of a prefill are the decode of its
newest tokens), by closed forms for uniform scores, and by the degenerate
cases (empty cache, fewer cached tokens than queries, garbage past the
length).  The merge is fixed by splitting keys into disjoint parts whose
results must recombine into the whole, and by its identities.  No GPU.
"""
import functools
import math

import numpy as np
import pytest

from tests import _bruteforce as bf

# absolute tolerances only: numpy's default rtol of 1e-7 would hide small relative errors
assert_close = functools.partial(np.testing.assert_allclose, rtol=0)

MODS = ("vanilla", "alibi", "softcap")
MASKS = (None, "causal", "sliding_window", "prefix_lm")


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def kw_for(mod, mask, window_causal=True):
    kw = dict(variant=mod if mask is None or mod != "vanilla" else mask)
    if mask is not None and mod != "vanilla":
        kw["mask"] = mask
    if mod == "softcap":
        kw["softcap"] = 1.5
    if mod == "alibi":
        kw["alibi_max_bias"] = 8.0
    if mask == "sliding_window":
        kw.update(window=4, window_causal=window_causal)
    if mask == "prefix_lm":
        kw["prefix"] = 5
    return kw


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
@pytest.mark.parametrize("Sq", [1, 3])
def test_decode_matches_bruteforce(oracle_mod, mod, mask, Sq):
    rng = np.random.default_rng(600 + 7 * MODS.index(mod) + MASKS.index(mask) + 31 * Sq)
    B, Hq, Hkv, S_cap, D, Dv = 5, 4, 2, 19, 8, 6
    q = rnd(rng, B, Hq, Sq, D, scale=2.0)
    k, v = rnd(rng, B, Hkv, S_cap, D), rnd(rng, B, Hkv, S_cap, Dv)
    seqlens = np.array([19, 11, Sq, 0, 2], np.int32)  # full, partial, exactly Sq, empty, short
    kw = kw_for(mod, mask)
    o, lse = oracle_mod.decode(q, k, v, seqlens, **kw)
    o_bf, lse_bf = bf.decode_attention(q, k, v, seqlens, **kw)
    assert_close(o, o_bf, rtol=0, atol=1e-12)
    assert_close(lse, lse_bf, rtol=1e-12, atol=1e-12)


def test_decode_two_sided_window_bruteforce(oracle_mod):
    rng = np.random.default_rng(640)
    q, k, v = rnd(rng, 2, 2, 4, 8), rnd(rng, 2, 2, 16, 8), rnd(rng, 2, 2, 16, 3)
    seqlens = np.array([16, 9], np.int32)
    kw = kw_for("alibi", "sliding_window", window_causal=False)
    o, lse = oracle_mod.decode(q, k, v, seqlens, **kw)
    o_bf, lse_bf = bf.decode_attention(q, k, v, seqlens, **kw)
    assert_close(o, o_bf, atol=1e-12)
    assert_close(lse, lse_bf, atol=1e-12)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
def test_decode_is_the_tail_of_prefill(oracle_mod, mod, mask):
    """The last Sq rows of a prefill over L tokens are the decode of those
    tokens against a cache holding all L of them; what the cache holds past L
    never matters."""
    rng = np.random.default_rng(650 + 7 * MODS.index(mod) + MASKS.index(mask))
    Hq, Hkv, L, S_cap, Sq, D = 4, 2, 23, 40, 5, 8
    x_q = rnd(rng, 1, Hq, L, D, scale=2.0)
    x_k, x_v = rnd(rng, 1, Hkv, L, D), rnd(rng, 1, Hkv, L, 6)
    kw = kw_for(mod, mask)
    o_pre, lse_pre = oracle_mod.attn(x_q, x_k, x_v, **kw)
    k_cache = np.full((1, Hkv, S_cap, D), np.nan)
    v_cache = np.full((1, Hkv, S_cap, 6), np.nan)
    k_cache[:, :, :L], v_cache[:, :, :L] = x_k, x_v
    o, lse = oracle_mod.decode(x_q[:, :, L - Sq:], k_cache, v_cache, np.array([L], np.int32), **kw)
    assert_close(o, o_pre[:, :, L - Sq:], rtol=0, atol=1e-12)
    assert_close(lse, lse_pre[:, :, L - Sq:], rtol=0, atol=1e-12)


def test_decode_uniform_scores_closed_form(oracle_mod):
    """Q = 0: with no mask every query averages the L cached values (LSE =
    ln L); under the causal mask query i averages keys 0..L-Sq+i."""
    rng = np.random.default_rng(660)
    B, H, Sq, S_cap = 3, 2, 4, 30
    q = np.zeros((B, H, Sq, 8))
    k, v = rnd(rng, B, H, S_cap, 8), rnd(rng, B, H, S_cap, 5)
    seqlens = np.array([30, 17, 6], np.int32)
    o, lse = oracle_mod.decode(q, k, v, seqlens)
    oc, lc = oracle_mod.decode(q, k, v, seqlens, variant="causal")
    for b, L in enumerate(seqlens):
        assert_close(o[b], np.broadcast_to(v[b, :, :L].mean(1)[:, None], o[b].shape),
                                   atol=1e-12)
        assert_close(lse[b], math.log(L), atol=1e-12)
        for i in range(Sq):
            n = L - Sq + i + 1
            assert_close(oc[b, :, i], v[b, :, :n].mean(1), atol=1e-12)
            assert_close(lc[b, :, i], math.log(n), atol=1e-12)


def test_decode_degenerate_lengths(oracle_mod):
    """An empty cache gives O = 0 and LSE = -inf; with fewer cached tokens
    than queries, the causal rows that sit before position 0 see nothing,
    while unmasked rows still see every cached token; lengths past the cache
    are clamped to it."""
    rng = np.random.default_rng(670)
    q, k, v = rnd(rng, 3, 2, 4, 8), rnd(rng, 3, 2, 10, 8), rnd(rng, 3, 2, 10, 3)
    seqlens = np.array([0, 2, 99], np.int32)
    o, lse = oracle_mod.decode(q, k, v, seqlens, variant="causal")
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    assert (o[1, :, :2] == 0).all() and np.isneginf(lse[1, :, :2]).all()  # positions -2, -1
    assert np.isfinite(lse[1, :, 2:]).all()
    ov, lv = oracle_mod.decode(q, k, v, seqlens)
    assert np.isfinite(lv[1]).all()
    o10, l10 = oracle_mod.decode(q, k, v, np.array([0, 2, 10], np.int32), variant="causal")
    np.testing.assert_array_equal(o[2], o10[2])
    np.testing.assert_array_equal(lse[2], l10[2])


def test_decode_online_twin(oracle_mod):
    rng = np.random.default_rng(680)
    q, k, v = rnd(rng, 2, 4, 3, 8, scale=3.0), rnd(rng, 2, 2, 50, 8), rnd(rng, 2, 2, 50, 4)
    seqlens = np.array([50, 31], np.int32)
    for kw in (dict(variant="softcap", softcap=2.0, mask="causal"), dict(variant="alibi")):
        o2, l2 = oracle_mod.decode(q, k, v, seqlens, **kw)
        o1, l1 = oracle_mod.decode(q, k, v, seqlens, block_keys=7, **kw)
        assert_close(o1, o2, rtol=1e-12, atol=1e-13)
        assert_close(l1, l2, rtol=1e-12, atol=1e-13)


def test_decode_rejects_bad_arguments(oracle_mod):
    q = np.zeros((1, 1, 1, 4))
    k = v = np.zeros((1, 1, 4, 4))
    L = np.array([4], np.int32)
    with pytest.raises(ValueError):
        oracle_mod.decode(q, k, v, L, variant="document")
    with pytest.raises(ValueError):
        oracle_mod.decode(q, k, v, L, variant="causal", mask="prefix_lm")
    with pytest.raises(ValueError):
        oracle_mod.decode(q, k, v, L, variant="vanilla", mask="document")


# --------------------------------------------------------------------------
# merge of partial results


@pytest.mark.parametrize("cuts", [(13,), (1, 2, 29), (10, 20)])
def test_merge_recombines_key_parts(oracle_mod, cuts):
    """Attention over disjoint key chunks, merged, is attention over all keys."""
    rng = np.random.default_rng(700 + len(cuts))
    q, k, v = rnd(rng, 2, 3, 5, 8, scale=2.0), rnd(rng, 2, 3, 30, 8), rnd(rng, 2, 3, 30, 7)
    o, lse = oracle_mod.attn(q, k, v, variant="softcap", softcap=3.0)
    edges = (0,) + cuts + (30,)
    parts = [oracle_mod.attn(q, k[:, :, a:b], v[:, :, a:b], variant="softcap", softcap=3.0)
             for a, b in zip(edges[:-1], edges[1:])]
    om, lm = oracle_mod.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert_close(om, o, atol=1e-12)
    assert_close(lm, lse, atol=1e-12)
    # the order of the parts does not matter
    om2, lm2 = oracle_mod.merge(np.stack([p[0] for p in parts[::-1]]),
                                np.stack([p[1] for p in parts[::-1]]))
    assert_close(om2, om, atol=1e-13)
    assert_close(lm2, lm, atol=1e-13)


def test_merge_identities(oracle_mod):
    rng = np.random.default_rng(710)
    o1, o2 = rnd(rng, 6, 4), rnd(rng, 6, 4)
    l1 = rnd(rng, 6)
    # one part: unchanged
    om, lm = oracle_mod.merge(o1[None], l1[None])
    assert_close(om, o1, atol=1e-15)
    assert_close(lm, l1, atol=1e-15)
    # equal LSE: the plain average, LSE + ln 2
    om, lm = oracle_mod.merge(np.stack([o1, o2]), np.stack([l1, l1]))
    assert_close(om, (o1 + o2) / 2, atol=1e-14)
    assert_close(lm, l1 + math.log(2), atol=1e-14)
    # an empty part (LSE = -inf, O = 0) weighs nothing
    ninf = np.full(6, -np.inf)
    om, lm = oracle_mod.merge(np.stack([o1, np.zeros_like(o1)]), np.stack([l1, ninf]))
    assert_close(om, o1, atol=1e-15)
    assert_close(lm, l1, atol=1e-15)
    # every part empty: O = 0, LSE = -inf
    om, lm = oracle_mod.merge(np.zeros((3, 6, 4)), np.full((3, 6), -np.inf))
    assert (om == 0).all() and np.isneginf(lm).all()
    # weights e^(l_p - L) for a worked pair: l = (0, ln 3) gives (1/4, 3/4)
    om, lm = oracle_mod.merge(np.stack([o1, o2]), np.stack([np.zeros(6), np.full(6, math.log(3))]))
    assert_close(om, 0.25 * o1 + 0.75 * o2, atol=1e-14)
    assert_close(lm, math.log(4), atol=1e-14)
