"""Pins of the CPU oracle against things other than itself.

Each test fixes part of the oracle by brute force on tiny inputs, a library
routine it reduces to (torch's scaled_dot_product_attention in float64 on the
CPU), a closed form, or an invariant of softmax attention, chosen so that a
dropped term, a wrong sign, an off-by-one mask or a transposed operand fails
at least one of them.  No GPU needed.
"""
import functools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from tests import _bruteforce as bf

# absolute tolerances only: numpy's default rtol of 1e-7 would hide small relative errors
assert_close = functools.partial(np.testing.assert_allclose, rtol=0)

VARIANTS = ("vanilla", "alibi", "softcap", "causal", "sliding_window", "prefix_lm", "document")


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def docs_for(rng, B, S, n):
    out = []
    for _ in range(B):
        n_eff = min(n, S)
        cuts = np.sort(rng.choice(np.arange(1, S), size=n_eff - 1, replace=False)) if n_eff > 1 else []
        out.append(np.concatenate([[0], cuts, [S]]).astype(np.int32))
    return np.stack(out)


def kw_for(variant, S, rng, B=1):
    kw = dict(variant=variant)
    if variant == "sliding_window":
        kw.update(window=3, window_causal=True)
    if variant == "prefix_lm":
        kw.update(prefix=min(4, S))
    if variant == "softcap":
        kw.update(softcap=1.5)
    if variant == "alibi":
        kw.update(alibi_max_bias=8.0)
    if variant == "document":
        kw.update(doc_offsets=docs_for(rng, B, S, 3))
    return kw


# --------------------------------------------------------------------------
# brute force on tiny inputs


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("S", [1, 5, 33])
def test_matches_bruteforce(oracle_mod, variant, S):
    rng = np.random.default_rng(100 + S)
    B, Hq, Hkv, D, Dv = 2, 4, 2, 8, 6
    q, k, v = rnd(rng, B, Hq, S, D, scale=2.0), rnd(rng, B, Hkv, S, D), rnd(rng, B, Hkv, S, Dv)
    kw = kw_for(variant, S, rng, B)
    o, lse = oracle_mod.attn(q, k, v, **kw)
    o_bf, lse_bf = bf.attention(q, k, v, **kw)
    assert_close(o, o_bf, rtol=0, atol=1e-12)
    assert_close(lse, lse_bf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window_causal", [True, False])
@pytest.mark.parametrize("window", [1, 2, 7, 40])
def test_window_bruteforce(oracle_mod, window, window_causal):
    rng = np.random.default_rng(7 * window + window_causal)
    q, k, v = rnd(rng, 1, 2, 21, 4), rnd(rng, 1, 2, 21, 4), rnd(rng, 1, 2, 21, 4)
    kw = dict(variant="sliding_window", window=window, window_causal=window_causal)
    o, lse = oracle_mod.attn(q, k, v, **kw)
    o_bf, lse_bf = bf.attention(q, k, v, **kw)
    assert_close(o, o_bf, atol=1e-12)
    assert_close(lse, lse_bf, atol=1e-12)


def test_bias_bruteforce(oracle_mod):
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 2, 3, 9, 5), rnd(rng, 2, 3, 11, 5), rnd(rng, 2, 3, 11, 4)
    bias = rnd(rng, 3, 9, 11)
    o, lse = oracle_mod.attn(q, k, v, bias=bias, scale=0.7)
    o_bf, lse_bf = bf.attention(q, k, v, bias=bias, scale=0.7)
    assert_close(o, o_bf, atol=1e-12)
    assert_close(lse, lse_bf, atol=1e-12)


# --------------------------------------------------------------------------
# reduction to a library routine: torch scaled_dot_product_attention, float64


def sdpa(q, k, v, **kw):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), **kw).numpy()


def test_vanilla_equals_sdpa(oracle_mod):
    rng = np.random.default_rng(11)
    q, k, v = rnd(rng, 2, 3, 17, 16), rnd(rng, 2, 3, 23, 16), rnd(rng, 2, 3, 23, 16)
    o, _ = oracle_mod.attn(q, k, v, scale=0.3)
    assert_close(o, sdpa(q, k, v, scale=0.3), atol=1e-12)


def test_causal_equals_sdpa(oracle_mod):
    rng = np.random.default_rng(12)
    q, k, v = rnd(rng, 1, 2, 31, 8), rnd(rng, 1, 2, 31, 8), rnd(rng, 1, 2, 31, 8)
    o, _ = oracle_mod.attn(q, k, v, variant="causal")
    assert_close(o, sdpa(q, k, v, is_causal=True), atol=1e-12)


def test_gqa_equals_sdpa(oracle_mod):
    rng = np.random.default_rng(13)
    q, k, v = rnd(rng, 2, 8, 13, 8), rnd(rng, 2, 2, 13, 8), rnd(rng, 2, 2, 13, 8)
    o, _ = oracle_mod.attn(q, k, v, variant="causal")
    assert_close(o, sdpa(q, k, v, is_causal=True, enable_gqa=True), atol=1e-12)


def test_bias_equals_sdpa_float_mask(oracle_mod):
    rng = np.random.default_rng(14)
    q, k, v = rnd(rng, 2, 2, 10, 8), rnd(rng, 2, 2, 12, 8), rnd(rng, 2, 2, 12, 8)
    bias = rnd(rng, 2, 10, 12, scale=3.0)
    o, _ = oracle_mod.attn(q, k, v, bias=bias)
    ref = sdpa(q, k, v, attn_mask=torch.from_numpy(bias)[None])
    assert_close(o, ref, atol=1e-12)


# --------------------------------------------------------------------------
# the single-pass online algorithm equals two-pass softmax (the homomorphism)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("block", [1, 7, 64])
def test_online_twin_equals_two_pass(oracle_mod, variant, block):
    rng = np.random.default_rng(200 + block)
    S = 45
    q, k, v = rnd(rng, 1, 2, S, 8, scale=3.0), rnd(rng, 1, 2, S, 8), rnd(rng, 1, 2, S, 8)
    kw = kw_for(variant, S, rng)
    o2, l2 = oracle_mod.attn(q, k, v, **kw)
    o1, l1 = oracle_mod.attn(q, k, v, block_keys=block, **kw)
    assert_close(o1, o2, rtol=1e-12, atol=1e-13)
    assert_close(l1, l2, rtol=1e-12, atol=1e-13)


def test_merge_of_key_halves(oracle_mod):
    """(O, LSE) of two disjoint key halves merge to the whole row."""
    rng = np.random.default_rng(21)
    q, k, v = rnd(rng, 1, 2, 9, 8), rnd(rng, 1, 2, 30, 8), rnd(rng, 1, 2, 30, 5)
    o, l = oracle_mod.attn(q, k, v)
    oa, la = oracle_mod.attn(q, k[:, :, :13], v[:, :, :13])
    ob, lb = oracle_mod.attn(q, k[:, :, 13:], v[:, :, 13:])
    lm = np.logaddexp(la, lb)
    om = np.exp(la - lm)[..., None] * oa + np.exp(lb - lm)[..., None] * ob
    assert_close(lm, l, atol=1e-12)
    assert_close(om, o, atol=1e-12)


# --------------------------------------------------------------------------
# normalisation invariants


@pytest.mark.parametrize("variant", VARIANTS)
def test_probability_rows(oracle_mod, variant):
    """With V = identity the output is the probability matrix: rows are >= 0
    and sum to 1; masked keys get exactly 0."""
    rng = np.random.default_rng(31)
    S = 24
    q, k = rnd(rng, 1, 2, S, 8, scale=2.0), rnd(rng, 1, 2, S, 8)
    v = np.broadcast_to(np.eye(S), (1, 2, S, S)).copy()
    kw = kw_for(variant, S, rng)
    p, _ = oracle_mod.attn(q, k, v, **kw)
    assert (p >= 0).all()
    assert_close(p.sum(-1), 1.0, atol=1e-12)
    allowed = bf.mask_matrix(variant, S, S, window=kw.get("window", 1), prefix=kw.get("prefix", 0),
                             offsets=None if variant != "document" else kw["doc_offsets"][0])
    assert (p[0, :, ~allowed] == 0).all()


@pytest.mark.parametrize("variant", VARIANTS)
def test_convex_hull(oracle_mod, variant):
    rng = np.random.default_rng(32)
    S = 30
    q, k, v = rnd(rng, 1, 1, S, 8, scale=2.0), rnd(rng, 1, 1, S, 8), rnd(rng, 1, 1, S, 6)
    kw = kw_for(variant, S, rng)
    o, _ = oracle_mod.attn(q, k, v, **kw)
    allowed = bf.mask_matrix(variant, S, S, window=kw.get("window", 1), prefix=kw.get("prefix", 0),
                             offsets=None if variant != "document" else kw["doc_offsets"][0])
    for i in range(S):
        vv = v[0, 0][allowed[i]]
        assert (o[0, 0, i] >= vv.min(0) - 1e-12).all() and (o[0, 0, i] <= vv.max(0) + 1e-12).all()


# --------------------------------------------------------------------------
# closed forms


@pytest.mark.parametrize("variant", ["vanilla", "causal", "sliding_window", "prefix_lm", "document"])
def test_uniform_scores_give_mean_of_allowed_values(oracle_mod, variant):
    """Q = 0 makes every score equal: O_i is the mean of v over the keys row i
    may see and LSE_i = ln(number of such keys)."""
    rng = np.random.default_rng(41)
    S = 40
    q, k, v = np.zeros((1, 1, S, 8)), rnd(rng, 1, 1, S, 8), rnd(rng, 1, 1, S, 3)
    kw = dict(variant=variant)
    i = np.arange(S)
    if variant == "vanilla":
        lo, hi = np.zeros(S, int), np.full(S, S - 1)
    elif variant == "causal":
        lo, hi = np.zeros(S, int), i
    elif variant == "sliding_window":
        kw.update(window=5, window_causal=True)
        lo, hi = np.maximum(0, i - 4), i
    elif variant == "prefix_lm":
        kw.update(prefix=11)
        lo, hi = np.zeros(S, int), np.maximum(i, 10)
    else:
        offs = np.array([[0, 3, 4, 20, 40]], np.int32)
        kw.update(doc_offsets=offs)
        d = np.searchsorted(offs[0], i, side="right") - 1
        lo, hi = offs[0][d], offs[0][d + 1] - 1
    o, lse = oracle_mod.attn(q, k, v, **kw)
    csum = np.concatenate([np.zeros((1, 3)), np.cumsum(v[0, 0], 0)])
    mean = (csum[hi + 1] - csum[lo]) / (hi - lo + 1)[:, None]
    assert_close(o[0, 0], mean, atol=1e-12)
    assert_close(lse[0, 0], np.log(hi - lo + 1), atol=1e-12)


def test_window_one_returns_own_value(oracle_mod):
    rng = np.random.default_rng(42)
    q, k, v = rnd(rng, 1, 2, 19, 8), rnd(rng, 1, 2, 19, 8), rnd(rng, 1, 2, 19, 4)
    for causal in (True, False):
        o, lse = oracle_mod.attn(q, k, v, variant="sliding_window", window=1, window_causal=causal)
        assert_close(o, v, atol=1e-14)


def test_unit_documents_return_own_value(oracle_mod):
    rng = np.random.default_rng(43)
    S = 12
    q, k, v = rnd(rng, 2, 1, S, 8), rnd(rng, 2, 1, S, 8), rnd(rng, 2, 1, S, 4)
    offs = np.tile(np.arange(S + 1, dtype=np.int32), (2, 1))
    o, _ = oracle_mod.attn(q, k, v, variant="document", doc_offsets=offs)
    assert_close(o, v, atol=1e-14)


def test_mask_algebra(oracle_mod):
    rng = np.random.default_rng(44)
    S = 26
    q, k, v = rnd(rng, 1, 2, S, 8, scale=2), rnd(rng, 1, 2, S, 8), rnd(rng, 1, 2, S, 4)
    A = lambda **kw: oracle_mod.attn(q, k, v, **kw)[0]
    van, cau = A(variant="vanilla"), A(variant="causal")
    assert_close(A(variant="sliding_window", window=S, window_causal=False), van, atol=1e-13)
    assert_close(A(variant="sliding_window", window=S + 5, window_causal=True), cau, atol=1e-13)
    assert_close(A(variant="prefix_lm", prefix=0), cau, atol=1e-13)
    assert_close(A(variant="prefix_lm", prefix=1), cau, atol=1e-13)
    assert_close(A(variant="prefix_lm", prefix=S), van, atol=1e-13)
    assert_close(A(variant="document", doc_offsets=np.array([[0, S]], np.int32)), van,
                               atol=1e-13)
    # a window that is too small must differ from causal
    assert np.abs(A(variant="sliding_window", window=S - 1, window_causal=True) - cau).max() > 1e-6


# --------------------------------------------------------------------------
# score modifications


def test_alibi_slopes_fixture():
    """ALiBi's geometric head slopes for 8 heads are 1/2, 1/4, ..., 1/256."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "alibi_slopes_h8.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    want = {int(h): float(s) for h, s in rows}
    assert want == {h: 2.0 ** -(h + 1) for h in range(8)}


def test_alibi_geometric_closed_form(oracle_mod):
    """Q = 0 and V = identity: the weights of row i are r^|i-j| / sum_j r^|i-j|
    with r = e^-slope; both sums are finite geometric series."""
    S, H = 15, 4
    q, k = np.zeros((1, H, S, 4)), np.ones((1, H, S, 4))
    v = np.broadcast_to(np.eye(S), (1, H, S, S)).copy()
    p, lse = oracle_mod.attn(q, k, v, variant="alibi", alibi_max_bias=8.0)
    for h in range(H):
        r = math.exp(-(2.0 ** (-8.0 * (h + 1) / H)))
        for i in range(S):
            left = (1 - r ** (i + 1)) / (1 - r)             # j = i, i-1, ..., 0
            right = r * (1 - r ** (S - 1 - i)) / (1 - r)    # j = i+1, ..., S-1
            z = left + right
            for j in (0, i, S - 1):
                assert abs(p[0, h, i, j] - r ** abs(i - j) / z) < 1e-13
            assert abs(lse[0, h, i] - math.log(z)) < 1e-12


def test_alibi_vanishing_slopes_is_vanilla(oracle_mod):
    """A huge max_bias drives every slope 2^(-max_bias*(h+1)/H) to ~0."""
    rng = np.random.default_rng(51)
    q, k, v = rnd(rng, 1, 3, 14, 8), rnd(rng, 1, 3, 14, 8), rnd(rng, 1, 3, 14, 8)
    assert_close(oracle_mod.attn(q, k, v, variant="alibi", alibi_max_bias=3000.0)[0],
                               oracle_mod.attn(q, k, v)[0], atol=1e-13)
    # max_bias = 0 gives slope 1 on every head, which is not vanilla
    assert np.abs(oracle_mod.attn(q, k, v, variant="alibi", alibi_max_bias=0.0)[0]
                  - oracle_mod.attn(q, k, v)[0]).max() > 1e-3


def test_alibi_on_causal_side_equals_sdpa_bias(oracle_mod):
    """On j <= i the symmetric distance penalty equals the causal ALiBi bias
    slope*(j-i): compare the causal half through sdpa with that float mask."""
    rng = np.random.default_rng(52)
    S, H = 12, 4
    q, k = rnd(rng, 1, H, S, 8), rnd(rng, 1, H, S, 8)
    v = np.broadcast_to(np.eye(S), (1, H, S, S)).copy()
    p, _ = oracle_mod.attn(q, k, v, variant="alibi")
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    slopes = 2.0 ** (-8.0 * (np.arange(H) + 1) / H)
    bias = np.where(j <= i, slopes[:, None, None] * (j - i), -np.inf)
    pc = sdpa(q, k, v, attn_mask=torch.from_numpy(bias)[None])
    # restrict both to the causal half and renormalise
    pn = np.where(j <= i, p, 0.0)
    pn = pn / pn.sum(-1, keepdims=True)
    assert_close(pn, pc, atol=1e-12)


def test_softcap_large_cap_is_vanilla(oracle_mod):
    rng = np.random.default_rng(61)
    q, k, v = rnd(rng, 1, 2, 16, 8), rnd(rng, 1, 2, 16, 8), rnd(rng, 1, 2, 16, 8)
    assert_close(oracle_mod.attn(q, k, v, variant="softcap", softcap=1e6)[0],
                               oracle_mod.attn(q, k, v)[0], atol=1e-9)


def test_softcap_bounds_score_spread(oracle_mod):
    """|score| <= cap, so any two log-probabilities differ by at most 2*cap;
    with sharpened Q the uncapped spread is far larger."""
    rng = np.random.default_rng(62)
    S = 20
    q, k = rnd(rng, 1, 1, S, 8, scale=8.0), rnd(rng, 1, 1, S, 8)
    v = np.eye(S)[None, None]
    for cap in (1.0, 2.0):
        p, _ = oracle_mod.attn(q, k, v, variant="softcap", softcap=cap)
        lp = np.log(p[0, 0])
        assert (lp.max(-1) - lp.min(-1) <= 2 * cap + 1e-12).all()
    p, _ = oracle_mod.attn(q, k, v)
    lp = np.log(p[0, 0])
    assert (lp.max(-1) - lp.min(-1)).max() > 10.0


# --------------------------------------------------------------------------
# head mapping and linear structure


def test_gqa_equals_repeated_mha(oracle_mod):
    rng = np.random.default_rng(71)
    q, k, v = rnd(rng, 2, 6, 9, 8), rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 2, 9, 5)
    for variant in ("vanilla", "causal", "alibi"):
        og, lg = oracle_mod.attn(q, k, v, variant=variant)
        om, lm = oracle_mod.attn(q, np.repeat(k, 3, 1), np.repeat(v, 3, 1), variant=variant)
        assert_close(og, om, atol=1e-14)
        assert_close(lg, lm, atol=1e-14)


def test_linear_in_v_and_key_permutation(oracle_mod):
    rng = np.random.default_rng(72)
    q, k = rnd(rng, 1, 2, 11, 8), rnd(rng, 1, 2, 13, 8)
    v1, v2 = rnd(rng, 1, 2, 13, 4), rnd(rng, 1, 2, 13, 4)
    o1, _ = oracle_mod.attn(q, k, v1)
    o2, _ = oracle_mod.attn(q, k, v2)
    o3, _ = oracle_mod.attn(q, k, 2.0 * v1 - 3.0 * v2)
    assert_close(o3, 2.0 * o1 - 3.0 * o2, atol=1e-12)
    perm = rng.permutation(13)
    op, _ = oracle_mod.attn(q, k[:, :, perm], v1[:, :, perm])
    assert_close(op, o1, atol=1e-13)


def test_fully_masked_rows(oracle_mod):
    """A -inf bias row leaves no key: O = 0 and LSE = -inf (explicit convention)."""
    rng = np.random.default_rng(73)
    q, k, v = rnd(rng, 1, 1, 6, 4), rnd(rng, 1, 1, 6, 4), rnd(rng, 1, 1, 6, 4)
    bias = np.zeros((1, 6, 6))
    bias[0, 2, :] = -np.inf
    o, lse = oracle_mod.attn(q, k, v, bias=bias)
    assert (o[0, 0, 2] == 0).all() and lse[0, 0, 2] == -np.inf
    assert np.isfinite(o).all() and np.isfinite(np.delete(lse[0, 0], 2)).all()
    o1, lse1 = oracle_mod.attn(q, k, v, bias=bias, block_keys=2)
    assert_close(o1, o, atol=1e-13)
    assert lse1[0, 0, 2] == -np.inf


def test_row_sampling_matches_full(oracle_mod):
    rng = np.random.default_rng(74)
    q, k, v = rnd(rng, 2, 4, 9, 8), rnd(rng, 2, 2, 9, 8), rnd(rng, 2, 2, 9, 3)
    o, lse = oracle_mod.attn(q, k, v, variant="causal")
    rows = np.array([0, 5, 17, 71, 40])
    os_, ls = oracle_mod.attn(q, k, v, variant="causal", rows=rows)
    assert_close(os_, o.reshape(-1, 3)[rows], atol=0)
    assert_close(ls, lse.reshape(-1)[rows], atol=0)


def test_rejects_bad_arguments(oracle_mod):
    q = np.zeros((1, 3, 4, 4))
    k = np.zeros((1, 2, 4, 4))
    with pytest.raises(ValueError):
        oracle_mod.attn(q, k, k)  # H_q not a multiple of H_kv
    q = np.zeros((1, 2, 4, 4))
    with pytest.raises(ValueError):
        oracle_mod.attn(q, k, k, rows=[99])


# --------------------------------------------------------------------------
# differential attention


def test_diffattn_pins(oracle_mod):
    rng = np.random.default_rng(81)
    B, H, S, D, Dv = 1, 2, 17, 8, 12
    q1, q2, k1, k2 = (rnd(rng, B, H, S, D) for _ in range(4))
    v = rnd(rng, B, H, S, Dv)
    for causal in (False, True):
        o, l1, l2 = oracle_mod.diffattn(q1, q2, k1, k2, v, lam=0.8, causal=causal, scale=0.125)
        ref = sdpa(q1, k1, v, scale=0.125, is_causal=causal) - 0.8 * sdpa(q2, k2, v, scale=0.125,
                                                                           is_causal=causal)
        assert_close(o, ref, atol=1e-12)
        # lambda = 0 is vanilla attention of the first stream
        o0, _, _ = oracle_mod.diffattn(q1, q2, k1, k2, v, lam=0.0, causal=causal, scale=0.125)
        assert_close(o0, sdpa(q1, k1, v, scale=0.125, is_causal=causal), atol=1e-12)
        # identical streams with lambda = 1 cancel exactly
        oz, _, _ = oracle_mod.diffattn(q1, q1, k1, k1, v, lam=1.0, causal=causal, scale=0.125)
        assert np.abs(oz).max() == 0.0
        # per-stream LSE equals the vanilla oracle's
        _, lv = oracle_mod.attn(q2, k2, v, variant="causal" if causal else "vanilla", scale=0.125)
        assert_close(l2, lv, atol=1e-14)


# --------------------------------------------------------------------------
# Evoformer gated self-attention


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def evo_sdpa_row(q, k, v, gate, bias, key_mask):
    """Row attention through torch sdpa: [N,L,H,C] -> heads first."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))  # [N,H,L,C]
    N, L, H, C = q.shape
    mask = np.zeros((N, 1, L, L))
    if bias is not None:
        mask = mask + bias[None]
    if key_mask is not None:
        mask = np.where(key_mask[:, None, None, :] != 0, mask, -np.inf)
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)).numpy()
    return o.transpose(0, 2, 1, 3) * sigmoid(gate)


def evo_inputs(rng, N, L, H, C):
    q, k, v, g = (rnd(rng, N, L, H, C) for _ in range(4))
    bias = rnd(rng, H, L, L)
    km = (rng.random((N, L)) >= 0.2).astype(np.uint8)
    km[:, 0] = 1  # keep every row non-empty for the sdpa comparison
    return q, k, v, g, bias, km


def test_evoformer_row_equals_sdpa(oracle_mod):
    rng = np.random.default_rng(91)
    q, k, v, g, bias, km = evo_inputs(rng, 3, 10, 2, 4)
    o = oracle_mod.evoformer(q, k, v, g, pair_bias=bias, key_mask=km)
    assert_close(o, evo_sdpa_row(q, k, v, g, bias, km), atol=1e-12)


def test_evoformer_col_equals_row_on_transposed(oracle_mod):
    rng = np.random.default_rng(92)
    q, k, v, g, _, km = evo_inputs(rng, 7, 5, 2, 4)
    km[0, :] = 1
    o = oracle_mod.evoformer(q, k, v, g, key_mask=km, axis="col")
    T = lambda a: a.transpose(1, 0, 2, 3)
    ref = T(evo_sdpa_row(T(q), T(k), T(v), T(g), None, km.T))
    assert_close(o, ref, atol=1e-12)


def test_evoformer_special_cases(oracle_mod):
    rng = np.random.default_rng(93)
    N, L, H, C = 2, 9, 3, 4
    q, k, v, g, bias, km = evo_inputs(rng, N, L, H, C)
    # no bias, no mask, sigmoid(+40) = 1: plain attention with scale 1/sqrt(C)
    o = oracle_mod.evoformer(q, k, v, np.full_like(g, 40.0))
    assert_close(o, evo_sdpa_row(q, k, v, np.full_like(g, 40.0), None, None), atol=1e-12)
    t = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    plain = sdpa(t(q), t(k), t(v)).transpose(0, 2, 1, 3)
    assert_close(o, plain * sigmoid(40.0), atol=1e-12)
    # G = 0 halves the output
    o0 = oracle_mod.evoformer(q, k, v, np.zeros_like(g))
    assert_close(o0, plain / 2, atol=1e-12)
    # a bias constant along the key axis changes nothing
    row_const = np.broadcast_to(rnd(rng, H, L, 1) * 5, (H, L, L)).copy()
    oc = oracle_mod.evoformer(q, k, v, g, pair_bias=row_const)
    assert_close(oc, oracle_mod.evoformer(q, k, v, g), atol=1e-12)
    # a single unmasked key returns sigmoid(G) * v_j
    one = np.zeros((N, L), np.uint8)
    one[:, 4] = 1
    o1 = oracle_mod.evoformer(q, k, v, g, pair_bias=bias, key_mask=one)
    assert_close(o1, sigmoid(g) * v[:, 4:5, :, :], atol=1e-14)
    # every key masked: the row is 0
    none = np.zeros((N, L), np.uint8)
    assert np.abs(oracle_mod.evoformer(q, k, v, g, pair_bias=bias, key_mask=none)).max() == 0.0


# --------------------------------------------------------------------------
# composed variants: a score modification under a mask

MODS = ("vanilla", "alibi", "softcap")
MASKS = ("causal", "sliding_window", "prefix_lm", "document")


def compose_kw(mod, mask, S, rng, B):
    kw = dict(variant=mod, mask=mask)
    kw.update({k: v for k, v in kw_for(mask, S, rng, B).items() if k != "variant"})
    if mod == "softcap":
        kw.update(softcap=1.5)  # small, so the cap matters
    if mod == "alibi":
        kw.update(alibi_max_bias=8.0)
    return kw


@pytest.mark.parametrize("mod", MODS)
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("S", [5, 33])
def test_composed_matches_bruteforce(oracle_mod, mod, mask, S):
    rng = np.random.default_rng(200 + S + 7 * MASKS.index(mask) + 31 * MODS.index(mod))
    B, Hq, Hkv, D, Dv = 2, 4, 2, 8, 6
    q, k, v = rnd(rng, B, Hq, S, D, scale=2.0), rnd(rng, B, Hkv, S, D), rnd(rng, B, Hkv, S, Dv)
    kw = compose_kw(mod, mask, S, rng, B)
    o, lse = oracle_mod.attn(q, k, v, **kw)
    o_bf, lse_bf = bf.attention(q, k, v, **kw)
    assert_close(o, o_bf, rtol=0, atol=1e-12)
    assert_close(lse, lse_bf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mask", MASKS)
def test_composed_special_cases(oracle_mod, mask):
    """vanilla under a mask is that mask's variant; softcap with a huge cap
    under a mask is the mask alone."""
    rng = np.random.default_rng(300 + MASKS.index(mask))
    B, S = 2, 24
    q, k, v = rnd(rng, B, 2, S, 8), rnd(rng, B, 2, S, 8), rnd(rng, B, 2, S, 5)
    kw = {k_: v_ for k_, v_ in kw_for(mask, S, rng, B).items() if k_ != "variant"}
    plain = oracle_mod.attn(q, k, v, variant=mask, **kw)
    same = oracle_mod.attn(q, k, v, variant="vanilla", mask=mask, **kw)
    np.testing.assert_array_equal(plain[0], same[0])
    big = oracle_mod.attn(q, k, v, variant="softcap", softcap=1e7, mask=mask, **kw)
    assert_close(big[0], plain[0], atol=1e-9)


def test_alibi_under_causal_equals_sdpa_bias(oracle_mod):
    """ALiBi composed with the causal mask is softmax(qk/sqrt(d) + slope*(j-i))
    over j <= i: SDPA in float64 with that additive float mask."""
    rng = np.random.default_rng(310)
    S, H = 17, 4
    q, k, v = rnd(rng, 1, H, S, 8), rnd(rng, 1, H, S, 8), rnd(rng, 1, H, S, 6)
    o, _ = oracle_mod.attn(q, k, v, variant="alibi", mask="causal")
    i, j = np.arange(S)[:, None], np.arange(S)[None, :]
    slopes = 2.0 ** (-8.0 * (np.arange(H) + 1) / H)
    bias = np.where(j <= i, slopes[:, None, None] * (j - i), -np.inf)
    assert_close(o, sdpa(q, k, v, attn_mask=torch.from_numpy(bias)[None]), atol=1e-12)


def test_alibi_causal_uniform_scores_closed_form(oracle_mod):
    """Q = 0 under ALiBi and the causal mask: row i weights key j <= i by
    r^(i-j) with r = e^(-slope), so O_i = sum r^(i-j) v_j / sum r^(i-j)."""
    S, H = 40, 2
    q = np.zeros((1, H, S, 4))
    k = np.ones((1, H, S, 4))
    v = np.random.default_rng(311).standard_normal((1, H, S, 3))
    o, lse = oracle_mod.attn(q, k, v, variant="alibi", mask="causal", alibi_max_bias=3.0)
    for h in range(H):
        r = math.exp(-(2.0 ** (-3.0 * (h + 1) / H)))
        for i in (0, 1, 7, S - 1):
            w = r ** (i - np.arange(i + 1))
            assert_close(o[0, h, i], w @ v[0, h, : i + 1] / w.sum(), atol=1e-12)
            assert abs(lse[0, h, i] - math.log(w.sum())) < 1e-12


def test_composed_rejects_bad_arguments(oracle_mod):
    rng = np.random.default_rng(312)
    q = k = v = rnd(rng, 1, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle_mod.attn(q, k, v, variant="causal", mask="prefix_lm")  # a mask variant takes no mask
    with pytest.raises(ValueError):
        oracle_mod.attn(q, k, v, variant="alibi", mask="softcap")  # not a mask
    with pytest.raises(ValueError):
        oracle_mod.attn(q, k, v, variant="softcap", mask="sliding_window", window=0)
