"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small problems are compared element by element on every output; the full
workload sizes are compared on sampled rows the oracle computes one by one.
Every input is seeded and synthetic (flashattention_attention_variants_amd.inputs).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, gpu_rows, np64, sample_rows

pytestmark = pytest.mark.gpu

VARIANTS = inputs.ALL_MASK_VARIANTS
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def variant_kw(variant, S, B, seed, window=37, prefix=50, n_docs=5, window_causal=True):
    kw = dict(variant=variant)
    if variant == "sliding_window":
        kw.update(window=window, window_causal=window_causal)
    elif variant == "prefix_lm":
        kw.update(prefix=prefix)
    elif variant == "softcap":
        kw.update(softcap=50.0)
    elif variant == "alibi":
        kw.update(alibi_max_bias=8.0)
    elif variant == "document":
        kw.update(doc_offsets=inputs.doc_offsets(B, S, min(n_docs, S), seed))
    return kw


def run_gpu_attn(q, k, v, bias=None, **kw):
    kw = dict(kw)
    docs = kw.pop("doc_offsets", None)
    o, lse = api.fl_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                             bias=None if bias is None else bias.to(DEV),
                             doc_offsets=None if docs is None else docs.to(DEV),
                             return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def run_oracle_attn(q, k, v, bias=None, rows=None, **kw):
    kw = dict(kw)
    docs = kw.pop("doc_offsets", None)
    return oracle.attn(np64(q), np64(k), np64(v), bias=None if bias is None else np64(bias),
                       doc_offsets=None if docs is None else docs.numpy(), rows=rows, **kw)


# ---------------------------------------------------------------------------
# float32: the 128-token MHA workload (with LSE) and every variant


def test_f32_mha_s128_with_lse():
    wl = inputs.WORKLOADS["mha_f32_b1_h2_s128_d64"]
    t = inputs.make(wl)
    o, lse = run_gpu_attn(t["q"], t["k"], t["v"])
    ro, rl = run_oracle_attn(t["q"], t["k"], t["v"])
    check(np64(o), ro, "f32", "O")
    check(np64(lse), rl, "f32", "LSE")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("variant", VARIANTS)
def test_f32_variants(variant, D):
    B, Hq, Hkv, S = 2, 4, 2, 150
    q, k, v = inputs.attn_inputs(B, Hq, Hkv, S, S, D, "f32", seed=11)
    kw = variant_kw(variant, S, B, seed=12)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "f32", variant)
    check(np64(lse), rl, "f32", variant + " lse")


# ---------------------------------------------------------------------------
# bf16: every variant, GQA and MHA, ragged lengths spanning several tiles


@pytest.mark.parametrize("S", [1, 17, 64, 100, 300, 513])
@pytest.mark.parametrize("variant", VARIANTS)
def test_bf16_variants(variant, S):
    B, Hq, Hkv, D = 2, 4, 2, 64
    q, k, v = inputs.attn_inputs(B, Hq, Hkv, S, S, D, "bf16", seed=20 + S)
    kw = variant_kw(variant, S, B, seed=21 + S)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "%s S=%d" % (variant, S))
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "lse %g" % mx


@pytest.mark.parametrize("B,S,n_docs,H", [(3, 1000, 5, 2), (2, 640, 40, 2), (1, 300, 300, 1),
                                          (2, 2048, 2, 8), (52, 520, 3, 1)])
def test_document_work_order(B, S, n_docs, H):
    """Under the document mask the (batch entry, query tile) items go out
    longest first when one work-group can rank them (at most 256 items and
    1024 offsets), else in the plain order: 52 entries of 520 rows are 260
    items and take the plain order, the rest the ranked one, with documents
    of one row each, many short ones, a few long ones and two per entry
    across eight heads.  Every row is compared with the oracle."""
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=400 + S)
    kw = dict(variant="document", doc_offsets=inputs.doc_offsets(B, S, n_docs, seed=401 + S))
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "document B=%d S=%d docs=%d" % (B, S, n_docs))
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "lse %g" % mx


@pytest.mark.parametrize("window_causal", [True, False])
@pytest.mark.parametrize("window", [1, 64, 100, 1000])
def test_bf16_window_shapes(window, window_causal):
    B, H, S = 1, 2, 700
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=window)
    kw = dict(variant="sliding_window", window=window, window_causal=window_causal)
    o, _ = run_gpu_attn(q, k, v, **kw)
    ro, _ = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "window %d" % window)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_bf16_gqa_groups(group):
    B, Hkv, S = 1, 2, 260
    q, k, v = inputs.attn_inputs(B, Hkv * group, Hkv, S, S, 64, "bf16", seed=30 + group)
    for variant in ("vanilla", "causal"):
        o, _ = run_gpu_attn(q, k, v, variant=variant)
        ro, _ = run_oracle_attn(q, k, v, variant=variant)
        check(np64(o), ro, "bf16", "gqa %d %s" % (group, variant))


def test_bf16_cross_lengths():
    """S_q != S_k (vanilla, ALiBi, softcap allow it)."""
    q, _, _ = inputs.attn_inputs(2, 2, 2, 77, 77, 64, "bf16", seed=40)
    _, k, v = inputs.attn_inputs(2, 2, 2, 333, 333, 64, "bf16", seed=41)
    for variant in ("vanilla", "alibi", "softcap"):
        o, lse = run_gpu_attn(q, k, v, variant=variant)
        ro, rl = run_oracle_attn(q, k, v, variant=variant)
        check(np64(o), ro, "bf16", variant)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bias(dtype):
    B, H, S = 2, 3, 136
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, dtype, seed=50)
    bias = inputs.bias_inputs(H, S, S, dtype, seed=51)
    for variant in ("vanilla", "causal", "alibi", "softcap"):
        o, lse = run_gpu_attn(q, k, v, bias=bias, variant=variant)
        ro, rl = run_oracle_attn(q, k, v, bias=bias, variant=variant)
        check(np64(o), ro, dtype, "bias " + variant)


# ---------------------------------------------------------------------------
# discriminating cases: effects large against the tolerance


def test_softcap_small_cap_sharpened():
    """cap = 2 with Q scaled by 4: softcap moves O by far more than the
    tolerance, and the GPU follows the oracle."""
    B, H, S = 1, 4, 256
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=60)
    q = (q.float() * 4).to(torch.bfloat16)
    o, _ = run_gpu_attn(q, k, v, variant="softcap", softcap=2.0)
    ro, _ = run_oracle_attn(q, k, v, variant="softcap", softcap=2.0)
    check(np64(o), ro, "bf16", "softcap 2")
    rv, _ = run_oracle_attn(q, k, v, variant="vanilla")
    assert np.abs(ro - rv).max() > 0.3


@pytest.mark.parametrize("cap", [2.0, 30.0, 60.0, 80.0, 400.0])
@pytest.mark.parametrize("S", [77, 300])
def test_softcap_caps_and_extremes(cap, S):
    """Softcap over a range of caps on both kernel paths (cap log2(e) <= 100
    needs no running reference; larger caps track one), with scores spread
    over several hundred units so that large caps leave them far from 0,
    causal and non-causal, O and LSE against the oracle."""
    B, H = 1, 2
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=65)
    q = (q.float() * 25).to(torch.bfloat16)
    for variant in ("softcap",):
        o, lse = run_gpu_attn(q, k, v, variant=variant, softcap=cap)
        ro, rl = run_oracle_attn(q, k, v, variant=variant, softcap=cap)
        check(np64(o), ro, "bf16", "softcap %g S=%d" % (cap, S))
        assert np.abs(np64(lse) - rl).max() < 2e-2 * max(1.0, np.abs(rl).max() / 64)


@pytest.mark.parametrize("case", ["low", "mixed"])
@pytest.mark.parametrize("causal", [False, True])
def test_softcap_first_pass_fallback(case, causal):
    """cap = 50 (c = cap log2(e) = 72.1): the first pass takes its terms
    relative to 2^c.  Rows whose every score sits near -cap end with sums
    near S_k 2^-2c, below its bound, and their work-group must redo the tile
    walk against the reference 0.  'low' makes every row so, 'mixed' only
    the rows from 150 on (the first work-group's rows pass, the others fall
    back); O and LSE against the oracle."""
    B, H, S, D = 1, 2, 300, 64
    q, k, v = inputs.attn_inputs(B, H, H, S, S, D, "bf16", seed=66)
    u = torch.full((D,), 1.0 / 8.0)  # unit vector
    k = (k.float() * 0.1 + 20 * u).to(torch.bfloat16)
    low = q.float() * 0.1 - 80 * u
    if case == "low":
        q = low.to(torch.bfloat16)
    else:
        q = torch.cat([q.float()[:, :, :150], low[:, :, 150:]], 2).to(torch.bfloat16)
    kw = dict(variant="softcap", softcap=50.0)
    if causal:
        kw["mask"] = "causal"
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "softcap fallback %s causal=%s" % (case, causal))
    assert np.abs(np64(lse) - rl).max() < 2e-2, np.abs(np64(lse) - rl).max()
    assert rl[:, :, 150:].max() < -40  # the low rows really are near -cap


def test_alibi_closed_form_on_gpu():
    """Q = 0, V = identity (S = D = 64): row i of O is r^|i-j| / Z_i."""
    H, S = 8, 64
    q = torch.zeros(1, H, S, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, H, S, 64, dtype=torch.bfloat16)
    v = torch.eye(S, dtype=torch.bfloat16).expand(1, H, S, S).contiguous()
    o, lse = run_gpu_attn(q, k, v, variant="alibi", alibi_max_bias=8.0)
    got = np64(o)[0]
    for h in range(H):
        r = math.exp(-(2.0 ** (-8.0 * (h + 1) / H)))
        i, j = np.arange(S)[:, None], np.arange(S)[None, :]
        w = r ** np.abs(i - j)
        want = w / w.sum(1, keepdims=True)
        assert np.abs(got[h] - want).max() < 4e-3, h


def test_uniform_scores_mean_of_values():
    """Q = 0: causal O_i is the prefix mean of V, LSE_i = ln(i+1)."""
    B, H, S = 1, 2, 333
    _, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=61)
    q = torch.zeros(B, H, S, 64, dtype=torch.bfloat16)
    o, lse = run_gpu_attn(q, k, v, variant="causal")
    vv = np64(v)
    want = np.cumsum(vv, 2) / np.arange(1, S + 1)[None, None, :, None]
    check(np64(o), want, "bf16", "prefix mean")
    assert np.abs(np64(lse) - np.log(np.arange(1, S + 1))[None, None]).max() < 1e-3


@pytest.mark.parametrize("variant", ["vanilla", "causal", "alibi", "document"])
@pytest.mark.parametrize("case", ["sharp", "low"])
def test_bf16_extreme_scores(variant, case):
    """Scores far outside the exponential's range, which the running
    reference has to absorb: 'sharp' scores spread over hundreds of base-2
    units (terms overflow unless the reference moves up); 'low' puts every
    score of every row below -190 in base 2 (the terms underflow to no mass
    unless the reference moves down).  scale * log2(e) = 1/8 keeps the
    kernel's pre-scaled Q exact, so only P's rounding separates the two
    sides; O and LSE are compared with the oracle."""
    B, H, S, D = 1, 2, 300, 64
    q, k, v = inputs.attn_inputs(B, H, H, S, S, D, "bf16", seed=63)
    u = torch.full((D,), 1.0 / 8.0)  # unit vector
    if case == "sharp":
        q = (q.float() * 30).to(torch.bfloat16)
    else:
        k = (k.float() * 0.1 + 20 * u).to(torch.bfloat16)
        q = (q.float() * 0.1 - 80 * u).to(torch.bfloat16)
    kw = dict(variant=variant, scale=0.125 / math.log2(math.e))
    if variant == "document":
        kw["doc_offsets"] = inputs.doc_offsets(B, S, 3, seed=64)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "%s %s O" % (variant, case))
    assert np.abs(np64(lse) - rl).max() < 1e-2, np.abs(np64(lse) - rl).max()
    if case == "low":
        assert rl.max() < -100  # the scores really are that low


@pytest.mark.parametrize("mul", [5, 25])
@pytest.mark.parametrize("variant", VARIANTS)
def test_bf16_large_logits_default_scale(variant, mul):
    """Logits of standard deviation 5 and 25 (Q scaled up) with the default
    scale 1/sqrt(D), whose scale * log2(e) is no power of two: the kernel
    must not round Q times that factor to bf16 (an error that grows with
    the logits), so O stays within the bf16 tolerance of the oracle."""
    B, H, S, D = 1, 2, 300, 64
    q, k, v = inputs.attn_inputs(B, H, H, S, S, D, "bf16", seed=70 + mul)
    q = (q.float() * mul).to(torch.bfloat16)
    kw = variant_kw(variant, S, B, seed=71)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "%s logits x%d" % (variant, mul))
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2 * max(1.0, np.abs(rl).max() / 64), "lse %g" % mx


@pytest.mark.parametrize("case", ["plain", "sharp", "low", "mixed"])
def test_alibi_two_blocks(case):
    """ALiBi on a grid deep enough for two query blocks per wave (1 x 128
    heads x 1024 rows: 512 work-groups of 256 rows), on sampled rows: plain
    inputs; 'sharp' and 'low' scores as in the extreme-score test, which
    every work-group's first pass must hand to the checked pass; 'mixed'
    makes only the first 64 heads low, so some work-groups keep their first
    pass and others redo the walk."""
    B, H, S, D = 1, 128, 1024, 64
    q, k, v = inputs.attn_inputs(B, H, H, S, S, D, "bf16", seed=74)
    u = torch.full((D,), 1.0 / 8.0)  # unit vector
    if case == "sharp":
        q = (q.float() * 30).to(torch.bfloat16)
    elif case in ("low", "mixed"):
        hs = slice(0, H if case == "low" else 64)
        kf, qf = k.float(), q.float()
        kf[:, hs] = kf[:, hs] * 0.1 + 20 * u
        qf[:, hs] = qf[:, hs] * 0.1 - 80 * u
        k, q = kf.to(torch.bfloat16), qf.to(torch.bfloat16)
    kw = dict(variant="alibi", alibi_max_bias=8.0)
    o, lse = run_gpu_attn(q, k, v, **kw)
    rows = sample_rows(B, H, S, 400, seed=75)
    ro, rl = oracle.attn(np64(q), np64(k), np64(v), rows=rows, **kw)
    check(gpu_rows(o, rows), ro, "bf16", "alibi two blocks %s" % case)
    mx, _, _ = errors(np64(lse).reshape(-1)[rows], rl)
    assert mx < 2e-2 * max(1.0, np.abs(rl).max() / 64), mx


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fully_masked_rows(dtype):
    """A -inf bias row and an empty key set give O = 0 and LSE = -inf."""
    B, H, S = 1, 2, 64
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, dtype, seed=62)
    bias = torch.zeros(H, S, S, dtype=q.dtype)
    bias[:, 5, :] = float("-inf")
    o, lse = run_gpu_attn(q, k, v, bias=bias)
    assert (np64(o)[:, :, 5] == 0).all() and np.isneginf(np64(lse)[:, :, 5]).all()
    ro, rl = run_oracle_attn(q, k, v, bias=bias)
    check(np64(o), ro, dtype, "masked row")
    # no keys at all
    k0 = torch.zeros(B, H, 0, 64, dtype=q.dtype)
    o, lse = run_gpu_attn(q, k0, k0)
    assert (np64(o) == 0).all() and np.isneginf(np64(lse)).all()


def test_empty_queries():
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16)
    _, k, v = inputs.attn_inputs(1, 2, 2, 10, 10, 64, "bf16", seed=63)
    o, lse = run_gpu_attn(q, k, v)
    assert o.shape == (1, 2, 0, 64)


def test_deterministic_and_guarded_outputs():
    """Two runs agree bit for bit; NaN guards around the output stay untouched."""
    B, H, S = 2, 4, 1000
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=64)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    n = B * H * S * 64
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = buf[guard:guard + n].view(B, H, S, 64)
    outs = []
    for variant in ("causal", "causal"):
        api.fl_attn_fwd(q, k, v, variant=variant, out=out)
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1])
    assert torch.isnan(buf[:guard].float()).all() and torch.isnan(buf[guard + n:].float()).all()
    assert torch.isfinite(out.float()).all()


# ---------------------------------------------------------------------------
# differential attention


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Dv", [64, 128])
def test_diffattn_small(dtype, causal, Dv):
    B, H, S = 2, 3, 190
    q1, q2, k1, k2, v = inputs.diffattn_inputs(B, H, S, 64, Dv, dtype, seed=70)
    g = [t.to(DEV) for t in (q1, q2, k1, k2, v)]
    o, l1, l2 = api.fl_diffattn_fwd(*g, lam=0.8, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    ro, rl1, rl2 = oracle.diffattn(*(np64(t) for t in (q1, q2, k1, k2, v)), lam=0.8, causal=causal,
                                   scale=0.125)
    check(np64(o), ro, dtype, "diffattn")
    check(np64(l1), rl1, "f32" if dtype == "f32" else "bf16", "lse1")
    check(np64(l2), rl2, "f32" if dtype == "f32" else "bf16", "lse2")
    # lambda = 0 is vanilla attention of the first stream
    o0 = api.fl_diffattn_fwd(*g, lam=0.0, causal=causal)
    torch.cuda.synchronize()
    rv, _ = oracle.attn(np64(q1), np64(k1), np64(v), variant="causal" if causal else "vanilla")
    check(np64(o0), rv, dtype, "diffattn lambda 0")


@pytest.mark.parametrize("causal", [False, True])
def test_diffattn_one_stream_out_of_range(causal):
    """The second stream's rows from 150 on have every score near -290 in
    base 2 (their terms underflow against a reference of 0), the first
    stream's stay ordinary.  The waves of the two streams share a
    work-group, so that work-group must redo both streams with a running
    reference; O and both LSEs against the oracle."""
    B, H, S, D = 1, 2, 300, 64
    q1, q2, k1, k2, v = inputs.diffattn_inputs(B, H, S, D, 128, "bf16", seed=72)
    u = torch.full((D,), 1.0 / 8.0)  # unit vector
    k2 = (k2.float() * 0.1 + 20 * u).to(torch.bfloat16)
    low = q2.float() * 0.1 - 80 * u
    q2 = torch.cat([q2.float()[:, :, :150], low[:, :, 150:]], 2).to(torch.bfloat16)
    g = [t.to(DEV) for t in (q1, q2, k1, k2, v)]
    o, l1, l2 = api.fl_diffattn_fwd(*g, lam=0.8, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    ro, rl1, rl2 = oracle.diffattn(*(np64(t) for t in (q1, q2, k1, k2, v)), lam=0.8, causal=causal,
                                   scale=0.125)
    check(np64(o), ro, "bf16", "diffattn one stream low")
    check(np64(l1), rl1, "bf16", "lse1")
    assert np.abs(np64(l2) - rl2).max() < 2e-2 * max(1.0, np.abs(rl2).max() / 64)
    assert rl2[:, :, 150:].max() < -150  # the low rows really are that low


@pytest.mark.parametrize("Dv", [64, 128])
def test_diffattn_cross_lengths_and_cancellation(Dv):
    # 70 queries against 200 keys (a partial query tile whose missing rows
    # still join the streams' hand-over, ragged key tiles), and identical
    # streams with lambda 1, whose outputs cancel (to within the rounding of
    # one normalised stream: the combine may fuse its multiply and subtract)
    q1, q2, _, _, _ = inputs.diffattn_inputs(2, 3, 70, 64, Dv, "bf16", seed=71)
    _, _, k1, k2, v = inputs.diffattn_inputs(2, 3, 200, 64, Dv, "bf16", seed=72)
    g = [t.to(DEV) for t in (q1, q2, k1, k2, v)]
    o, l1, l2 = api.fl_diffattn_fwd(*g, lam=0.8, return_lse=True)
    torch.cuda.synchronize()
    ro, rl1, rl2 = oracle.diffattn(*(np64(t) for t in (q1, q2, k1, k2, v)), lam=0.8, scale=0.125)
    check(np64(o), ro, "bf16", "diffattn cross lengths")
    check(np64(l1), rl1, "bf16", "lse1")
    check(np64(l2), rl2, "bf16", "lse2")
    o1 = api.fl_diffattn_fwd(g[0], g[0], g[2], g[2], g[4], lam=1.0)
    torch.cuda.synchronize()
    assert np.abs(np64(o1)).max() <= 1e-6


# ---------------------------------------------------------------------------
# Evoformer gated attention


def evo_small(dtype, N_seq=6, N_res=72, H=4, C=32, seed=80):
    q, k, v, gate, bias, km = inputs.evoformer_inputs(N_seq, N_res, H, C, dtype, seed)
    km[1, :] = 0          # a fully masked MSA row
    km[:, 3] = 0          # a fully masked residue column
    return q, k, v, gate, bias, km


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("N_res", [72, 200])
def test_evoformer_row(dtype, with_bias, N_res):
    # 72 residues: one partial query tile and a partial key tile; 200: two
    # query tiles (the second partial) and four key tiles of the staged bias
    q, k, v, gate, bias, km = evo_small(dtype, N_res=N_res)
    pb = bias if with_bias else None
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        pair_bias=None if pb is None else pb.to(DEV),
                                        key_mask=km.to(DEV), axis="row")
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate),
                          pair_bias=None if pb is None else np64(pb), key_mask=km.numpy(), axis="row")
    check(np64(o), ro, dtype, "evoformer row")
    assert (np64(o)[1] == 0).all()


@pytest.mark.parametrize("axis", ["row", "col"])
def test_evoformer_large_logits(axis):
    """Queries scaled by 25 at the scale 1/sqrt(C), whose scale * log2(e) is
    no power of two: both forms (the row form with the pair bias on the
    vector path, the column form on the folded one) stay within the bf16
    tolerance of the oracle."""
    q, k, v, gate, bias, km = evo_small("bf16", N_seq=40 if axis == "col" else 6,
                                        N_res=24 if axis == "col" else 72)
    q = (q.float() * 25).to(torch.bfloat16)
    pb = bias if axis == "row" else None
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        pair_bias=None if pb is None else pb.to(DEV),
                                        key_mask=km.to(DEV), axis=axis)
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate),
                          pair_bias=None if pb is None else np64(pb), key_mask=km.numpy(), axis=axis)
    check(np64(o), ro, "bf16", "evoformer %s large logits" % axis)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N_seq", [40, 129, 200])
def test_evoformer_col(dtype, N_seq):
    q, k, v, gate, _, km = evo_small(dtype, N_seq=N_seq, N_res=24)
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        key_mask=km.to(DEV), axis="col")
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate), key_mask=km.numpy(), axis="col")
    check(np64(o), ro, dtype, "evoformer col")
    assert (np64(o)[:, 3] == 0).all()


@pytest.mark.parametrize("axis,n", [("row", 72), ("row", 200), ("col", 40), ("col", 129)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_evoformer_no_key_mask(axis, n, with_bias):
    """No key mask: every key below the length counts (the instances without
    a mask, with ragged key tiles, one and two query blocks per wave)."""
    if axis == "col" and with_bias:
        pytest.skip("the column form takes no pair bias")
    q, k, v, gate, bias, _ = evo_small("bf16", N_seq=n if axis == "col" else 5,
                                       N_res=n if axis == "row" else 24, seed=85)
    pb = bias if with_bias else None
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        pair_bias=None if pb is None else pb.to(DEV),
                                        key_mask=None, axis=axis)
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate),
                          pair_bias=None if pb is None else np64(pb), key_mask=None, axis=axis)
    check(np64(o), ro, "bf16", "evoformer %s without a key mask" % axis)


# ---------------------------------------------------------------------------
# a score modification composed with a mask


MODS = ("vanilla", "alibi", "softcap")
MASKS = ("causal", "sliding_window", "prefix_lm", "document")


def composed_kw(mod, mask, S, B, seed, window_causal=True):
    kw = variant_kw(mod, S, B, seed)
    m = variant_kw(mask, S, B, seed, window_causal=window_causal)
    m["mask"] = m.pop("variant")
    kw.update(m)
    return kw


@pytest.mark.parametrize("S", [77, 300, 513])
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
def test_bf16_composed(mod, mask, S):
    B, Hq, Hkv, D = 2, 4, 2, 64
    seed = 400 + S + 7 * MASKS.index(mask) + 31 * MODS.index(mod)
    q, k, v = inputs.attn_inputs(B, Hq, Hkv, S, S, D, "bf16", seed=seed)
    kw = composed_kw(mod, mask, S, B, seed + 1)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "%s+%s S=%d" % (mod, mask, S))
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "lse %g" % mx


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", ["alibi", "softcap"])
def test_f32_composed(mod, mask):
    B, Hq, Hkv, S, D = 2, 4, 2, 150, 64
    seed = 500 + 7 * MASKS.index(mask) + 31 * MODS.index(mod)
    q, k, v = inputs.attn_inputs(B, Hq, Hkv, S, S, D, "f32", seed=seed)
    kw = composed_kw(mod, mask, S, B, seed + 1)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "f32", "%s+%s" % (mod, mask))
    check(np64(lse), rl, "f32", "%s+%s lse" % (mod, mask))


@pytest.mark.parametrize("mod", ["alibi", "softcap"])
def test_bf16_composed_two_sided_window_and_bias(mod):
    # a two-sided window puts ALiBi keys on both sides of the diagonal; a bias
    # sends the modified scores through the general path
    B, H, S = 1, 4, 336  # bf16 bias rows are whole 16-byte groups
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=77)
    kw = composed_kw(mod, "sliding_window", S, B, 78, window_causal=False)
    o, lse = run_gpu_attn(q, k, v, **kw)
    ro, rl = run_oracle_attn(q, k, v, **kw)
    check(np64(o), ro, "bf16", "%s two-sided" % mod)
    bias = inputs.bias_inputs(H, S, S, "bf16", seed=79)
    kw = composed_kw(mod, "causal", S, B, 80)
    o, lse = run_gpu_attn(q, k, v, bias=bias, **kw)
    ro, rl = run_oracle_attn(q, k, v, bias=bias, **kw)
    check(np64(o), ro, "bf16", "%s causal + bias" % mod)


def test_composed_equals_variant_when_trivial():
    # vanilla scores under a composed causal mask are the causal variant, bit
    # for bit: the same kernel instance runs
    B, H, S = 1, 2, 300
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=81)
    a, la = run_gpu_attn(q, k, v, variant="vanilla", mask="causal")
    b, lb = run_gpu_attn(q, k, v, variant="causal")
    assert torch.equal(a, b) and torch.equal(la, lb)


# ---------------------------------------------------------------------------
# full workload sizes, sampled rows


def _full_attn(name, variants, n_rows):
    wl = inputs.WORKLOADS[name]
    t = inputs.make(wl)
    s = wl.shape
    q, k, v = t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV)
    q64, k64, v64 = np64(t["q"]), np64(t["k"]), np64(t["v"])
    rows = sample_rows(s["B"], s["Hq"], s["S"], n_rows, seed=len(name))
    for variant in variants:
        kw = dict(variant=variant)
        for key in ("softcap", "alibi_max_bias", "window", "window_causal", "prefix"):
            if key in wl.params:
                kw[key] = wl.params[key]
        docs = t.get("doc_offsets")
        if variant == "document":
            kw["doc_offsets"] = docs
        o, lse = run_gpu_attn(q, k, v, **kw)
        kw.pop("doc_offsets", None)
        ro, rl = oracle.attn(q64, k64, v64, rows=rows,
                             doc_offsets=None if variant != "document" else docs.numpy(), **kw)
        check(gpu_rows(o, rows), ro, "bf16", "%s %s" % (name, variant))
        mx, _, _ = errors(np64(lse).reshape(-1)[rows], rl)
        assert mx < 2e-2, (variant, mx)
        assert torch.isfinite(o.float()).all()


def test_full_mha_s2048_all_variants():
    _full_attn("mha_bf16_b4_h16_s2048_d64", inputs.ALL_MASK_VARIANTS, 384)


def test_full_mha_s4096_all_variants():
    _full_attn("mha_bf16_b4_h16_s4096_d64", inputs.ALL_MASK_VARIANTS, 256)


def test_full_mha_s4096_composed():
    wl = inputs.WORKLOADS["mha_bf16_b4_h16_s4096_d64"]
    t = inputs.make(wl)
    s = wl.shape
    q, k, v = t["q"].to(DEV), t["k"].to(DEV), t["v"].to(DEV)
    q64, k64, v64 = np64(t["q"]), np64(t["k"]), np64(t["v"])
    rows = sample_rows(s["B"], s["Hq"], s["S"], 192, seed=9)
    docs = t["doc_offsets"]
    for mod, mask in (("alibi", "causal"), ("softcap", "causal"), ("softcap", "sliding_window"),
                      ("alibi", "document"), ("softcap", "prefix_lm")):
        kw = dict(variant=mod, mask=mask)
        for key in ("softcap", "alibi_max_bias", "window", "window_causal", "prefix"):
            if key in wl.params:
                kw[key] = wl.params[key]
        o, lse = run_gpu_attn(q, k, v, doc_offsets=docs if mask == "document" else None, **kw)
        ro, rl = oracle.attn(q64, k64, v64, rows=rows,
                             doc_offsets=docs.numpy() if mask == "document" else None, **kw)
        check(gpu_rows(o, rows), ro, "bf16", "%s+%s" % (mod, mask))
        mx, _, _ = errors(np64(lse).reshape(-1)[rows], rl)
        assert mx < 2e-2, (mod, mask, mx)


def test_full_gqa_s16384():
    _full_attn("gqa_bf16_b1_hq32_hkv8_s16384_d64", ("causal", "sliding_window"), 192)


def test_full_diffattn_s4096():
    wl = inputs.WORKLOADS["diffattn_bf16_b4_h16_s4096_dqk64_dv128"]
    t = inputs.make(wl)
    s = wl.shape
    g = [t[n].to(DEV) for n in ("q1", "q2", "k1", "k2", "v")]
    c = [np64(t[n]) for n in ("q1", "q2", "k1", "k2", "v")]
    rows = sample_rows(s["B"], s["H"], s["S"], 192, seed=4)
    for causal in (False, True):
        o = api.fl_diffattn_fwd(*g, lam=wl.params["lam"], causal=causal)
        torch.cuda.synchronize()
        ro, _, _ = oracle.diffattn(*c, lam=wl.params["lam"], causal=causal, scale=0.125, rows=rows)
        check(gpu_rows(o, rows), ro, "bf16", "diffattn causal=%s" % causal)


def test_full_evoformer():
    wl = inputs.WORKLOADS["evoformer_bf16_nseq128_nres256_h8_c32"]
    t = inputs.make(wl)
    g = {n: t[n].to(DEV) for n in ("q", "k", "v", "gate", "pair_bias", "key_mask")}
    c = {n: np64(t[n]) for n in ("q", "k", "v", "gate", "pair_bias")}
    km = t["key_mask"].numpy()
    N_seq, N_res, H, C = t["q"].shape
    rng = np.random.default_rng(5)
    # row-wise: sampled (s, r, h) positions
    rows = np.unique(rng.choice(N_seq * N_res * H, 2048, replace=False))
    o = api.fl_evoformer_gated_attn_fwd(g["q"], g["k"], g["v"], g["gate"], pair_bias=g["pair_bias"],
                                        key_mask=g["key_mask"], axis="row")
    torch.cuda.synchronize()
    ro = oracle.evoformer(c["q"], c["k"], c["v"], c["gate"], pair_bias=c["pair_bias"], key_mask=km,
                          axis="row", rows=rows)
    check(np64(o).reshape(-1, C)[rows], ro, "bf16", "evoformer row")
    # column-wise: the oracle indexes the transposed problem (r*N_seq + s)*H + h
    o = api.fl_evoformer_gated_attn_fwd(g["q"], g["k"], g["v"], g["gate"], key_mask=g["key_mask"],
                                        axis="col")
    torch.cuda.synchronize()
    ro = oracle.evoformer(c["q"], c["k"], c["v"], c["gate"], key_mask=km, axis="col", rows=rows)
    h = rows % H
    s_ = (rows // H) % N_seq
    r_ = rows // (H * N_seq)
    got = np64(o)[s_, r_, h]
    check(got, ro, "bf16", "evoformer col")
