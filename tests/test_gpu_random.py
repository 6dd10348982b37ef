"""Seeded random sweep of the forward and backward against the float64 oracle.

Each case draws its shape and variant from a generator seeded by the case
number: batch 1-2, K/V heads 1-4 and GQA group 1-4, lengths 1-600 (query
and key lengths apart only without a mask, the cases the boundary accepts),
a score modification (none, ALiBi with a random maximum bias, softcap with a
random cap) composed with a mask (none, causal, a causal or two-sided
window of random width, a random prefix, 1-6 documents), sometimes a bias,
a negative or zero scale, or queries scaled by 5 or 25 (a bias rounds the
key length up to a multiple of 8, as the boundary requires for bf16).
Every element of O and the LSE is compared (bf16 tolerance), and of dQ, dK
and dV for the backward cases (the backward parity tolerance).  Decode,
differential attention, both Evoformer forms and the IPA core get sweeps
of their own.  The case
parameters are printed before each GPU call, so a failing case names
itself.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"

MASKS = (None, "causal", "sliding_window", "prefix_lm", "document")
MODS = ("vanilla", "alibi", "softcap")


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def draw(case, max_len):
    """One random configuration (a dict of shapes and keyword arguments)."""
    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4]))
    mod = str(rng.choice(MODS))
    mask = MASKS[int(rng.integers(0, len(MASKS)))]
    Sq = int(rng.integers(1, max_len + 1))
    Sk = Sq if mask is not None or rng.random() < 0.5 else int(rng.integers(1, max_len + 1))
    kw = {}
    if mask is None:
        kw["variant"] = mod
    elif mod == "vanilla":
        kw["variant"] = mask
    else:
        kw["variant"], kw["mask"] = mod, mask
    if mod == "alibi":
        kw["alibi_max_bias"] = float(rng.uniform(1.0, 16.0))
    if mod == "softcap":
        kw["softcap"] = float(rng.uniform(5.0, 100.0))
    if mask == "sliding_window":
        kw["window"] = int(rng.integers(1, Sq + 40))
        kw["window_causal"] = bool(rng.random() < 0.6)
    if mask == "prefix_lm":
        kw["prefix"] = int(rng.integers(0, Sq + 20))
    if mask == "document":
        kw["doc_offsets"] = inputs.doc_offsets(B, Sq, min(int(rng.integers(1, 7)), Sq),
                                               seed=9500 + case)
    r = rng.random()
    if r < 0.1:
        kw["scale"] = -1.0 / math.sqrt(64)
    elif r < 0.15:
        kw["scale"] = 0.0
    q_mul = float(rng.choice([1.0, 1.0, 1.0, 5.0, 25.0]))
    with_bias = bool(rng.random() < 0.2)
    if with_bias and Sk % 8:
        # a bf16 bias needs S_k % 8 == 0 (16-byte bias rows)
        Sk = Sk + 8 - Sk % 8
        if mask is not None:
            Sq = Sk
            if mask == "document":
                kw["doc_offsets"] = inputs.doc_offsets(B, Sq, min(int(rng.integers(1, 7)), Sq),
                                                       seed=9600 + case)
    return dict(B=B, Hkv=Hkv, Hq=Hkv * G, Sq=Sq, Sk=Sk, kw=kw, q_mul=q_mul, with_bias=with_bias)


def describe(case, c):
    kw = {k: v for k, v in c["kw"].items() if k != "doc_offsets"}
    return "case %d: B=%d Hq=%d Hkv=%d Sq=%d Sk=%d q*%g bias=%s %s" % (
        case, c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], c["q_mul"], c["with_bias"], kw)


def make_inputs(case, c, D=64):
    q, _, _ = inputs.attn_inputs(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sq"], D, "bf16",
                                 seed=9100 + case)
    _, k, v = inputs.attn_inputs(c["B"], c["Hq"], c["Hkv"], c["Sk"], c["Sk"], D, "bf16",
                                 seed=9200 + case)
    if c["q_mul"] != 1.0:
        q = (q.float() * c["q_mul"]).to(torch.bfloat16)
    bias = inputs.bias_inputs(c["Hq"], c["Sq"], c["Sk"], "bf16", seed=9300 + case) \
        if c["with_bias"] else None
    return q, k, v, bias


@pytest.mark.parametrize("case", range(48))
def test_random_forward(case):
    c = draw(case, 600)
    what = describe(case, c)
    print(what, flush=True)
    q, k, v, bias = make_inputs(case, c)
    kw = dict(c["kw"])
    docs = kw.pop("doc_offsets", None)
    o, lse = api.fl_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                             bias=None if bias is None else bias.to(DEV),
                             doc_offsets=None if docs is None else docs.to(DEV),
                             return_lse=True, **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(np64(q), np64(k), np64(v), bias=None if bias is None else np64(bias),
                         doc_offsets=None if docs is None else docs.numpy(), **kw)
    check(np64(o), ro, "bf16", what)
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "%s: lse %g" % (what, mx)


def check_grad(got, want, what):
    # the tolerance of the backward parity tests: errors against the size of
    # each gradient tensor (largest element 2e-2, mean 5e-3, sizes >= 0.05)
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert np.isfinite(got).all(), what + ": non-finite"
    err = np.abs(got - want)
    smax = max(np.abs(want).max(), 0.05)
    smean = max(np.abs(want).mean(), 0.05)
    assert err.max() <= 2e-2 * smax and err.mean() <= 5e-3 * smean, \
        "%s: max err %.3g (|ref| max %.3g), mean err %.3g (|ref| mean %.3g)" % (
            what, err.max(), smax, err.mean(), smean)


@pytest.mark.parametrize("case", range(100, 124))
def test_random_backward(case):
    c = draw(case, 300)
    if c["with_bias"]:
        c["with_bias"] = False  # the backward takes no bias
    if c["q_mul"] == 25.0:
        c["q_mul"] = 5.0
    what = describe(case, c)
    print(what, flush=True)
    q, k, v, _ = make_inputs(case, c)
    do = inputs.randn(torch.Generator().manual_seed(9400 + case), tuple(q.shape), "bf16")
    kw = dict(c["kw"])
    docs = kw.pop("doc_offsets", None)
    dkw = dict(kw)
    if docs is not None:
        dkw["doc_offsets"] = docs.to(DEV)
    g = [t.to(DEV) for t in (q, k, v, do)]
    o, lse = api.fl_attn_fwd(g[0], g[1], g[2], return_lse=True, **dkw)
    dq, dk, dv = api.fl_attn_bwd(g[0], g[1], g[2], o, lse, g[3], **dkw)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(np64(q), np64(k), np64(v), np64(do),
                          doc_offsets=None if docs is None else docs.numpy(), **kw)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(np64(got), want, "%s %s" % (what, name))


DEC_MASKS = (None, "causal", "sliding_window", "prefix_lm")


@pytest.mark.parametrize("case", range(200, 224))
def test_random_decode(case):
    """Decode against KV caches of random capacity and lengths (0 .. capacity),
    GQA groups 1-8, 1-8 new tokens, either cache layout, 0-5 key splits."""
    rng = np.random.default_rng(9000 + case)
    B = int(rng.integers(1, 6))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    Sq = int(rng.integers(1, 9))
    S_cap = int(rng.integers(1, 801))
    layout = str(rng.choice(["bhsd", "bshd"]))
    splits = int(rng.choice([0, 1, 2, 3, 5]))
    mod = str(rng.choice(MODS))
    mask = DEC_MASKS[int(rng.integers(0, len(DEC_MASKS)))]
    kw = dict(variant=mod if mask is None or mod != "vanilla" else mask)
    if mask is not None and mod != "vanilla":
        kw["mask"] = mask
    if mod == "alibi":
        kw["alibi_max_bias"] = float(rng.uniform(1.0, 16.0))
    if mod == "softcap":
        kw["softcap"] = float(rng.uniform(5.0, 100.0))
    if mask == "sliding_window":
        kw["window"] = int(rng.integers(1, S_cap + 40))
        kw["window_causal"] = mod == "alibi" or bool(rng.random() < 0.6)
    if mask == "prefix_lm":
        kw["prefix"] = int(rng.integers(0, S_cap + 20))
    if rng.random() < 0.1:
        kw["scale"] = -1.0 / math.sqrt(64)
    q_mul = float(rng.choice([1.0, 1.0, 5.0, 25.0]))
    seqlens = torch.tensor(rng.integers(0, S_cap + 1, size=B), dtype=torch.int32)
    what = "case %d: B=%d Hq=%d Hkv=%d Sq=%d S_cap=%d %s splits=%d q*%g %s lens=%s" % (
        case, B, Hkv * G, Hkv, Sq, S_cap, layout, splits, q_mul, kw, seqlens.tolist())
    print(what, flush=True)
    q, kc, vc = inputs.decode_inputs(B, Hkv * G, Hkv, Sq, S_cap, 64, seed=9700 + case,
                                     layout=layout)
    if q_mul != 1.0:
        q = (q.float() * q_mul).to(torch.bfloat16)
    o, lse = api.fl_attn_decode_fwd(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV),
                                    layout=layout, num_splits=splits, return_lse=True, **kw)
    torch.cuda.synchronize()
    if layout == "bshd":
        kc, vc = kc.transpose(1, 2), vc.transpose(1, 2)
    ro, rl = oracle.decode(np64(q), np64(kc), np64(vc), seqlens.numpy(), **kw)
    check(np64(o), ro, "bf16", what)
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "%s: lse %g" % (what, mx)


@pytest.mark.parametrize("case", range(300, 312))
def test_random_diffattn(case):
    """Differential attention: random lengths (equal under the causal mask),
    heads, lambda in [0, 1.2], value dims 64 or 128, logits x1 or x5."""
    rng = np.random.default_rng(9000 + case)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    causal = bool(rng.random() < 0.5)
    Sq = int(rng.integers(1, 500))
    Sk = Sq if causal else int(rng.integers(1, 500))
    Dv = int(rng.choice([64, 128]))
    lam = float(rng.uniform(0.0, 1.2))
    q_mul = float(rng.choice([1.0, 5.0]))
    what = "case %d: B=%d H=%d Sq=%d Sk=%d Dv=%d causal=%s lam=%.3f q*%g" % (
        case, B, H, Sq, Sk, Dv, causal, lam, q_mul)
    print(what, flush=True)
    g = torch.Generator().manual_seed(9800 + case)
    q1, q2 = (inputs.randn(g, (B, H, Sq, 64), "bf16") for _ in range(2))
    k1, k2 = (inputs.randn(g, (B, H, Sk, 64), "bf16") for _ in range(2))
    v = inputs.randn(g, (B, H, Sk, Dv), "bf16")
    if q_mul != 1.0:
        q1, q2 = ((t.float() * q_mul).to(torch.bfloat16) for t in (q1, q2))
    o = api.fl_diffattn_fwd(*(t.to(DEV) for t in (q1, q2, k1, k2, v)), lam=lam, causal=causal)
    torch.cuda.synchronize()
    ro, _, _ = oracle.diffattn(*(np64(t) for t in (q1, q2, k1, k2, v)), lam=lam, causal=causal)
    check(np64(o), ro, "bf16", what)


@pytest.mark.parametrize("case", range(400, 416))
def test_random_evoformer(case):
    """Evoformer gated attention: row form (with or without the pair bias) or
    column form, random MSA sizes and heads, random key masks with some rows
    or columns fully masked, or no mask."""
    rng = np.random.default_rng(9000 + case)
    axis = str(rng.choice(["row", "col"]))
    H = int(rng.integers(1, 9))
    with_bias = axis == "row" and bool(rng.random() < 0.7)
    N_seq = int(rng.integers(1, 90))
    N_res = int(rng.integers(1, 300))
    if with_bias:
        N_res = N_res + (-N_res) % 8  # a bf16 pair bias needs N_res % 8 == 0
    with_mask = bool(rng.random() < 0.8)
    what = "case %d: %s N_seq=%d N_res=%d H=%d bias=%s mask=%s" % (
        case, axis, N_seq, N_res, H, with_bias, with_mask)
    print(what, flush=True)
    q, k, v, gate, bias, km = inputs.evoformer_inputs(N_seq, N_res, H, 32, "bf16", 9900 + case,
                                                      masked_frac=float(rng.uniform(0.0, 0.3)))
    if with_mask and N_seq > 2 and N_res > 2:
        km[int(rng.integers(0, N_seq)), :] = 0
        km[:, int(rng.integers(0, N_res))] = 0
    pb = bias if with_bias else None
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        pair_bias=None if pb is None else pb.to(DEV),
                                        key_mask=km.to(DEV) if with_mask else None, axis=axis)
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate),
                          pair_bias=None if pb is None else np64(pb),
                          key_mask=km.numpy() if with_mask else None, axis=axis)
    check(np64(o), ro, "bf16", what)


PTS_MAX_ABS, PTS_MEAN_ABS = 1e-3, 1e-4  # the IPA parity tests' o_pts bar


@pytest.mark.parametrize("case", range(500, 512))
def test_random_ipa(case):
    """IPA core: random residue counts 1-200, heads 1-12, pair channels 0, 64
    or 128, with or without bias and key mask, key-mask density 0-50%."""
    rng = np.random.default_rng(9000 + case)
    B, L, H = int(rng.integers(1, 3)), int(rng.integers(1, 201)), int(rng.integers(1, 13))
    cz = int(rng.choice([0, 64, 128]))
    with_bias, with_mask = bool(rng.random() < 0.7), bool(rng.random() < 0.7)
    frac = float(rng.uniform(0.0, 0.5))
    what = "case %d: B=%d L=%d H=%d cz=%d bias=%s mask=%s (%.2f)" % (
        case, B, L, H, cz, with_bias, with_mask, frac)
    print(what, flush=True)
    t = inputs.ipa_inputs(B, L, H, 16, 4, 8, cz or 128, "bf16", seed=10000 + case,
                          masked_frac=frac)
    if cz == 64:
        t["z"] = t["z"][..., :64].contiguous()
    g = {n: x.to(DEV) for n, x in t.items()}
    o, op, oz = api.fl_ipa_attn_fwd(g["q"], g["k"], g["v"], g["q_pts"], g["k_pts"], g["v_pts"],
                                    g["rot"], g["trans"], g["gamma"],
                                    pair_bias=g["pair_bias"] if with_bias else None,
                                    z=g["z"] if cz else None,
                                    key_mask=g["key_mask"] if with_mask else None)
    torch.cuda.synchronize()
    c = {n: np64(x) for n, x in t.items()}
    ro, rp, rz = oracle.ipa(c["q"], c["k"], c["v"], c["q_pts"], c["k_pts"], c["v_pts"],
                            c["rot"], c["trans"], c["gamma"],
                            pair_bias=c["pair_bias"] if with_bias else None,
                            z=c["z"] if cz else None,
                            key_mask=t["key_mask"].numpy() if with_mask else None)
    check(np64(o), ro, "bf16", what + " o")
    mx, mean, _ = errors(np64(op), rp)
    assert mx <= PTS_MAX_ABS and mean <= PTS_MEAN_ABS, "%s o_pts: max %.3g mean %.3g" % (
        what, mx, mean)
    if cz:
        check(np64(oz), rz, "bf16", what + " o_pair")
