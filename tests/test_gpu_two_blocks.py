"""GPU parity of the two-query-block kernel instances, and of signed and
zero scales.

The launcher gives each wave two 32-row query blocks (256-row work-groups)
when the grid of 256-row work-groups is deep enough: at least 512 of them
for rows that see every key (vanilla, ALiBi, softcap, with or without a
bias; ALiBi with a bias keeps one block), at least 1024 under a causal or
PrefixLM mask, at least 2048 under a document mask; a sliding window always
keeps one.  The shapes below pass those thresholds, so every two-block
instance the launcher can choose runs here, with ragged tails (S % 64 != 0
and rows past S_q inside the last 256-row tile), on sampled rows against
the float64 oracle:

* dense, no bias, B4 H32 S1000 (512 work-groups): plain scores, ALiBi, the
  bounded softcap (cap 50) and the softcap with a running reference (cap 80);
* dense with a bias, B8 H16 S1000 (512): plain and softcap (caps 50 and 80:
  a bias always takes the running reference);
* masked, B1 H128 S4000 (2048): causal, PrefixLM, document, and ALiBi,
  softcap (both caps) composed with them;
* masked with a bias, B64 H4 S2000 (2048): causal, document and
  softcap + causal;
* masked at the causal threshold, B2 H32 S4000 (1024): causal, PrefixLM,
  ALiBi + causal, softcap + PrefixLM at two blocks, and the document mask,
  which keeps one block there.

Row sampling takes random rows plus the first and last rows of a few heads
and the rows on both sides of each 64, 128, 256, 512 and 768-row boundary.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, gpu_rows, np64, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILES = (64, 128, 256, 512, 768)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def two_block_grid(B, H, S, masked, document=False):
    """The launcher's depth rule for two query blocks per wave."""
    wg2 = B * H * ((S + 255) // 256)
    return wg2 >= (512 if not masked else 2048 if document else 1024)


def compare_rows(q, k, v, kw, rows, what, bias=None, lse_scale=False):
    docs = kw.get("doc_offsets")
    gkw = dict(kw)
    if docs is not None:
        gkw["doc_offsets"] = docs.to(DEV)
    o, lse = api.fl_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV),
                             bias=None if bias is None else bias.to(DEV), return_lse=True, **gkw)
    torch.cuda.synchronize()
    okw = dict(kw)
    if docs is not None:
        okw["doc_offsets"] = docs.numpy()
    ro, rl = oracle.attn(np64(q), np64(k), np64(v), bias=None if bias is None else np64(bias),
                         rows=rows, **okw)
    check(gpu_rows(o, rows), ro, "bf16", what)
    mx, _, _ = errors(np64(lse).reshape(-1)[rows], rl)
    tol = 2e-2 * max(1.0, np.abs(rl[np.isfinite(rl)]).max() / 64) if lse_scale else 2e-2
    assert mx <= tol, "%s: lse %g" % (what, mx)
    assert torch.isfinite(o.float()).all(), what


DENSE = [("vanilla", {}), ("alibi", dict(alibi_max_bias=8.0)), ("softcap", dict(softcap=50.0)),
         ("softcap", dict(softcap=80.0))]


@pytest.mark.parametrize("variant,extra", DENSE, ids=["vanilla", "alibi", "softcap50", "softcap80"])
def test_two_blocks_dense_ragged(variant, extra):
    B, H, S = 4, 32, 1000
    assert two_block_grid(B, H, S, masked=False)
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=900)
    rows = sample_rows(B, H, S, 384, seed=901, extra_tiles=TILES)
    compare_rows(q, k, v, dict(variant=variant, **extra), rows, "%s %s QB2 ragged" % (variant, extra))


@pytest.mark.parametrize("variant,extra", [("vanilla", {}), ("softcap", dict(softcap=50.0)),
                                           ("softcap", dict(softcap=80.0)),
                                           ("alibi", dict(alibi_max_bias=8.0))],
                         ids=["vanilla", "softcap50", "softcap80", "alibi"])
def test_two_blocks_dense_bias(variant, extra):
    """(ALiBi with a bias keeps one block per wave; it runs here at the same
    shape for comparison.)"""
    B, H, S = 8, 16, 1000
    assert two_block_grid(B, H, S, masked=False)
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=910)
    bias = inputs.bias_inputs(H, S, S, "bf16", seed=911)
    rows = sample_rows(B, H, S, 384, seed=912, extra_tiles=TILES)
    compare_rows(q, k, v, dict(variant=variant, **extra), rows, "%s %s QB2 bias" % (variant, extra),
                 bias=bias)


MASKED = [
    ("causal", None, {}), ("prefix_lm", None, dict(prefix=512)), ("document", None, {}),
    ("alibi", "causal", dict(alibi_max_bias=8.0)), ("alibi", "prefix_lm", dict(alibi_max_bias=8.0, prefix=512)),
    ("alibi", "document", dict(alibi_max_bias=8.0)),
    ("softcap", "causal", dict(softcap=50.0)), ("softcap", "prefix_lm", dict(softcap=50.0, prefix=512)),
    ("softcap", "document", dict(softcap=50.0)), ("softcap", "causal", dict(softcap=80.0)),
]


@pytest.mark.parametrize("variant,mask,extra", MASKED,
                         ids=["causal", "prefix", "document", "alibi+causal", "alibi+prefix",
                              "alibi+document", "softcap+causal", "softcap+prefix",
                              "softcap+document", "softcap80+causal"])
def test_two_blocks_masked_deep(variant, mask, extra):
    B, H, S = 1, 128, 4000
    assert two_block_grid(B, H, S, masked=True, document="document" in (variant, mask))
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=920)
    kw = dict(variant=variant, **extra)
    if mask is not None:
        kw["mask"] = mask
    if "document" in (variant, mask):
        kw["doc_offsets"] = inputs.doc_offsets(B, S, 8, seed=921)
    rows = sample_rows(B, H, S, 384, seed=922, extra_tiles=TILES)
    compare_rows(q, k, v, kw, rows, "%s+%s QB2 masked" % (variant, mask))


@pytest.mark.parametrize("variant,mask,extra", [("causal", None, {}), ("document", None, {}),
                                                ("softcap", "causal", dict(softcap=50.0))],
                         ids=["causal", "document", "softcap+causal"])
def test_two_blocks_masked_bias(variant, mask, extra):
    B, H, S = 64, 4, 2000
    assert two_block_grid(B, H, S, masked=True, document=variant == "document")
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=930)
    bias = inputs.bias_inputs(H, S, S, "bf16", seed=931)
    kw = dict(variant=variant, **extra)
    if mask is not None:
        kw["mask"] = mask
    if variant == "document":
        kw["doc_offsets"] = inputs.doc_offsets(B, S, 8, seed=932)
    rows = sample_rows(B, H, S, 384, seed=933, extra_tiles=TILES)
    compare_rows(q, k, v, kw, rows, "%s+%s QB2 masked bias" % (variant, mask), bias=bias)


MID = [("causal", None, {}), ("prefix_lm", None, dict(prefix=512)),
       ("alibi", "causal", dict(alibi_max_bias=8.0)), ("softcap", "prefix_lm", dict(softcap=50.0, prefix=777)),
       ("document", None, {})]


@pytest.mark.parametrize("variant,mask,extra", MID,
                         ids=["causal", "prefix", "alibi+causal", "softcap+prefix", "document"])
def test_two_blocks_masked_threshold(variant, mask, extra):
    """1024 two-block work-groups: causal and PrefixLM rows take two blocks,
    document rows one."""
    B, H, S = 2, 32, 4000
    doc = "document" in (variant, mask)
    assert two_block_grid(B, H, S, masked=True) and not two_block_grid(B, H, S, True, document=True)
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=940)
    kw = dict(variant=variant, **extra)
    if mask is not None:
        kw["mask"] = mask
    if doc:
        kw["doc_offsets"] = inputs.doc_offsets(B, S, 8, seed=941)
    rows = sample_rows(B, H, S, 384, seed=942, extra_tiles=TILES)
    compare_rows(q, k, v, kw, rows, "%s+%s at the causal threshold" % (variant, mask))


# ---------------------------------------------------------------------------
# signed and zero scales


SCALED = [("vanilla", None, {}), ("alibi", None, dict(alibi_max_bias=8.0)),
          ("softcap", None, dict(softcap=50.0)), ("causal", None, {}),
          ("alibi", "causal", dict(alibi_max_bias=8.0)), ("softcap", "causal", dict(softcap=80.0))]


@pytest.mark.parametrize("shape", ["small", "two_blocks"])
@pytest.mark.parametrize("variant,mask,extra", SCALED,
                         ids=["vanilla", "alibi", "softcap", "causal", "alibi+causal", "softcap80+causal"])
def test_negative_scale_large_logits(variant, mask, extra, shape):
    """scale = -1/sqrt(D) at logits x25: the largest term sits at the most
    negative q.k, where a reference chosen as the row maximum of the raw
    product would sit at the wrong end."""
    B, H, S = (1, 2, 300) if shape == "small" else (4, 32, 1000)
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=940)
    q = (q.float() * 25).to(torch.bfloat16)
    kw = dict(variant=variant, scale=-1.0 / 8.0, **extra)
    if mask is not None:
        kw["mask"] = mask
    rows = sample_rows(B, H, S, 384, seed=941, extra_tiles=TILES)
    compare_rows(q, k, v, kw, rows, "%s+%s scale<0 %s" % (variant, mask, shape), lse_scale=True)


@pytest.mark.parametrize("variant,mask,extra", SCALED[:3] + [("causal", None, {})],
                         ids=["vanilla", "alibi", "softcap", "causal"])
def test_zero_scale(variant, mask, extra):
    """scale = 0: every score is 0 (vanilla, softcap: O is the mean of the
    allowed values) or the ALiBi penalty alone."""
    B, H, S = 1, 4, 300
    q, k, v = inputs.attn_inputs(B, H, H, S, S, 64, "bf16", seed=950)
    kw = dict(variant=variant, scale=0.0, **extra)
    rows = np.arange(B * H * S)
    compare_rows(q, k, v, kw, rows, "%s scale 0" % variant)


def test_negative_scale_decode_diffattn_evoformer():
    """The other entry points with folded scores take a negative scale too:
    decode (plain and ALiBi, split keys), DiffAttn (both streams) and the
    key-masked column Evoformer, at logits x25."""
    # decode
    B, Hq, Hkv, Sq, S_cap = 3, 8, 2, 2, 900
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, Sq, S_cap, 64, seed=960)
    q = (q.float() * 25).to(torch.bfloat16)
    seqlens = torch.tensor([900, 400, 77], dtype=torch.int32)
    for variant in ("vanilla", "alibi"):
        for splits in (1, 3):
            kw = dict(variant=variant, scale=-0.125, num_splits=splits)
            o, lse = api.fl_attn_decode_fwd(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV),
                                            return_lse=True, **kw)
            torch.cuda.synchronize()
            kw.pop("num_splits")
            ro, rl = oracle.decode(np64(q), np64(kc), np64(vc), seqlens.numpy(), **kw)
            check(np64(o), ro, "bf16", "decode %s scale<0 splits=%d" % (variant, splits))
            mx, _, _ = errors(np64(lse), rl)
            assert mx <= 2e-2 * max(1.0, np.abs(rl).max() / 64), mx
    # DiffAttn
    q1, q2, k1, k2, v = inputs.diffattn_inputs(2, 3, 190, 64, 128, "bf16", seed=961)
    q1 = (q1.float() * 25).to(torch.bfloat16)
    q2 = (q2.float() * 25).to(torch.bfloat16)
    g = [t.to(DEV) for t in (q1, q2, k1, k2, v)]
    for causal in (False, True):
        o = api.fl_diffattn_fwd(*g, lam=0.8, causal=causal, scale=-0.125)
        torch.cuda.synchronize()
        ro, _, _ = oracle.diffattn(*(np64(t) for t in (q1, q2, k1, k2, v)), lam=0.8, causal=causal,
                                   scale=-0.125)
        check(np64(o), ro, "bf16", "diffattn scale<0 causal=%s" % causal)
    # Evoformer, column form (key mask folded into the product)
    qe, ke, ve, gate, _, km = inputs.evoformer_inputs(40, 24, 4, 32, "bf16", 962)
    qe = (qe.float() * 25).to(torch.bfloat16)
    sc = -1.0 / math.sqrt(32)
    o = api.fl_evoformer_gated_attn_fwd(qe.to(DEV), ke.to(DEV), ve.to(DEV), gate.to(DEV),
                                        key_mask=km.to(DEV), axis="col", scale=sc)
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(qe), np64(ke), np64(ve), np64(gate), key_mask=km.numpy(), axis="col",
                          scale=sc)
    check(np64(o), ro, "bf16", "evoformer col scale<0")
