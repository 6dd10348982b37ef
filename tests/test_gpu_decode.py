"""GPU parity of decode against a KV cache and of the (O, LSE) merge: the HIP
path through the C ABI against the float64 oracle on the same seeded inputs.

Small caches are compared on every output; the decode workload at full size
on every row of a few sampled sequences.  The oracle takes the cache in the
[B, H_kv, S_cap, D] layout; the [B, S_cap, H_kv, D] layout holds the same
values.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"

MODS = ("vanilla", "alibi", "softcap")
MASKS = (None, "causal", "sliding_window", "prefix_lm")


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def variant_kw(mod, mask, window=37, window_causal=True, prefix=50):
    kw = dict(variant=mod if mask is None or mod != "vanilla" else mask)
    if mask is not None and mod != "vanilla":
        kw["mask"] = mask
    if mod == "softcap":
        kw["softcap"] = 50.0
    if mod == "alibi":
        kw["alibi_max_bias"] = 8.0
    if mask == "sliding_window":
        kw.update(window=window, window_causal=window_causal)
    if mask == "prefix_lm":
        kw["prefix"] = prefix
    return kw


def run_decode(q, kc, vc, seqlens, layout="bhsd", **kw):
    o, lse = api.fl_attn_decode_fwd(q.to(DEV), kc.to(DEV), vc.to(DEV), seqlens.to(DEV),
                                    layout=layout, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def run_oracle(q, kc, vc, seqlens, layout="bhsd", rows=None, **kw):
    kw = {k: v for k, v in kw.items() if k not in ("num_splits", "max_seqlen")}
    if layout == "bshd":
        kc, vc = kc.transpose(1, 2), vc.transpose(1, 2)
    return oracle.decode(np64(q), np64(kc), np64(vc), seqlens.numpy(), rows=rows, **kw)


def compare(q, kc, vc, seqlens, what, layout="bhsd", **kw):
    o, lse = run_decode(q, kc, vc, seqlens, layout=layout, **kw)
    ro, rl = run_oracle(q, kc, vc, seqlens, layout=layout, **kw)
    check(np64(o), ro, "bf16", what)
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "%s: lse %g" % (what, mx)
    return o, lse


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
def test_decode_small(mod, mask, splits):
    B, Hq, Hkv, Sq, S_cap = 5, 8, 2, 1, 700
    seed = 800 + 7 * MODS.index(mod) + MASKS.index(mask)
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, Sq, S_cap, 64, seed=seed)
    seqlens = torch.tensor([700, 333, 1, 0, 64], dtype=torch.int32)
    compare(q, kc, vc, seqlens, "%s+%s splits=%d" % (mod, mask, splits), num_splits=splits,
            **variant_kw(mod, mask))


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("mod", MODS)
def test_decode_large_logits(mod, splits):
    """Query rows scaled by 25 (logits of standard deviation about 25) at the
    default scale, whose scale * log2(e) is no power of two: the decode form
    applies the scale exactly, so O stays within the bf16 tolerance."""
    B, Hq, Hkv, Sq, S_cap = 3, 8, 2, 4, 500
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, Sq, S_cap, 64, seed=830)
    q = (q.float() * 25).to(torch.bfloat16)
    seqlens = torch.tensor([500, 200, 37], dtype=torch.int32)
    compare(q, kc, vc, seqlens, "%s large logits splits=%d" % (mod, splits), num_splits=splits,
            **variant_kw(mod, "causal"))


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mod", MODS)
def test_decode_several_new_tokens_bshd(mod, mask):
    # S_q = 5: positions L-5 .. L-1; a cache shorter than S_q puts rows before 0
    B, Hq, Hkv, Sq, S_cap = 4, 8, 2, 5, 520
    seed = 850 + 7 * MODS.index(mod) + MASKS.index(mask)
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, Sq, S_cap, 64, seed=seed, layout="bshd")
    seqlens = torch.tensor([520, 3, 129, 64], dtype=torch.int32)
    compare(q, kc, vc, seqlens, "%s+%s Sq=5" % (mod, mask), layout="bshd", num_splits=0,
            **variant_kw(mod, mask, window_causal=mask != "sliding_window" or mod != "alibi"))


@pytest.mark.parametrize("G,Sq", [(1, 1), (8, 1), (8, 20), (4, 40)])
def test_decode_group_shapes(G, Sq):
    # G * Sq above 128 rows spans several query tiles of one K/V head
    B, Hkv, S_cap = 2, 2, 1000
    q, kc, vc = inputs.decode_inputs(B, G * Hkv, Hkv, Sq, S_cap, 64, seed=900 + G + Sq)
    seqlens = torch.tensor([1000, 517], dtype=torch.int32)
    for kw in (dict(variant="causal"), dict(variant="alibi", mask="sliding_window", window=100)):
        compare(q, kc, vc, seqlens, "G=%d Sq=%d %s" % (G, Sq, kw), num_splits=0, **kw)


def test_decode_ignores_cache_past_length_and_clamps():
    B, Hq, Hkv, S_cap = 3, 4, 1, 300
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, 2, S_cap, 64, seed=950)
    seqlens = torch.tensor([300, 120, 7], dtype=torch.int32)
    clean, lc = run_decode(q, kc, vc, seqlens, num_splits=2, variant="softcap")
    kd, vd = kc.clone(), vc.clone()
    for b, L in enumerate(seqlens.tolist()):
        kd[b, :, L:] = float("nan")
        vd[b, :, L:] = float("nan")
    dirty, ld = run_decode(q, kd, vd, seqlens, num_splits=2, variant="softcap")
    assert torch.equal(clean, dirty) and torch.equal(lc, ld)
    # lengths above max_seqlen count as max_seqlen
    big = torch.tensor([5000, 120, 7], dtype=torch.int32)
    o, lse = run_decode(q, kc, vc, big, max_seqlen=200, variant="causal")
    ro, rl = run_oracle(q, kc, vc, torch.tensor([200, 120, 7], dtype=torch.int32),
                        variant="causal")
    check(np64(o), ro, "bf16", "clamped length")


def test_decode_empty_cache_and_split_agreement():
    B, Hq, Hkv, S_cap = 2, 4, 2, 4096
    q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, 1, S_cap, 64, seed=960)
    seqlens = torch.tensor([0, 4096], dtype=torch.int32)
    outs = []
    for splits in (1, 2, 7, 64):
        o, lse = run_decode(q, kc, vc, seqlens, num_splits=splits, variant="alibi")
        assert (o[0] == 0).all() and torch.isneginf(lse[0]).all()
        outs.append(np64(o[1]))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-2


def test_decode_matches_prefill_tail():
    """The decode of the last tokens equals the last rows of the prefill over
    the same tokens (both on the GPU, both against the oracle)."""
    Hq, Hkv, L, Sq = 8, 2, 777, 3
    q, k, v = inputs.attn_inputs(1, Hq, Hkv, L, L, 64, seed=970)
    for kw in (dict(variant="causal"), dict(variant="softcap", mask="causal"),
               dict(variant="alibi", mask="sliding_window", window=300)):
        pre = api.fl_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
        dec = api.fl_attn_decode_fwd(q[:, :, L - Sq:].contiguous().to(DEV), k.to(DEV), v.to(DEV),
                                     torch.tensor([L], dtype=torch.int32, device=DEV), **kw)
        torch.cuda.synchronize()
        assert np.abs(np64(dec) - np64(pre[:, :, L - Sq:])).max() < 2e-2, kw


def test_decode_full_workload_sampled():
    wl = inputs.WORKLOADS["decode_bf16_b64_hq32_hkv8_cap8192_d64"]
    t = inputs.make(wl)
    g = {k: v.to(DEV) for k, v in t.items()}
    pick = np.array([0, 5, 17, 42, 63])
    L = t["seqlens"]
    sub = {k: t[k][pick].contiguous() for k in ("q", "k_cache", "v_cache")}
    for vname in wl.variants:
        kw = dict(variant=vname)
        for key in ("softcap", "alibi_max_bias", "window", "window_causal"):
            if key in wl.params:
                kw[key] = wl.params[key]
        o, lse = api.fl_attn_decode_fwd(g["q"], g["k_cache"], g["v_cache"], g["seqlens"],
                                        max_seqlen=int(L.max()), return_lse=True, **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all()
        ro, rl = oracle.decode(np64(sub["q"]), np64(sub["k_cache"]), np64(sub["v_cache"]),
                               L[pick].numpy(), **kw)
        check(np64(o[pick]), ro, "bf16", "decode " + vname)
        mx, _, _ = errors(np64(lse[pick]), rl)
        assert mx <= 2e-2, (vname, mx)


# ---------------------------------------------------------------------------
# merge


@pytest.mark.parametrize("D", [64, 100])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_merge_against_oracle(D, out_dtype):
    rng = np.random.default_rng(990 + D)
    P, rows = 5, 300
    o_parts = rng.standard_normal((P, rows, D)).astype(np.float32)
    lse_parts = (rng.standard_normal((P, rows)) * 4).astype(np.float32)
    lse_parts[1, ::3] = -np.inf        # empty parts
    o_parts[1, ::3] = 0.0
    lse_parts[:, 7] = -np.inf          # a row with no key at all
    o_parts[:, 7] = 0.0
    o, lse = api.fl_attn_merge(torch.from_numpy(o_parts).to(DEV), torch.from_numpy(lse_parts).to(DEV),
                               out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.merge(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    check(np64(o), ro, "bf16" if out_dtype == torch.bfloat16 else "f32", "merge D=%d" % D)
    assert (np64(o)[7] == 0).all() and np.isneginf(np64(lse)[7])
    mx, _, _ = errors(np64(lse), rl)
    assert mx < 1e-5


def test_merge_of_attention_over_key_halves():
    """Attention over two halves of the keys, merged on the GPU, is attention
    over all of them."""
    B, H, S = 2, 4, 640
    q, k, v = inputs.attn_inputs(B, H, H, 100, S, 64, "f32", seed=995)
    parts = [api.fl_attn_fwd(q.to(DEV), k[:, :, a:b].contiguous().to(DEV),
                             v[:, :, a:b].contiguous().to(DEV), return_lse=True)
             for a, b in ((0, 300), (300, S))]
    o, lse = api.fl_attn_merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]),
                               out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(np64(q), np64(k), np64(v))
    check(np64(o), ro, "f32", "merged halves")
    check(np64(lse), rl, "f32", "merged halves lse")


def test_decode_large_cache_offsets_bshd():
    # One sequence whose [S_cap, H_kv, D] cache block spans 1.5 GiB, so tile
    # byte offsets run past 2^30 (the launcher's limit is 2^31).  The cache is
    # a seeded 4096-row block repeated with a position ramp added to V, so a
    # wrong row (or a zero read) anywhere changes the output.
    Hq, Hkv, D, S_cap = 4, 4, 64, 3_000_000
    L = S_cap - 37
    q, kb, vb = inputs.decode_inputs(1, Hq, Hkv, 1, 4096, D, seed=990, layout="bshd")
    reps = (S_cap + 4095) // 4096
    kc = kb.repeat(1, reps, 1, 1)[:, :S_cap].contiguous()
    ramp = torch.linspace(-1.0, 1.0, S_cap, dtype=torch.float32).view(1, S_cap, 1, 1)
    vc = (vb.repeat(1, reps, 1, 1)[:, :S_cap].float() + ramp).to(torch.bfloat16).contiguous()
    seqlens = torch.tensor([L], dtype=torch.int32)
    o, lse = run_decode(q, kc, vc, seqlens, layout="bshd", variant="causal", num_splits=0)
    ro, rl = run_oracle(q, kc, vc, seqlens, layout="bshd", variant="causal")
    check(np64(o), ro, "bf16", "1.5 GiB cache block")
    mx, _, _ = errors(np64(lse), rl)
    assert mx <= 2e-2, "lse %g" % mx
