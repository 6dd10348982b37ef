"""Host logic: useful-FLOP closed forms against brute-force pair counts, and
the seeded input generators."""
import numpy as np
import pytest
import torch

from flashattention_attention_variants_amd import flops, inputs
from tests import _bruteforce as bf


@pytest.mark.parametrize("S", [1, 7, 64, 300])
@pytest.mark.parametrize("variant", ["vanilla", "causal", "sliding_window", "prefix_lm", "document"])
def test_allowed_pairs_closed_forms(variant, S):
    for window, wc, prefix in ((1, True, 0), (5, True, 3), (64, False, 64), (1000, True, 1000),
                               (7, False, 1)):
        offs = inputs.doc_offsets(1, S, min(4, S), seed=S)[0].numpy()
        m = bf.mask_matrix(variant, S, S, window=window, window_causal=wc, prefix=prefix,
                           offsets=offs)
        got = flops.allowed_pairs(variant, S, S, window=window, window_causal=wc, prefix=prefix,
                                  doc_offsets=offs)
        assert got == int(m.sum()), (variant, S, window, wc, prefix)


def test_headline_flop_counts():
    # B4 H16 S4096 D64: vanilla 2*S^2*128 per head
    assert flops.attn_flops("vanilla", 4, 16, 4096, 4096, 64) == 2 * 4096 ** 2 * 128 * 64
    assert flops.attn_flops("causal", 4, 16, 4096, 4096, 64) == 2 * (4096 * 4097 // 2) * 128 * 64
    assert flops.roofline_tflops(1.0, 1.0)[0] == "hbm"
    assert flops.roofline_tflops(1e6, 1.0)[0] == "mfma"


def test_doc_offsets_are_compositions():
    offs = inputs.doc_offsets(6, 2048, 8, seed=2002)
    assert offs.shape == (6, 9) and offs.dtype == torch.int32
    for row in offs.numpy():
        assert row[0] == 0 and row[-1] == 2048 and (np.diff(row) > 0).all()
    assert torch.equal(offs, inputs.doc_offsets(6, 2048, 8, seed=2002))


def test_inputs_seeded_and_rounded():
    a = inputs.attn_inputs(1, 2, 1, 8, 8, 64, "bf16", seed=3)
    b = inputs.attn_inputs(1, 2, 1, 8, 8, 64, "bf16", seed=3)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert a[0].dtype == torch.bfloat16 and a[1].shape == (1, 1, 8, 64)
    # bf16 values are the round-to-nearest-even images of the float32 draw
    g = torch.Generator().manual_seed(3)
    f = torch.randn(1, 2, 8, 64, generator=g)
    assert torch.equal(a[0], f.to(torch.bfloat16))
    q, k, v, gate, bias, km = inputs.evoformer_inputs(16, 32, 2, 32, "bf16", seed=5)
    assert km.dtype == torch.uint8 and 0.8 < km.float().mean() < 1.0


@pytest.mark.parametrize("mask", [None, "causal", "sliding_window", "prefix_lm"])
@pytest.mark.parametrize("wc", [True, False])
def test_decode_pairs_and_keys_bruteforce(mask, wc):
    """Decode pair counts and the keys any row needs, against the brute-force
    decode's own allowed matrix (a key's row of weights is non-zero exactly
    where it is allowed, with V = identity)."""
    for L, Sq in ((1, 1), (9, 3), (40, 1), (40, 7), (2, 5)):
        q = np.zeros((1, 1, Sq, 4))
        kc = np.zeros((1, 1, L, 4))
        vc = np.eye(L)[None, None] if L else np.zeros((1, 1, 0, 0))
        kw = dict(window=4, window_causal=wc, prefix=6)
        p, _ = bf.decode_attention(q, kc, vc, [L], variant=mask or "vanilla", **kw)
        allowed = p[0, 0] > 0
        pairs, keys = flops.decode_keys(mask, L, Sq, **kw)
        assert pairs == int(allowed.sum())
        cols = np.nonzero(allowed.any(0))[0]
        assert keys == (0 if cols.size == 0 else cols.max() - cols.min() + 1)


def test_decode_inputs_and_lengths():
    q, k, v = inputs.decode_inputs(2, 4, 2, 3, 10, 64, "bf16", seed=9)
    q2, k2, v2 = inputs.decode_inputs(2, 4, 2, 3, 10, 64, "bf16", seed=9, layout="bshd")
    assert k.shape == (2, 2, 10, 64) and k2.shape == (2, 10, 2, 64)
    assert torch.equal(k2.transpose(1, 2), k) and torch.equal(q, q2)
    L = inputs.cache_lengths(1000, 512, 8192, seed=7007)
    assert L.dtype == torch.int32 and int(L.min()) >= 512 and int(L.max()) <= 8192
    assert 4000 < float(L.float().mean()) < 4700
