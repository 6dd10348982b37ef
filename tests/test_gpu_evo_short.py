"""GPU parity of Evoformer gated attention over rows of at most 256 positions.

Rows of at most 256 positions run on the kernel whose work-groups hold a
whole (entry, head) and walk several entries of one head: with the row
form's pair bias held in registers and added through the matrix cores, or
without a bias at three waves per SIMD; rows past 256 positions run on the
general kernel's gated form.  Each
case is compared element by element with the float64 oracle (papers.lqhl.me
wiki, "设计取舍": a bias broadcast over an extra dimension; AlphaFold2's
row- and column-wise gated self-attention).

Shapes are picked so that the short-row kernel's work-group count rule
gives several entries per work-group with a shorter last group (131 MSA
rows at 8 heads: five entries per work-group, 27 groups), and so that the
row lengths cross every instance boundary (64, 128 and 256 positions) and
end in ragged key units.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def run(axis, N_seq, N_res, H, seed, *, with_bias=True, with_mask=True, scale=None, q_mul=None,
        edit_mask=None, rows=None):
    q, k, v, gate, bias, km = inputs.evoformer_inputs(N_seq, N_res, H, 32, "bf16", seed)
    if q_mul is not None:
        q = (q.float() * q_mul).to(torch.bfloat16)
    if edit_mask is not None:
        edit_mask(km)
    pb = bias if (with_bias and axis == "row") else None
    kmask = km if with_mask else None
    o = api.fl_evoformer_gated_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gate.to(DEV),
                                        pair_bias=None if pb is None else pb.to(DEV),
                                        key_mask=None if kmask is None else kmask.to(DEV),
                                        axis=axis, scale=scale)
    torch.cuda.synchronize()
    ro = oracle.evoformer(np64(q), np64(k), np64(v), np64(gate),
                          pair_bias=None if pb is None else np64(pb),
                          key_mask=None if kmask is None else kmask.numpy(), axis=axis,
                          scale=scale, rows=rows)
    got = np64(o)
    if rows is not None:
        C = q.shape[-1]
        if axis == "row":
            got = got.reshape(-1, C)[rows]
        else:
            Hh = q.shape[2]
            h, s_, r_ = rows % Hh, (rows // Hh) % N_seq, rows // (Hh * N_seq)
            got = got[s_, r_, h]
    check(got, ro, "bf16", "evoformer %s N_seq=%d N_res=%d H=%d" % (axis, N_seq, N_res, H))
    return got, ro, km


@pytest.mark.parametrize("N_res", [8, 56, 64, 72, 128, 136, 256])
@pytest.mark.parametrize("with_bias", [True, False])
def test_row_lengths(N_res, with_bias):
    """Row form at lengths on both sides of the 64/128/256 instance limits
    (the pair bias needs N_res % 8 == 0)."""
    run("row", 5, N_res, 3, 300 + N_res, with_bias=with_bias)


@pytest.mark.parametrize("N_seq", [1, 2, 33, 64, 65, 100, 128, 129, 255, 256])
def test_col_lengths(N_seq):
    """Column form (no bias) at lengths 1 .. 256, ragged key units included."""
    run("col", N_seq, 6, 2, 400 + N_seq)


def test_row_multi_entry_walk():
    """131 MSA rows x 256 residues x 8 heads: 27 work-groups per head, each
    walking five MSA rows (the last group one), with two fully masked MSA
    rows, one of them the last entry of a work-group."""
    def edit(km):
        km[7, :] = 0
        km[9, :] = 0
    rng = np.random.default_rng(11)
    rows = np.unique(rng.choice(131 * 256 * 8, 6000, replace=False))
    # every query row of entries 0..10 of head 5 (covers the masked rows,
    # the hand-over between the first two groups and a whole walk)
    extra = [((s * 256 + r) * 8 + 5) for s in range(11) for r in range(256)]
    rows = np.unique(np.concatenate([rows, np.array(extra, np.int64)]))
    got, ro, _ = run("row", 131, 256, 8, 501, edit_mask=edit, rows=rows)
    for s in (7, 9):
        sel = (rows // (256 * 8)) == s
        assert sel.any() and (got[sel] == 0).all()


def test_col_multi_entry_walk():
    """128 sequences x 71 residue columns x 8 heads: columns walked two or
    three per work-group, the last group shorter; a fully masked column."""
    def edit(km):
        km[:, 4] = 0
    got, ro, _ = run("col", 128, 71, 8, 502, edit_mask=edit)
    assert (got[:, 4] == 0).all()


@pytest.mark.parametrize("axis", ["row", "col"])
def test_large_logits_checked_pass(axis):
    """Queries scaled by 25 (and by 60 for the row form, whose bias keeps
    the sums of some rows in range): rows whose first-pass sums leave
    [2^-60, 2^100] rerun with the running reference."""
    for mul in (25.0, 60.0):
        if axis == "row":
            run("row", 4, 128, 2, 601, q_mul=mul)
        else:
            run("col", 128, 5, 2, 602, q_mul=mul)


def test_scales_and_no_mask():
    """A negative scale (sign through the exact power-of-two factor), a zero
    scale (uniform weights over the allowed keys, the bias alone in the row
    form), and no key mask."""
    run("row", 4, 96, 2, 701, scale=-1.0 / np.sqrt(32))
    run("row", 4, 96, 2, 702, scale=0.0)
    run("col", 96, 4, 2, 703, scale=0.0)
    run("row", 4, 256, 2, 704, with_mask=False)
    run("col", 200, 4, 2, 705, with_mask=False)


def test_all_keys_masked_but_one():
    """Entries with a single allowed key return that key's gated value."""
    def edit(km):
        km[:] = 0
        km[:, 17] = 1
    got, ro, _ = run("row", 3, 64, 2, 801, edit_mask=edit)


@pytest.mark.parametrize("axis,n,with_bias", [("row", 264, True), ("row", 300, False), ("col", 300, False)])
def test_long_rows_general_kernel(axis, n, with_bias):
    """Rows longer than 256 positions take the general kernel's gated form."""
    if axis == "row":
        run("row", 3, n, 2, 900 + n, with_bias=with_bias)
    else:
        run("col", n, 3, 2, 900 + n)


def test_row_odd_heads_multi_entry():
    """100 MSA rows x 256 residues x 3 heads: two MSA rows per work-group,
    head pairs dealt to one XCD with the second head of the last pair
    missing (those work-groups end at once), compared on sampled rows."""
    rng = np.random.default_rng(13)
    rows = np.unique(rng.choice(100 * 256 * 3, 5000, replace=False))
    # every query row of head 2 (the unpaired head) of MSA rows 0..3
    extra = [((s * 256 + r) * 3 + 2) for s in range(4) for r in range(256)]
    rows = np.unique(np.concatenate([rows, np.array(extra, np.int64)]))
    run("row", 100, 256, 3, 1001, rows=rows)
