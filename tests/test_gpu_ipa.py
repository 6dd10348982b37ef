"""GPU parity of the Invariant Point Attention core: the HIP path through the
C ABI against the float64 oracle on the same seeded inputs.

Tolerances: o and o_pair are bf16 outputs of float32 arithmetic (the pair
output's weights rounded to bf16 for the matrix cores), held to the bf16
bar of the other kernels (max-abs 2e-2, mean-abs 2e-3).  o_pts is a float32
output of float32 arithmetic on coordinates of up to about 60 angstroms:
one rounding of such a coordinate is 60 * 2^-24 = 4e-6, the weights carry
relative errors of a few 1e-6 from the logits (float32, |logit| up to ~10^2
before the maximum is subtracted), and the weighted mean and the return to
the query's frame add a few roundings more, so 1e-3 max-abs and 1e-4
mean-abs leave a margin of about 100.
"""
import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
PTS_MAX_ABS, PTS_MEAN_ABS = 1e-3, 1e-4


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


def run_both(t, rows=None, with_bias=True, with_z=True, with_mask=True):
    g = {n: x.to(DEV) for n, x in t.items()}
    o, op, oz = api.fl_ipa_attn_fwd(g["q"], g["k"], g["v"], g["q_pts"], g["k_pts"], g["v_pts"],
                                    g["rot"], g["trans"], g["gamma"],
                                    pair_bias=g["pair_bias"] if with_bias else None,
                                    z=g["z"] if with_z else None,
                                    key_mask=g["key_mask"] if with_mask else None)
    torch.cuda.synchronize()
    c = {n: np64(x) for n, x in t.items()}
    ro, rp, rz = oracle.ipa(c["q"], c["k"], c["v"], c["q_pts"], c["k_pts"], c["v_pts"], c["rot"],
                            c["trans"], c["gamma"], pair_bias=c["pair_bias"] if with_bias else None,
                            z=c["z"] if with_z else None,
                            key_mask=t["key_mask"].numpy() if with_mask else None, rows=rows)
    return (o, op, oz), (ro, rp, rz)


def compare(got, want, what, rows=None):
    o, op, oz = got
    ro, rp, rz = want
    sel = (lambda x: x.reshape(-1, *x.shape[3:])[rows]) if rows is not None else (lambda x: x)
    check(sel(np64(o)), ro, "bf16", what + " o")
    mx, mean, _ = errors(sel(np64(op)), rp)
    assert mx <= PTS_MAX_ABS and mean <= PTS_MEAN_ABS, "%s o_pts: max %.3g mean %.3g" % (what, mx, mean)
    if rz is not None:
        check(sel(np64(oz)), rz, "bf16", what + " o_pair")
    else:
        assert oz is None


@pytest.mark.parametrize("L", [1, 37, 64, 100, 130])
@pytest.mark.parametrize("H", [1, 3, 12])
def test_ipa_shapes(L, H):
    """Ragged key tiles (L % 64 != 0), head groups with idle waves (H = 1, 3),
    residue counts that do and do not split over the 8 XCDs."""
    t = inputs.ipa_inputs(2, L, H, 16, 4, 8, 128, "bf16", seed=1000 + L + H, masked_frac=0.1)
    got, want = run_both(t)
    compare(got, want, "L=%d H=%d" % (L, H))


@pytest.mark.parametrize("cz", [0, 64, 128])
@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("with_mask", [True, False])
def test_ipa_options(cz, with_bias, with_mask):
    t = inputs.ipa_inputs(1, 96, 4, 16, 4, 8, cz or 128, "bf16", seed=1100 + cz, masked_frac=0.2)
    if cz == 64:
        t["z"] = t["z"][..., :64].contiguous()
    got, want = run_both(t, with_bias=with_bias, with_z=cz > 0, with_mask=with_mask)
    compare(got, want, "cz=%d bias=%s mask=%s" % (cz, with_bias, with_mask))


def test_ipa_masked_keys_and_empty_rows():
    """A batch entry with one key kept, one with none: the first returns that
    key's value, value points in each query's frame and pair features; the
    second returns zeros."""
    t = inputs.ipa_inputs(3, 70, 5, 16, 4, 8, 128, "bf16", seed=1200)
    t["key_mask"][0] = 0
    t["key_mask"][0, 33] = 1
    t["key_mask"][1] = 0
    got, want = run_both(t)
    compare(got, want, "masked")
    o, op, oz = got
    assert (np64(o)[1] == 0).all() and (np64(op)[1] == 0).all() and (np64(oz)[1] == 0).all()


def test_ipa_sharp_point_term():
    """Large gamma: the point term dominates (weights concentrate on the
    nearest residues, logits spanning thousands of base-2 units), so the
    running maximum must move across tiles."""
    t = inputs.ipa_inputs(1, 200, 4, 16, 4, 8, 128, "bf16", seed=1300)
    t["gamma"] = t["gamma"] * 40
    got, want = run_both(t)
    compare(got, want, "sharp")


def test_ipa_rigid_motion_on_gpu():
    """The GPU outputs are invariant under a global rigid motion of every
    frame (within the float32 rounding of the moved frames)."""
    t = inputs.ipa_inputs(1, 128, 12, 16, 4, 8, 128, "bf16", seed=1400)
    base, _ = run_both(t)
    Qm, Rm = np.linalg.qr(np.random.default_rng(45).standard_normal((3, 3)))
    G = Qm * np.sign(np.diag(Rm))
    if np.linalg.det(G) < 0:
        G[:, 0] = -G[:, 0]
    moved = dict(t)
    moved["rot"] = torch.from_numpy(np.einsum("xy,blyz->blxz", G, t["rot"].double().numpy())).float()
    moved["trans"] = torch.from_numpy(np.einsum("xy,bly->blx", G, t["trans"].double().numpy())
                                      + np.array([20.0, -5.0, 11.0])).float()
    out, want = run_both(moved)
    compare(out, want, "moved")
    assert np.abs(np64(out[1]) - np64(base[1])).max() < 2e-3
    check(np64(out[0]), np64(base[0]), "bf16", "o invariance")


def test_ipa_full_structure_module_shape():
    """AlphaFold2's structure-module shape (256 residues, 12 heads, C_z 128),
    every output of every row against the oracle."""
    wl = inputs.WORKLOADS["ipa_bf16_nres256_h12"]
    t = inputs.make(wl)
    got, want = run_both(t)
    compare(got, want, "structure module")
