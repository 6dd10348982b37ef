"""Shared helpers of the GPU parity tests: tolerance checks and row sampling."""
import numpy as np
import torch

# bf16 inputs with float32 accumulation: every output element within 2e-2 of
# the float64 oracle and their mean distance within 2e-3; float32 inputs:
# within 1e-4 (on O and on LSE).
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4


def np64(t):
    """Exact float64 copy of a GPU/CPU tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def errors(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    with np.errstate(invalid="ignore"):  # inf - inf where both are the same infinity
        diff = np.where(both_inf, 0.0, got - want)
    d = np.abs(diff)
    rel = np.linalg.norm(diff) / max(np.linalg.norm(np.where(both_inf, 0, want)), 1e-30)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0, float(rel)


def check(got, want, dtype, what=""):
    mx, mean, rel = errors(got, want)
    assert np.isfinite(mx), "%s: non-finite error" % what
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, \
            "%s: max-abs %.3g mean-abs %.3g rel-l2 %.3g" % (what, mx, mean, rel)
    else:
        assert mx <= F32_MAX_ABS, "%s: max-abs %.3g rel-l2 %.3g" % (what, mx, rel)
    return mx, mean, rel


def sample_rows(B, H, S, n, seed, extra_tiles=(64, 128, 256)):
    """Flat row indices (b*H + h)*S + i: n random rows plus the first and last
    row of every head sampled and rows on both sides of tile boundaries."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(B * H * S, size=min(n, B * H * S), replace=False).tolist())
    for bh in rng.choice(B * H, size=min(4, B * H), replace=False):
        base = int(bh) * S
        rows.update([base, base + S - 1])
        for t in extra_tiles:
            for i in (t - 1, t, S - t, S - t - 1):
                if 0 <= i < S:
                    rows.add(base + i)
    return np.array(sorted(rows), np.int64)


def gpu_rows(t, rows):
    """Rows of a [B,H,S,D] tensor at flat indices, as float64 [n, D]."""
    B, H, S, D = t.shape
    return np64(t.reshape(B * H * S, D)[torch.as_tensor(rows, device=t.device)])
