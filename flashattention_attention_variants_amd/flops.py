"""Useful work and algorithmic bytes of each attention call (closed forms).

Useful FLOPs count only the two products on allowed (query, key) pairs:
2*N*D for Q K^T plus 2*N*D_v for P V, where N is the exact number of allowed
pairs of one (batch, head).  Exponentials and masked pairs are not counted.
Algorithmic bytes count every input read once and every output written once;
they never include the score matrix the fused kernel avoids.
"""
from __future__ import annotations

import numpy as np

# MI355X published peaks
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 matrix cores (256 CU x 2.4 GHz x 4096 = 2516.6)
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def allowed_pairs(variant: str, S_q: int, S_k: int, *, window: int = 256, window_causal=True,
                  prefix: int = 512, doc_offsets=None) -> int:
    """Allowed (i, j) pairs of one (batch, head); doc_offsets is one row [n+1]."""
    if variant in ("vanilla", "alibi", "softcap"):
        return S_q * S_k
    S = S_q
    if variant == "causal":
        return S * (S + 1) // 2
    if variant == "sliding_window":
        W = min(window, S)
        if window_causal:
            # row i sees min(i+1, W) keys
            return W * (W + 1) // 2 + (S - W) * W
        # row i sees keys with |i - j| < W inside [0, S)
        i = np.arange(S)
        return int((np.minimum(i + W - 1, S - 1) - np.maximum(i - W + 1, 0) + 1).sum())
    if variant == "prefix_lm":
        P = min(max(prefix, 0), S)
        if P == 0:
            return S * (S + 1) // 2
        # rows i < P see P keys; rows i >= P see i+1 keys
        return P * P + (S * (S + 1) - P * (P + 1)) // 2
    if variant == "document":
        lens = np.diff(np.asarray(doc_offsets, np.int64))
        return int((lens * lens).sum())
    raise ValueError(variant)


def attn_flops(variant, B, Hq, S_q, S_k, D, Dv=None, doc_offsets=None, **kw) -> int:
    Dv = Dv or D
    if variant == "document":
        n = sum(allowed_pairs(variant, S_q, S_k, doc_offsets=doc_offsets[b]) for b in range(B)) * Hq
    else:
        n = allowed_pairs(variant, S_q, S_k, **kw) * B * Hq
    return 2 * n * (D + Dv)


def attn_bytes(B, Hq, Hkv, S_q, S_k, D, Dv=None, elem=2, lse=False, bias=False) -> int:
    Dv = Dv or D
    b = elem * (B * Hq * S_q * D + B * Hkv * S_k * (D + Dv) + B * Hq * S_q * Dv)
    if lse:
        b += 4 * B * Hq * S_q
    if bias:
        b += elem * Hq * S_q * S_k
    return b


def attn_bwd_flops(variant, B, Hq, S_q, S_k, D, **kw) -> int:
    """Useful FLOPs of the backward: the five products on allowed pairs (S
    recomputed, dP, dV, dK, dQ), i.e. 2.5 times the forward's two; the dQ
    launch's second recomputation of S and dP is not counted."""
    return attn_flops(variant, B, Hq, S_q, S_k, D, **kw) * 5 // 2


def diffattn_flops(B, H, S, Dqk, Dv, causal) -> int:
    n = (S * (S + 1) // 2 if causal else S * S) * B * H
    return 2 * 2 * n * (Dqk + Dv)


def diffattn_bytes(B, H, S, Dqk, Dv, elem=2) -> int:
    return elem * B * H * S * (4 * Dqk + Dv + Dv)


def evoformer_flops(N_seq, N_res, H, C, axis) -> int:
    rows, L = (N_seq, N_res) if axis == "row" else (N_res, N_seq)
    return 4 * C * L * L * rows * H


def evoformer_bytes(N_seq, N_res, H, C, axis, elem=2) -> int:
    b = elem * 5 * N_seq * N_res * H * C + N_seq * N_res  # q, k, v, gate, o + key mask
    if axis == "row":
        b += elem * H * N_res * N_res                      # pair bias
    return b


def decode_keys(mask, L: int, S_q: int, *, window: int = 256, window_causal=True,
                prefix: int = 512):
    """(allowed pairs, keys any row needs) of one (sequence, head) in decode:
    the S_q queries sit at positions L-S_q .. L-1 and see keys 0 .. L-1.
    ``mask`` is None (no mask) or a mask variant name."""
    pairs, lo_u, hi_u = 0, None, None
    for pos in range(L - S_q, L):
        if mask in (None, "vanilla", "alibi", "softcap"):
            lo, hi = 0, L - 1
        elif mask == "causal":
            lo, hi = 0, pos
        elif mask == "sliding_window":
            lo = pos - window + 1
            hi = pos if window_causal else pos + window - 1
        elif mask == "prefix_lm":
            lo, hi = 0, max(pos, prefix - 1)
        else:
            raise ValueError(mask)
        lo, hi = max(lo, 0), min(hi, L - 1)
        if lo > hi:
            continue
        pairs += hi - lo + 1
        lo_u = lo if lo_u is None else min(lo_u, lo)
        hi_u = hi if hi_u is None else max(hi_u, hi)
    return pairs, (0 if lo_u is None else hi_u - lo_u + 1)


def decode_work(mask, lengths, Hq, Hkv, S_q, D, elem=2, lse=False, **kw):
    """(useful FLOPs, algorithmic bytes) of a decode call: the K/V rows some
    query needs, read once per K/V head, plus q and o."""
    f, b = 0, 0
    for L in lengths:
        pairs, keys = decode_keys(mask, int(L), S_q, **kw)
        f += 2 * pairs * 2 * D * Hq
        b += elem * keys * 2 * D * Hkv
    rows = len(lengths) * Hq * S_q
    b += elem * 2 * rows * D + (4 * rows if lse else 0)
    return f, b


def roofline_tflops(flops: float, nbytes: float, peak_tflops=PEAK_BF16_TFLOPS,
                    hbm_gbs=PEAK_HBM_GBS):
    """(bound, attainable TFLOP/s) of a kernel with that work and traffic."""
    mem = hbm_gbs * 1e9 * flops / nbytes / 1e12
    return ("mfma", peak_tflops) if peak_tflops <= mem else ("hbm", mem)


def ipa_work(B, L, H, C, Pq, Pv, Cz, elem=2, masked_keys=0):
    """(useful FLOPs, algorithmic bytes) of one Invariant Point Attention
    core call.  Per allowed (query, key, head) triple the products are
    counted as multiply-adds: the scalar logit (C), the point distances
    (3 Pq), and the three weighted sums (C values, 3 Pv point coordinates,
    Cz pair features).  Bytes: q, k, v, pair bias, z and the outputs o,
    o_pair in the compute dtype; points, frames and o_pts in float32; gamma
    and the u8 key mask."""
    pairs = B * H * L * (L - masked_keys)
    f = 2 * pairs * (C + 3 * Pq + C + 3 * Pv + Cz)
    nb = elem * (3 * B * L * H * C + B * H * L * L + B * L * L * Cz + B * L * H * (C + Cz))
    nb += 4 * (B * L * H * 3 * (2 * Pq + Pv) + B * L * 12 + H + B * L * H * 3 * Pv) + B * L
    return f, nb
