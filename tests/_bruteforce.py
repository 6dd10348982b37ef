"""Independent brute-force attention for tiny inputs (tests only).

It materialises the whole score matrix with numpy, builds each mask as an
explicit boolean matrix with its own construction (triangles, distance bands,
document-id equality), and normalises with ``scipy.special.logsumexp``.  It
shares no code with the oracle, which walks rows and keys one at a time.
"""
import numpy as np
from scipy.special import logsumexp


def mask_matrix(variant, Sq, Sk, *, window=1, window_causal=True, prefix=0, offsets=None):
    if variant in ("vanilla", "alibi", "softcap"):
        return np.ones((Sq, Sk), bool)
    tri = np.tril(np.ones((Sq, Sk), bool))  # j <= i
    if variant == "causal":
        return tri
    if variant == "sliding_window":
        dist = np.arange(Sq)[:, None] - np.arange(Sk)[None, :]
        if window_causal:
            return tri & (dist < window)
        return np.abs(dist) < window
    if variant == "prefix_lm":
        m = tri.copy()
        m[:, :prefix] = True
        return m
    if variant == "document":
        lengths = np.diff(np.asarray(offsets))
        ids = np.repeat(np.arange(len(lengths)), lengths)
        return ids[:Sq, None] == ids[None, :Sk]
    raise ValueError(variant)


def attention(q, k, v, *, variant="vanilla", scale=None, bias=None, softcap=50.0,
              alibi_max_bias=8.0, window=1, window_causal=True, prefix=0, doc_offsets=None,
              mask=None):
    """q [B,Hq,Sq,D], k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv] -> (o, lse), float64.
    ``mask`` composes a mask variant with the score modification of ``variant``."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        allowed = mask_matrix(mask or variant, Sq, Sk, window=window, window_causal=window_causal,
                              prefix=prefix,
                              offsets=None if doc_offsets is None else doc_offsets[b])
        for h in range(Hq):
            kk, vv = k[b, h // G], v[b, h // G]
            s = scale * (q[b, h] @ kk.T)
            if variant == "alibi":
                slope = 2.0 ** (-alibi_max_bias * (h + 1) / Hq)
                s = s - slope * np.abs(np.subtract.outer(np.arange(Sq), np.arange(Sk)))
            if variant == "softcap":
                s = softcap * np.tanh(s / softcap)
            if bias is not None:
                s = s + np.asarray(bias, np.float64)[h]
            s = np.where(allowed, s, -np.inf)
            rows = allowed.any(1)
            l = np.full(Sq, -np.inf)
            l[rows] = logsumexp(s[rows], axis=1)
            p = np.zeros_like(s)
            p[rows] = np.exp(s[rows] - l[rows, None])
            o[b, h] = p @ vv
            lse[b, h] = l
    return o, lse
