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


def decode_attention(q, k_cache, v_cache, seqlens, *, variant="vanilla", scale=None, softcap=50.0,
                     alibi_max_bias=8.0, window=1, window_causal=True, prefix=0, mask=None):
    """Decode against a KV cache, by brute force: for each batch entry the
    cache is cut to its length L, the Sq queries are given the positions of
    the last Sq tokens (L - Sq .. L - 1), and the mask and ALiBi distances are
    built from those position vectors."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k_cache, v_cache))
    B, Hq, Sq, D = q.shape
    Hkv, S_cap, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    kind = mask or variant
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        L = int(min(max(seqlens[b], 0), S_cap))
        qpos = np.arange(L - Sq, L)
        kpos = np.arange(L)
        rel = qpos[:, None] - kpos[None, :]  # query position minus key position
        if kind in ("vanilla", "alibi", "softcap"):
            allowed = np.ones((Sq, L), bool)
        elif kind == "causal":
            allowed = rel >= 0
        elif kind == "sliding_window":
            allowed = (rel >= 0) & (rel < window) if window_causal else np.abs(rel) < window
        elif kind == "prefix_lm":
            allowed = (rel >= 0) | (kpos[None, :] < prefix)
        else:
            raise ValueError(kind)
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // G, :L].T)
            if variant == "alibi":
                s = s - 2.0 ** (-alibi_max_bias * (h + 1) / Hq) * np.abs(rel)
            if variant == "softcap":
                s = softcap * np.tanh(s / softcap)
            s = np.where(allowed, s, -np.inf)
            rows = allowed.any(1)
            l = np.full(Sq, -np.inf)
            if rows.any():
                l[rows] = logsumexp(s[rows], axis=1)
                p = np.zeros_like(s)
                p[rows] = np.exp(s[rows] - l[rows, None])
                o[b, h] = p @ v[b, h // G, :L]
            lse[b, h] = l
    return o, lse
