"""CPU float64 oracle for the fused attention-variant forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  It shares
no code with the GPU library.  The arithmetic lives in ``oracle.c`` (plain C,
float64, two passes per query row); this module only marshals numpy arrays
through ctypes.

Every function takes float64 (or uint8 / int32 where stated) numpy arrays in
the layouts documented in ``oracle.h`` and returns float64 outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

VANILLA, ALIBI, SOFTCAP, CAUSAL, SLIDING_WINDOW, PREFIX_LM, DOCUMENT = range(7)
VARIANTS = {
    "vanilla": VANILLA,
    "alibi": ALIBI,
    "softcap": SOFTCAP,
    "causal": CAUSAL,
    "sliding_window": SLIDING_WINDOW,
    "prefix_lm": PREFIX_LM,
    "document": DOCUMENT,
}


_SOURCES = ("oracle.c", "ipa.c", "oracle.h")


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` and ``ipa.c`` into ``liboracle.so`` with gcc (no GPU code)."""
    srcs = [os.path.join(_HERE, f) for f in _SOURCES]
    newest = max(os.path.getmtime(f) for f in srcs)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < newest:
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-o", tmp, *[f for f in srcs if f.endswith(".c")], "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Params(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int),
        ("scale", ctypes.c_double),
        ("softcap", ctypes.c_double),
        ("alibi_max_bias", ctypes.c_double),
        ("window", ctypes.c_int),
        ("window_causal", ctypes.c_int),
        ("prefix", ctypes.c_int),
        ("doc_offsets", ctypes.c_void_p),
        ("n_docs", ctypes.c_int),
        ("mask", ctypes.c_int),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_attn_rows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I,
                                         ctypes.POINTER(_Params), P, I64, I, I]
        lib.oracle_diffattn_rows.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                             D, D, I, P, I64, I]
        lib.oracle_evoformer_row.argtypes = [P, P, P, P, P, P, P, I, I, I, I, D, P, I64, I]
        lib.oracle_evoformer_col.argtypes = [P, P, P, P, P, P, I, I, I, I, D, P, I64, I]
        lib.oracle_decode_rows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I,
                                           ctypes.POINTER(_Params), P, I64, I, I]
        lib.oracle_merge_rows.argtypes = [P, P, P, P, I, I64, I]
        lib.oracle_ipa_rows.argtypes = [P] * 15 + [I] * 7 + [P, I64, I]
        for f in (lib.oracle_attn_rows, lib.oracle_diffattn_rows, lib.oracle_evoformer_row,
                  lib.oracle_evoformer_col, lib.oracle_decode_rows, lib.oracle_merge_rows,
                  lib.oracle_ipa_rows):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _rows(rows, total):
    if rows is None:
        return None, total
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


def attn(q, k, v, *, variant="vanilla", scale=None, bias=None, softcap=50.0,
         alibi_max_bias=8.0, window=256, window_causal=True, prefix=512,
         doc_offsets=None, mask=None, rows=None, block_keys=0, threads=None):
    """Attention forward for q [B,Hq,Sq,D], k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv].

    Returns (o, lse).  With ``rows`` (flat indices (b*Hq+h)*Sq+i) the outputs
    are compact [n_rows, Dv] and [n_rows]; otherwise [B,Hq,Sq,Dv] and [B,Hq,Sq].
    ``mask`` (a mask variant name) composes a mask with the score modification
    of ``variant`` (vanilla, alibi or softcap).  ``block_keys > 0`` selects
    the online twin.
    """
    q, k, v, bias = _f64(q), _f64(k), _f64(v), _f64(bias)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, Dv = v.shape
    assert k.shape == (B, Hkv, Sk, D) and v.shape[:3] == (B, Hkv, Sk)
    if bias is not None:
        assert bias.shape == (Hq, Sq, Sk)
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    msk = 0 if mask is None else (VARIANTS[mask] if isinstance(mask, str) else int(mask))
    docs = None
    if var == DOCUMENT or msk == DOCUMENT:
        docs = np.ascontiguousarray(doc_offsets, dtype=np.int32)
        assert docs.ndim == 2 and docs.shape[0] == B
    p = _Params(var, float(scale if scale is not None else 1.0 / np.sqrt(D)), float(softcap),
                float(alibi_max_bias), int(window), int(bool(window_causal)), int(prefix),
                None if docs is None else docs.ctypes.data,
                0 if docs is None else docs.shape[1] - 1, msk)
    r, n = _rows(rows, B * Hq * Sq)
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(o), _ptr(lse),
                                  B, Hq, Hkv, Sq, Sk, D, Dv, ctypes.byref(p), _ptr(r), n,
                                  int(block_keys), threads or default_threads())
    if rc:
        raise ValueError("oracle_attn_rows rejected its arguments (%d)" % rc)
    if rows is None:
        return o.reshape(B, Hq, Sq, Dv), lse.reshape(B, Hq, Sq)
    return o, lse


def decode(q, k_cache, v_cache, seqlens, *, variant="vanilla", scale=None, softcap=50.0,
           alibi_max_bias=8.0, window=256, window_causal=True, prefix=512, mask=None, rows=None,
           block_keys=0, threads=None):
    """Decode attention against a KV cache: q [B,Hq,Sq,D] are the Sq newest
    tokens of each sequence, k_cache/v_cache [B,Hkv,S_cap,D/Dv] hold
    seqlens[b] tokens, so query i sits at position seqlens[b] - Sq + i.
    Returns (o, lse) shaped like :func:`attn`."""
    q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, Sq, D = q.shape
    _, Hkv, S_cap, Dv = v.shape
    assert k.shape == (B, Hkv, S_cap, D)
    L = np.ascontiguousarray(seqlens, dtype=np.int32)
    assert L.shape == (B,)
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    msk = 0 if mask is None else (VARIANTS[mask] if isinstance(mask, str) else int(mask))
    p = _Params(var, float(scale if scale is not None else 1.0 / np.sqrt(D)), float(softcap),
                float(alibi_max_bias), int(window), int(bool(window_causal)), int(prefix),
                None, 0, msk)
    r, n = _rows(rows, B * Hq * Sq)
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_decode_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(L), _ptr(o), _ptr(lse),
                                    B, Hq, Hkv, Sq, S_cap, D, Dv, ctypes.byref(p), _ptr(r), n,
                                    int(block_keys), threads or default_threads())
    if rc:
        raise ValueError("oracle_decode_rows rejected its arguments (%d)" % rc)
    if rows is None:
        return o.reshape(B, Hq, Sq, Dv), lse.reshape(B, Hq, Sq)
    return o, lse


def merge(o_parts, lse_parts):
    """Merge partial results over disjoint key sets: o_parts [P, ..., Dv],
    lse_parts [P, ...] -> (o [..., Dv], lse [...])."""
    op, lp = _f64(o_parts), _f64(lse_parts)
    assert op.shape[:-1] == lp.shape and op.ndim >= 2
    P, Dv = op.shape[0], op.shape[-1]
    n = int(np.prod(lp.shape[1:], dtype=np.int64))
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    rc = _load().oracle_merge_rows(_ptr(op), _ptr(lp), _ptr(o), _ptr(lse), P, n, Dv)
    if rc:
        raise ValueError("oracle_merge_rows rejected its arguments (%d)" % rc)
    return o.reshape(lp.shape[1:] + (Dv,)), lse.reshape(lp.shape[1:])


def _allowed(kind, Sq, Sk, window, window_causal, prefix, offsets):
    """Boolean [Sq, Sk] matrix of the keys each query may see (the same mask
    definitions as oracle.c, as whole matrices)."""
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    if kind in (VANILLA, ALIBI, SOFTCAP):
        return np.ones((Sq, Sk), bool)
    if kind == CAUSAL:
        return j <= i
    if kind == SLIDING_WINDOW:
        return (j <= i) & (j > i - window) if window_causal else np.abs(i - j) < window
    if kind == PREFIX_LM:
        return (j < prefix) | (j <= i)
    if kind == DOCUMENT:
        off = np.asarray(offsets)
        doc = lambda x: np.searchsorted(off, x, side="right") - 1
        return doc(np.arange(Sq))[:, None] == doc(np.arange(Sk))[None, :]
    raise ValueError(kind)


def attn_bwd(q, k, v, do, *, variant="vanilla", scale=None, softcap=50.0, alibi_max_bias=8.0,
             window=256, window_causal=True, prefix=512, doc_offsets=None, mask=None,
             heads=None):
    """Gradients (dq, dk, dv) of sum(do * O) for O = attn(q, k, v, ...) (no bias).

    The chain rule written out per (batch, query head) on whole float64
    matrices (gist.science explainer, "Technical Summary: Methodology": the
    forward is the plain softmax attention, so its gradient is the plain one):
      S = scale q k^T, s = mod(S) masked, P = softmax_rows(s)
      dV += P^T dO;  dP = dO V^T;  ds = P * (dP - rowsum(P * dP))
      dS = ds * mod'(S);  dQ = scale dS K;  dK += scale dS^T Q
    with mod' = 1 for vanilla and ALiBi (an additive term) and 1 - tanh^2(S /
    cap) for softcap.  Rows with no allowed key get P = 0.  Query heads of a
    group add into their K/V head's dK, dV.  ``heads`` restricts the work to
    a list of (b, h_kv) pairs (their dk, dv are complete; dq is computed for
    the query heads of those groups only, zero elsewhere).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, Dv = v.shape
    G = Hq // Hkv
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    msk = 0 if mask is None else (VARIANTS[mask] if isinstance(mask, str) else int(mask))
    kind = var if var >= CAUSAL else msk
    sc = float(scale if scale is not None else 1.0 / np.sqrt(D))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = heads if heads is not None else [(b, hk) for b in range(B) for hk in range(Hkv)]
    for b, hk in todo:
        allowed = _allowed(kind, Sq, Sk, window, window_causal, prefix,
                           None if doc_offsets is None else doc_offsets[b])
        live = allowed.any(1)
        for h in range(hk * G, (hk + 1) * G):
            S = sc * (q[b, h] @ k[b, hk].T)
            if var == ALIBI:
                slope = 2.0 ** (-alibi_max_bias * (h + 1) / Hq)
                S = S - slope * np.abs(np.arange(Sq)[:, None] - np.arange(Sk)[None, :])
            dmod = 1.0
            if var == SOFTCAP:
                t = np.tanh(S / softcap)
                S = softcap * t
                dmod = 1.0 - t * t
            s = np.where(allowed, S, -np.inf)
            P = np.zeros_like(s)
            m = np.max(s[live], axis=1, keepdims=True)
            e = np.exp(s[live] - m)
            P[live] = e / e.sum(1, keepdims=True)
            dv[b, hk] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, hk].T
            ds = P * (dP - (P * dP).sum(1, keepdims=True))
            dS = ds * dmod
            dq[b, h] = sc * (dS @ k[b, hk])
            dk[b, hk] += sc * (dS.T @ q[b, h])
    return dq, dk, dv


def diffattn(q1, q2, k1, k2, v, *, scale=None, lam=0.8, causal=False, rows=None,
             threads=None):
    """Differential attention; returns (o, lse1, lse2) shaped like :func:`attn`."""
    q1, q2, k1, k2, v = map(_f64, (q1, q2, k1, k2, v))
    B, H, Sq, Dqk = q1.shape
    Sk, Dv = v.shape[2], v.shape[3]
    r, n = _rows(rows, B * H * Sq)
    o = np.empty((n, Dv), np.float64)
    l1 = np.empty((n,), np.float64)
    l2 = np.empty((n,), np.float64)
    rc = _load().oracle_diffattn_rows(_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), _ptr(o),
                                      _ptr(l1), _ptr(l2), B, H, Sq, Sk, Dqk, Dv,
                                      float(scale if scale is not None else 1.0 / np.sqrt(Dqk)),
                                      float(lam), int(bool(causal)), _ptr(r), n,
                                      threads or default_threads())
    if rc:
        raise ValueError("oracle_diffattn_rows rejected its arguments (%d)" % rc)
    if rows is None:
        return o.reshape(B, H, Sq, Dv), l1.reshape(B, H, Sq), l2.reshape(B, H, Sq)
    return o, l1, l2


def evoformer(q, k, v, gate, *, pair_bias=None, key_mask=None, axis="row", scale=None,
              rows=None, threads=None):
    """Evoformer gated self-attention on MSA tensors [N_seq, N_res, H, C].

    axis="row": attention along residues, optional pair_bias [H,N_res,N_res],
    key_mask [N_seq,N_res] (uint8, 1 keep).  axis="col": attention along
    sequences within each residue column (no pair bias); rows then index the
    transposed problem and the full output is returned in [N_seq,N_res,H,C].
    """
    q, k, v, gate, pair_bias = map(_f64, (q, k, v, gate, pair_bias))
    N_seq, N_res, H, C = q.shape
    km = None if key_mask is None else np.ascontiguousarray(key_mask, dtype=np.uint8)
    sc = float(scale if scale is not None else 1.0 / np.sqrt(C))
    lib = _load()
    th = threads or default_threads()
    if axis == "row":
        r, n = _rows(rows, N_seq * N_res * H)
        o = np.empty((n, C), np.float64)
        rc = lib.oracle_evoformer_row(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(pair_bias),
                                      _ptr(km), _ptr(o), N_seq, N_res, H, C, sc, _ptr(r), n, th)
        if rc:
            raise ValueError("oracle_evoformer_row rejected its arguments (%d)" % rc)
        return o.reshape(N_seq, N_res, H, C) if rows is None else o
    if axis == "col":
        assert pair_bias is None
        r, n = _rows(rows, N_seq * N_res * H)
        o = np.empty((n, C), np.float64)
        rc = lib.oracle_evoformer_col(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(km), _ptr(o),
                                      N_seq, N_res, H, C, sc, _ptr(r), n, th)
        if rc:
            raise ValueError("oracle_evoformer_col rejected its arguments (%d)" % rc)
        if rows is None:
            return o.reshape(N_res, N_seq, H, C).transpose(1, 0, 2, 3).copy()
        return o
    raise ValueError("axis must be 'row' or 'col'")


def ipa(q, k, v, q_pts, k_pts, v_pts, rot, trans, gamma, *, pair_bias=None, z=None,
        key_mask=None, rows=None, threads=None):
    """Attention core of Invariant Point Attention (see ``ipa.c``).

    q, k, v [B,L,H,C]; q_pts, k_pts [B,L,H,Pq,3]; v_pts [B,L,H,Pv,3] (local
    frames); rot [B,L,3,3], trans [B,L,3]; gamma [H]; pair_bias [B,H,L,L];
    z [B,L,L,Cz]; key_mask [B,L] uint8.  Returns (o, o_pts, o_pair): with
    ``rows`` (flat (b*L + i)*H + h) compact [n,C], [n,Pv,3], [n,Cz]; else
    [B,L,H,C], [B,L,H,Pv,3], [B,L,H,Cz].  o_pair is None without z.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    q_pts, k_pts, v_pts = _f64(q_pts), _f64(k_pts), _f64(v_pts)
    rot, trans, gamma = _f64(rot), _f64(trans), _f64(gamma)
    pair_bias, z = _f64(pair_bias), _f64(z)
    B, L, H, C = q.shape
    Pq, Pv = q_pts.shape[3], v_pts.shape[3]
    Cz = 0 if z is None else z.shape[3]
    assert k.shape == v.shape == q.shape and k_pts.shape == q_pts.shape
    assert rot.shape == (B, L, 3, 3) and trans.shape == (B, L, 3) and gamma.shape == (H,)
    km = None if key_mask is None else np.ascontiguousarray(key_mask, dtype=np.uint8)
    r, n = _rows(rows, B * L * H)
    o = np.zeros((n, C))
    op = np.zeros((n, Pv, 3))
    oz = None if z is None else np.zeros((n, Cz))
    rc = _load().oracle_ipa_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(q_pts), _ptr(k_pts), _ptr(v_pts),
                                 _ptr(rot), _ptr(trans), _ptr(gamma), _ptr(pair_bias), _ptr(z),
                                 _ptr(km), _ptr(o), _ptr(op), _ptr(oz), B, L, H, C, Pq, Pv, Cz,
                                 _ptr(r), n, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_ipa_rows failed: %d" % rc)
    if rows is None:
        o, op = o.reshape(B, L, H, C), op.reshape(B, L, H, Pv, 3)
        oz = None if oz is None else oz.reshape(B, L, H, Cz)
    return o, op, oz
