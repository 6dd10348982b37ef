"""ctypes binding of ``libflattn.so`` (entry points declared in include/flattn.h).

Argument marshalling only: each function checks that the torch tensors are
contiguous, on the GPU and of the right dtype, allocates the outputs it was
not given, and passes raw device pointers plus torch's current HIP stream to
the C entry point of the same name.  Every step of the computation runs in
the library's kernels; there is no fallback.  A missing library or a
non-zero status raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflattn.so")

(FL_OK, FL_ERR_NULL, FL_ERR_SHAPE, FL_ERR_ALIGN, FL_ERR_UNSUPPORTED, FL_ERR_PARAM, FL_ERR_LAUNCH,
 FL_ERR_SCRATCH) = range(8)
FL_BF16, FL_F32 = 0, 1
VARIANTS = {"vanilla": 0, "alibi": 1, "softcap": 2, "causal": 3, "sliding_window": 4,
            "prefix_lm": 5, "document": 6}
EVO_AXES = {"row": 0, "col": 1}
KV_LAYOUTS = {"bhsd": 0, "bshd": 1}
SYMBOLS = ("fl_attn_fwd", "fl_diffattn_fwd", "fl_evoformer_gated_attn_fwd", "fl_attn_decode_fwd",
           "fl_attn_decode_workspace_size", "fl_attn_decode_num_splits", "fl_attn_merge",
           "fl_attn_decode_fwd_noalloc", "fl_attn_bwd", "fl_ipa_attn_fwd", "fl_status_str",
           "fl_abi_version")


class FlError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


class AttnParams(ctypes.Structure):
    """Mirror of ``fl_attn_params``."""

    _fields_ = [
        ("variant", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("alibi_max_bias", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("window_causal", ctypes.c_int32),
        ("prefix", ctypes.c_int32),
        ("n_docs", ctypes.c_int32),
        ("doc_offsets", ctypes.c_void_p),
        ("mask", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str | None = None):
    """Load the shared library (once); raises if it has not been built.

    FLATTN_LIB, when set, names another build of the same library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("FLATTN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libflattn.so is not built (%s); run "
                           "`python -m flashattention_attention_variants_amd.build`" % p)
    lib = ctypes.CDLL(p)
    V, I, F, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_size_t
    lib.fl_attn_fwd.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, I, ctypes.POINTER(AttnParams), V]
    lib.fl_diffattn_fwd.argtypes = [V, V, V, V, V, V, V, V, I, I, I, I, I, I, I, F, F, I, V]
    lib.fl_evoformer_gated_attn_fwd.argtypes = [V, V, V, V, V, V, V, I, I, I, I, I, I, F, V]
    lib.fl_attn_decode_fwd.argtypes = [V, V, V, V, V, V, V, SZ, I, I, I, I, I, I, I, I, I,
                                       ctypes.POINTER(AttnParams), I, V]
    lib.fl_attn_decode_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(AttnParams), I]
    lib.fl_attn_decode_workspace_size.restype = I64
    lib.fl_attn_decode_num_splits.argtypes = [I, I, I, I, I, ctypes.POINTER(AttnParams), I]
    lib.fl_attn_decode_num_splits.restype = I
    lib.fl_attn_merge.argtypes = [V, V, V, V, I, I64, I, I, V]
    lib.fl_attn_bwd.argtypes = [V, V, V, V, V, V, V, V, V, V, I, I, I, I, I, I, I,
                                ctypes.POINTER(AttnParams), V]
    lib.fl_ipa_attn_fwd.argtypes = [V] * 15 + [I] * 8 + [V]
    lib.fl_attn_decode_fwd_noalloc.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, I, I, I,
                                               ctypes.POINTER(AttnParams), I, V]
    for f in (lib.fl_attn_fwd, lib.fl_diffattn_fwd, lib.fl_evoformer_gated_attn_fwd,
              lib.fl_attn_decode_fwd, lib.fl_attn_merge, lib.fl_attn_bwd, lib.fl_ipa_attn_fwd,
              lib.fl_attn_decode_fwd_noalloc):
        f.restype = ctypes.c_int
    lib.fl_status_str.argtypes = [I]
    lib.fl_status_str.restype = ctypes.c_char_p
    lib.fl_abi_version.argtypes = []
    lib.fl_abi_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(fn, status):
    if status != FL_OK:
        raise FlError(fn, status, load_library().fl_status_str(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FL_BF16
    if t.dtype == torch.float32:
        return FL_F32
    raise TypeError("dtype must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fl_attn_fwd(q, k, v, *, variant="vanilla", scale=None, bias=None, softcap=50.0,
                alibi_max_bias=8.0, window=256, window_causal=True, prefix=512,
                doc_offsets=None, mask=None, out=None, lse=None, return_lse=False, stream=None):
    """softmax(score_mod(scale q k^T) + bias) v for q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D].

    ``mask`` (a mask variant name) composes a mask with the score
    modification of ``variant`` (vanilla, alibi or softcap).  Returns ``o``
    or ``(o, lse)``; ``lse`` [B,Hq,Sq] float32 is computed when given or when
    ``return_lse``.
    """
    q = _dev(q, "q")
    dt = q.dtype
    k, v = _dev(k, "k", dt), _dev(v, "v", dt)
    bias = _dev(bias, "bias", dt)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    if out is None:
        out = torch.empty(B, Hq, Sq, v.shape[3], dtype=dt, device=q.device)
    _dev(out, "out", dt)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
    _dev(lse, "lse", torch.float32)
    docs = None
    if VARIANTS["document"] in (VARIANTS.get(variant, variant), VARIANTS.get(mask, mask)):
        docs = _dev(doc_offsets, "doc_offsets", torch.int32)
    p = _params(variant, mask, scale, D, softcap, alibi_max_bias, window, window_causal, prefix,
                docs)
    st = load_library().fl_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(out), _ptr(lse),
                                    B, Hq, Hkv, Sq, Sk, D, _dtype_code(q), ctypes.byref(p),
                                    _stream(stream))
    _check("fl_attn_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def _params(variant, mask, scale, D, softcap, alibi_max_bias, window, window_causal, prefix,
            docs=None):
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    msk = 0 if mask is None else (VARIANTS[mask] if isinstance(mask, str) else int(mask))
    return AttnParams(var, float(scale if scale is not None else 1.0 / math.sqrt(D)), float(softcap),
                      float(alibi_max_bias), int(window), int(bool(window_causal)), int(prefix),
                      0 if docs is None else docs.shape[-1] - 1,
                      None if docs is None else docs.data_ptr(), msk)


def _window_params(variant, mask, window, window_causal):
    return _params(variant, mask, None, 64, 50.0, 8.0, window, window_causal, 0)


def fl_attn_decode_workspace_size(B, Hq, Hkv, Sq, max_seqlen, D=64, num_splits=0, *,
                                  variant="vanilla", mask=None, window=256, window_causal=True):
    """Bytes of device workspace :func:`fl_attn_decode_fwd` needs (0: none)."""
    p = _window_params(variant, mask, window, window_causal)
    n = load_library().fl_attn_decode_workspace_size(B, Hq, Hkv, Sq, max_seqlen, D,
                                                     ctypes.byref(p), num_splits)
    if n < 0:
        raise ValueError("invalid decode sizes")
    return int(n)


def fl_attn_decode_num_splits(B, Hq, Hkv, Sq, max_seqlen, num_splits=0, *, variant="vanilla",
                              mask=None, window=256, window_causal=True):
    """Key ranges per (sequence, K/V head) the decode call uses."""
    p = _window_params(variant, mask, window, window_causal)
    n = load_library().fl_attn_decode_num_splits(B, Hq, Hkv, Sq, max_seqlen, ctypes.byref(p),
                                                 num_splits)
    if n < 0:
        raise ValueError("invalid decode sizes")
    return int(n)


def fl_attn_decode_fwd(q, k_cache, v_cache, cache_seqlens, *, max_seqlen=None, layout="bhsd",
                       variant="vanilla", mask=None, scale=None, softcap=50.0, alibi_max_bias=8.0,
                       window=256, window_causal=True, prefix=512, num_splits=0, workspace=None,
                       out=None, lse=None, return_lse=False, stream=None):
    """Decode attention of q [B,Hq,Sq,D] (the Sq newest tokens) against a KV
    cache ([B,Hkv,S_cap,D] for layout "bhsd", [B,S_cap,Hkv,D] for "bshd")
    holding cache_seqlens[b] (int32, on the GPU) tokens per sequence.

    ``max_seqlen`` bounds the lengths (default: the cache capacity).  A
    workspace of :func:`fl_attn_decode_workspace_size` bytes (a uint8 GPU
    tensor) is allocated here when not given.
    """
    q = _dev(q, "q")
    dt = q.dtype
    k_cache, v_cache = _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt)
    seqlens = _dev(cache_seqlens, "cache_seqlens", torch.int32)
    B, Hq, Sq, D = q.shape
    lay = KV_LAYOUTS[layout]
    if lay == 0:
        _, Hkv, S_cap, _ = k_cache.shape
    else:
        _, S_cap, Hkv, _ = k_cache.shape
    if max_seqlen is None:
        max_seqlen = S_cap
    if out is None:
        out = torch.empty(B, Hq, Sq, D, dtype=dt, device=q.device)
    _dev(out, "out", dt)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=q.device)
    _dev(lse, "lse", torch.float32)
    p = _params(variant, mask, scale, D, softcap, alibi_max_bias, window, window_causal, prefix)
    need = load_library().fl_attn_decode_workspace_size(B, Hq, Hkv, Sq, int(max_seqlen), D,
                                                        ctypes.byref(p), int(num_splits))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    st = load_library().fl_attn_decode_fwd(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out), _ptr(lse), _ptr(workspace),
        0 if workspace is None else workspace.numel(), B, Hq, Hkv, Sq, S_cap, int(max_seqlen), D,
        lay, _dtype_code(q), ctypes.byref(p), int(num_splits), _stream(stream))
    _check("fl_attn_decode_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def fl_attn_decode_fwd_noalloc(q, k_cache, v_cache, cache_seqlens, *, out, lse=None,
                               max_seqlen=None, layout="bhsd", variant="vanilla", mask=None,
                               scale=None, softcap=50.0, alibi_max_bias=8.0, window=256,
                               window_causal=True, prefix=512, num_splits=0, stream=None):
    """:func:`fl_attn_decode_fwd` with the library's static scratch buffer in
    place of a workspace; ``out`` (and ``lse``, if wanted) are the caller's
    tensors, so nothing is allocated here either.  Returns ``out`` or
    ``(out, lse)``."""
    q = _dev(q, "q")
    dt = q.dtype
    k_cache, v_cache = _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt)
    seqlens = _dev(cache_seqlens, "cache_seqlens", torch.int32)
    B, Hq, Sq, D = q.shape
    lay = KV_LAYOUTS[layout]
    if lay == 0:
        _, Hkv, S_cap, _ = k_cache.shape
    else:
        _, S_cap, Hkv, _ = k_cache.shape
    if max_seqlen is None:
        max_seqlen = S_cap
    _dev(out, "out", dt)
    _dev(lse, "lse", torch.float32)
    p = _params(variant, mask, scale, D, softcap, alibi_max_bias, window, window_causal, prefix)
    st = load_library().fl_attn_decode_fwd_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq,
        S_cap, int(max_seqlen), D, lay, _dtype_code(q), ctypes.byref(p), int(num_splits),
        _stream(stream))
    _check("fl_attn_decode_fwd_noalloc", st)
    return (out, lse) if lse is not None else out


def fl_attn_merge(o_parts, lse_parts, *, out_dtype=torch.bfloat16, out=None, lse=None,
                  return_lse=False, stream=None):
    """Merge partial results o_parts [P, ..., D] (float32, each normalised over
    its keys) with lse_parts [P, ...] (float32, natural log) into o [..., D]."""
    o_parts = _dev(o_parts, "o_parts", torch.float32)
    lse_parts = _dev(lse_parts, "lse_parts", torch.float32)
    if tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape) or o_parts.dim() < 2:
        raise ValueError("o_parts must be lse_parts' shape plus a head dimension")
    P, D = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if out is None:
        out = torch.empty(tuple(o_parts.shape[1:]), dtype=out_dtype, device=o_parts.device)
    _dev(out, "out", out_dtype)
    if lse is None and return_lse:
        lse = torch.empty(tuple(lse_parts.shape[1:]), dtype=torch.float32, device=o_parts.device)
    _dev(lse, "lse", torch.float32)
    st = load_library().fl_attn_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse), P, rows,
                                      D, _dtype_code(out), _stream(stream))
    _check("fl_attn_merge", st)
    return (out, lse) if (return_lse or lse is not None) else out


def fl_attn_bwd(q, k, v, o, lse, d_o, *, variant="vanilla", scale=None, softcap=50.0,
                alibi_max_bias=8.0, window=256, window_causal=True, prefix=512, doc_offsets=None,
                mask=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the forward call with the same arguments,
    given its output ``o``, its ``lse`` and the output gradient ``d_o``."""
    q = _dev(q, "q")
    dt = q.dtype
    k, v, o, d_o = (_dev(t, n, dt) for t, n in ((k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")))
    lse = _dev(lse, "lse", torch.float32)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    dq = torch.empty_like(q) if dq is None else _dev(dq, "dq", dt)
    dk = torch.empty_like(k) if dk is None else _dev(dk, "dk", dt)
    dv = torch.empty_like(v) if dv is None else _dev(dv, "dv", dt)
    if workspace is None:
        workspace = torch.empty(max(2 * B * Hq * Sq, 1), dtype=torch.float32, device=q.device)
    _dev(workspace, "workspace", torch.float32)
    if workspace.numel() < 2 * B * Hq * Sq:
        raise ValueError("fl_attn_bwd: workspace needs %d float32 values, got %d"
                         % (2 * B * Hq * Sq, workspace.numel()))
    docs = None
    if VARIANTS["document"] in (VARIANTS.get(variant, variant), VARIANTS.get(mask, mask)):
        docs = _dev(doc_offsets, "doc_offsets", torch.int32)
    p = _params(variant, mask, scale, D, softcap, alibi_max_bias, window, window_causal, prefix,
                docs)
    st = load_library().fl_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), B, Hq, Hkv, Sq,
                                    Sk, D, _dtype_code(q), ctypes.byref(p), _stream(stream))
    _check("fl_attn_bwd", st)
    return dq, dk, dv


def fl_diffattn_fwd(q1, q2, k1, k2, v, *, lam=0.8, scale=None, causal=False, out=None,
                    return_lse=False, stream=None):
    """softmax(scale q1 k1^T) v - lam * softmax(scale q2 k2^T) v (MHA)."""
    q1 = _dev(q1, "q1")
    dt = q1.dtype
    q2, k1, k2, v = (_dev(t, n, dt) for t, n in ((q2, "q2"), (k1, "k1"), (k2, "k2"), (v, "v")))
    B, H, Sq, Dqk = q1.shape
    Sk, Dv = v.shape[2], v.shape[3]
    if out is None:
        out = torch.empty(B, H, Sq, Dv, dtype=dt, device=q1.device)
    _dev(out, "out", dt)
    l1 = l2 = None
    if return_lse:
        l1 = torch.empty(B, H, Sq, dtype=torch.float32, device=q1.device)
        l2 = torch.empty_like(l1)
    st = load_library().fl_diffattn_fwd(_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), _ptr(out),
                                        _ptr(l1), _ptr(l2), B, H, Sq, Sk, Dqk, Dv, _dtype_code(q1),
                                        float(scale if scale is not None else 1.0 / math.sqrt(Dqk)),
                                        float(lam), int(bool(causal)), _stream(stream))
    _check("fl_diffattn_fwd", st)
    return (out, l1, l2) if return_lse else out


def fl_evoformer_gated_attn_fwd(q, k, v, gate, *, pair_bias=None, key_mask=None, axis="row",
                                scale=None, out=None, stream=None):
    """Evoformer gated self-attention on [N_seq, N_res, H, C] MSA tensors."""
    q = _dev(q, "q")
    dt = q.dtype
    k, v, gate = _dev(k, "k", dt), _dev(v, "v", dt), _dev(gate, "gate", dt)
    pair_bias = _dev(pair_bias, "pair_bias", dt)
    key_mask = _dev(key_mask, "key_mask", torch.uint8)
    N_seq, N_res, H, C = q.shape
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dt)
    st = load_library().fl_evoformer_gated_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(pair_bias), _ptr(key_mask), _ptr(out),
        N_seq, N_res, H, C, EVO_AXES[axis], _dtype_code(q),
        float(scale if scale is not None else 1.0 / math.sqrt(C)), _stream(stream))
    _check("fl_evoformer_gated_attn_fwd", st)
    return out


def fl_ipa_attn_fwd(q, k, v, q_pts, k_pts, v_pts, rot, trans, gamma, *, pair_bias=None, z=None,
                    key_mask=None, out=None, stream=None):
    """Attention core of Invariant Point Attention.

    q, k, v [B,L,H,C] bf16; q_pts, k_pts [B,L,H,Pq,3], v_pts [B,L,H,Pv,3],
    rot [B,L,3,3], trans [B,L,3], gamma [H] float32; pair_bias [B,H,L,L] and
    z [B,L,L,Cz] bf16; key_mask [B,L] uint8.  Returns (o, o_pts, o_pair);
    o_pair is None without z.  ``out`` may pass the three output tensors.
    """
    q = _dev(q, "q")
    dt = q.dtype
    k, v = _dev(k, "k", dt), _dev(v, "v", dt)
    f32 = torch.float32
    q_pts, k_pts, v_pts = _dev(q_pts, "q_pts", f32), _dev(k_pts, "k_pts", f32), _dev(v_pts, "v_pts", f32)
    rot, trans, gamma = _dev(rot, "rot", f32), _dev(trans, "trans", f32), _dev(gamma, "gamma", f32)
    pair_bias, z = _dev(pair_bias, "pair_bias", dt), _dev(z, "z", dt)
    key_mask = _dev(key_mask, "key_mask", torch.uint8)
    B, L, H, C = q.shape
    Pq, Pv = q_pts.shape[3], v_pts.shape[3]
    Cz = 0 if z is None else z.shape[3]
    if out is None:
        out = (torch.empty_like(q), torch.empty(B, L, H, Pv, 3, dtype=f32, device=q.device),
               None if z is None else torch.empty(B, L, H, Cz, dtype=dt, device=q.device))
    o, o_pts, o_pair = out
    _dev(o, "o", dt)
    _dev(o_pts, "o_pts", f32)
    _dev(o_pair, "o_pair", dt)
    st = load_library().fl_ipa_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_pts), _ptr(k_pts), _ptr(v_pts), _ptr(rot), _ptr(trans),
        _ptr(gamma), _ptr(pair_bias), _ptr(z), _ptr(key_mask), _ptr(o), _ptr(o_pts), _ptr(o_pair),
        B, L, H, C, Pq, Pv, Cz, _dtype_code(q), _stream(stream))
    _check("fl_ipa_attn_fwd", st)
    return o, o_pts, o_pair
