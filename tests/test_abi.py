"""The C-ABI library loads, exports every symbol include/flattn.h declares,
and rejects bad arguments on the host before anything is launched.

No GPU is needed: every call here fails validation, which happens before the
library touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

from flashattention_attention_variants_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "flattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        pytest.fail("libflattn.so is not built; run python -m flashattention_attention_variants_amd.build")
    return api.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(api.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.fl_abi_version() == 5
    for s in range(8):
        assert lib.fl_status_str(s)
    assert lib.fl_status_str(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x10000)        # 16-byte aligned, never dereferenced: validation fails first
MISALIGNED = P(0x10008)


def params(variant=0, **kw):
    p = api.AttnParams(variant, 0.125, 50.0, 8.0, 256, 1, 512, 0, None, 0)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def attn(lib, p, q=FAKE, k=FAKE, v=FAKE, bias=None, o=FAKE, lse=None, B=1, Hq=2, Hkv=2, Sq=8,
         Sk=8, D=64, dt=api.FL_BF16):
    return lib.fl_attn_fwd(q, k, v, bias, o, lse, B, Hq, Hkv, Sq, Sk, D, dt,
                           None if p is None else ctypes.byref(p), None)


def test_attn_validation(lib):
    assert attn(lib, None) == api.FL_ERR_NULL
    assert attn(lib, params(), q=None) == api.FL_ERR_NULL
    assert attn(lib, params(), o=None) == api.FL_ERR_NULL
    assert attn(lib, params(), Hq=3, Hkv=2) == api.FL_ERR_SHAPE
    assert attn(lib, params(), B=-1) == api.FL_ERR_SHAPE
    assert attn(lib, params(), D=48) == api.FL_ERR_UNSUPPORTED
    assert attn(lib, params(), D=128) == api.FL_ERR_UNSUPPORTED          # bf16 is D=64 only
    assert attn(lib, params(), dt=7) == api.FL_ERR_UNSUPPORTED
    assert attn(lib, params(), q=MISALIGNED) == api.FL_ERR_ALIGN
    assert attn(lib, params(), lse=P(0x10002)) == api.FL_ERR_ALIGN
    assert attn(lib, params(), bias=FAKE, Sk=12, Sq=12) == api.FL_ERR_ALIGN  # bf16 bias rows
    assert attn(lib, params(variant=9)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=2, softcap=0.0)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=2, softcap=float("inf"))) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=1, alibi_max_bias=-1.0)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=4, window=0)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=5, prefix=-1)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=6, n_docs=0)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=6, n_docs=2)) == api.FL_ERR_NULL     # no offsets
    assert attn(lib, params(scale=float("nan"))) == api.FL_ERR_PARAM
    for var in (3, 4, 5):  # positional masks need S_q == S_k
        assert attn(lib, params(variant=var), Sq=8, Sk=16) == api.FL_ERR_SHAPE
    # a composed mask: only with a score modification, only a mask kind
    assert attn(lib, params(variant=3, mask=4)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=1, mask=2)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=2, mask=7)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=1, mask=3), Sq=8, Sk=16) == api.FL_ERR_SHAPE
    assert attn(lib, params(variant=2, mask=4, window=0)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=0, mask=5, prefix=-1)) == api.FL_ERR_PARAM
    assert attn(lib, params(variant=1, mask=6, n_docs=2)) == api.FL_ERR_NULL
    # nothing to write: success without touching the pointers
    assert attn(lib, params(), q=None, k=None, v=None, o=None, B=0) == api.FL_OK
    assert attn(lib, params(), q=None, k=None, v=None, o=None, Sq=0) == api.FL_OK


def test_diffattn_validation(lib):
    f = lambda **kw: lib.fl_diffattn_fwd(*[kw.get(n, FAKE) for n in ("q1", "q2", "k1", "k2", "v", "o")],
                                         kw.get("lse1"), kw.get("lse2"), kw.get("B", 1), 2,
                                         kw.get("Sq", 8), kw.get("Sk", 8), kw.get("Dqk", 64),
                                         kw.get("Dv", 128), kw.get("dt", api.FL_BF16), 0.125,
                                         kw.get("lam", 0.8), kw.get("causal", 0), None)
    assert f(q2=None) == api.FL_ERR_NULL
    assert f(Dqk=32) == api.FL_ERR_UNSUPPORTED
    assert f(Dv=96) == api.FL_ERR_UNSUPPORTED
    assert f(causal=1, Sk=16) == api.FL_ERR_SHAPE
    assert f(v=MISALIGNED) == api.FL_ERR_ALIGN
    assert f(lam=float("inf")) == api.FL_ERR_PARAM
    assert f(B=0, q1=None, q2=None) == api.FL_OK


def test_evoformer_validation(lib):
    f = lambda **kw: lib.fl_evoformer_gated_attn_fwd(
        *[kw.get(n, FAKE) for n in ("q", "k", "v", "gate")], kw.get("bias"), kw.get("mask"),
        kw.get("o", FAKE), kw.get("N_seq", 4), kw.get("N_res", 16), 2, kw.get("C", 32),
        kw.get("axis", 0), kw.get("dt", api.FL_BF16), 0.17, None)
    assert f(gate=None) == api.FL_ERR_NULL
    assert f(C=16) == api.FL_ERR_UNSUPPORTED
    assert f(axis=1, bias=FAKE) == api.FL_ERR_PARAM   # column attention has no pair bias
    assert f(axis=2) == api.FL_ERR_PARAM
    assert f(bias=FAKE, N_res=12) == api.FL_ERR_ALIGN
    assert f(o=MISALIGNED) == api.FL_ERR_ALIGN
    assert f(N_seq=0, q=None) == api.FL_OK


def decode(lib, p, q=FAKE, kc=FAKE, vc=FAKE, seqlens=FAKE, o=FAKE, lse=None, ws=None, ws_bytes=0,
           B=2, Hq=8, Hkv=2, Sq=1, S_cap=256, max_len=256, D=64, layout=0, dt=api.FL_BF16,
           splits=1):
    return lib.fl_attn_decode_fwd(q, kc, vc, seqlens, o, lse, ws, ws_bytes, B, Hq, Hkv, Sq, S_cap,
                                  max_len, D, layout, dt,
                                  None if p is None else ctypes.byref(p), splits, None)


def test_decode_validation(lib):
    assert decode(lib, None) == api.FL_ERR_NULL
    assert decode(lib, params(), seqlens=None) == api.FL_ERR_NULL
    assert decode(lib, params(), q=None) == api.FL_ERR_NULL
    assert decode(lib, params(), D=128) == api.FL_ERR_UNSUPPORTED
    assert decode(lib, params(), dt=api.FL_F32) == api.FL_ERR_UNSUPPORTED
    assert decode(lib, params(variant=6, n_docs=1)) == api.FL_ERR_UNSUPPORTED
    assert decode(lib, params(variant=1, mask=6, n_docs=1)) == api.FL_ERR_UNSUPPORTED
    assert decode(lib, params(variant=3, mask=4)) == api.FL_ERR_PARAM
    assert decode(lib, params(variant=4, window=0)) == api.FL_ERR_PARAM
    assert decode(lib, params(variant=2, softcap=-1.0)) == api.FL_ERR_PARAM
    assert decode(lib, params(), max_len=300) == api.FL_ERR_PARAM     # beyond the cache
    assert decode(lib, params(), max_len=-1) == api.FL_ERR_SHAPE
    assert decode(lib, params(), Hq=6, Hkv=4) == api.FL_ERR_SHAPE
    assert decode(lib, params(), layout=2) == api.FL_ERR_PARAM
    assert decode(lib, params(), splits=-1) == api.FL_ERR_PARAM
    assert decode(lib, params(), o=MISALIGNED) == api.FL_ERR_ALIGN
    assert decode(lib, params(), seqlens=P(0x10002)) == api.FL_ERR_ALIGN
    # four key ranges need a workspace of the size the library reports
    need = lib.fl_attn_decode_workspace_size(2, 8, 2, 1, 256, 64, None, 4)
    assert need == 4 * 16 * 64 * 4 + 4 * 16 * 4
    assert decode(lib, params(), splits=4) == api.FL_ERR_NULL
    assert decode(lib, params(), splits=4, ws=FAKE, ws_bytes=need - 1) == api.FL_ERR_PARAM
    assert decode(lib, params(), splits=4, ws=MISALIGNED, ws_bytes=need) == api.FL_ERR_ALIGN
    assert decode(lib, params(), B=0, q=None, o=None) == api.FL_OK


def test_decode_split_choice(lib):
    ns = lambda *a, p=None: lib.fl_attn_decode_num_splits(*a[:5], p and ctypes.byref(p), a[5])
    ws = lambda *a, p=None: lib.fl_attn_decode_workspace_size(*a[:6], p and ctypes.byref(p), a[6])
    assert ns(2, 8, 2, 1, 256, 1) == 1 and ws(2, 8, 2, 1, 256, 64, 1) == 0
    assert ns(2, 8, 2, 1, 256, 100) == 4          # capped at the 4 tiles of 64 keys
    assert ns(1, 8, 8, 1, 300, 2) == 2
    # chosen: enough work-groups, but ranges of at least 16 tiles
    assert ns(64, 32, 8, 1, 8192, 0) == 8         # 512 (sequence, head) pairs x 8
    assert ns(1, 32, 8, 1, 8192, 0) == 8          # 128 tiles / 16
    assert ns(1, 32, 8, 1, 1024, 0) == 1
    # a sliding window bounds the keys a row needs, whatever the cache length
    win = params(variant=4, window=1024)
    assert ns(1, 32, 8, 1, 65536, 0, p=win) == 1
    assert ns(1, 32, 8, 1, 65536, 0, p=params(variant=4, window=4096)) == 4
    assert ns(1, 32, 8, 1, 65536, 0, p=params(variant=1, mask=4, window=2048, window_causal=0)) == 4
    assert ns(1, 32, 8, 1, 65536, 0, p=params(variant=3)) == 64
    assert ns(4, 32, 8, 1, 0, 0) == 1 and ws(4, 32, 8, 1, 0, 64, 0) == 0
    assert ns(2, 8, 3, 1, 256, 0) == -1 and ws(-1, 8, 2, 1, 256, 64, 0) == -1
    # 16-byte rounding of the LSE block
    assert ws(1, 1, 1, 3, 256, 64, 2) == 2 * 3 * 64 * 4 + 32


def test_merge_validation(lib):
    f = lambda **kw: lib.fl_attn_merge(kw.get("op", FAKE), kw.get("lp", FAKE), kw.get("o", FAKE),
                                       kw.get("lse"), kw.get("n", 2), kw.get("rows", 10),
                                       kw.get("D", 64), kw.get("dt", api.FL_BF16), None)
    assert f(n=0) == api.FL_ERR_SHAPE
    assert f(D=0) == api.FL_ERR_SHAPE
    assert f(dt=5) == api.FL_ERR_UNSUPPORTED
    assert f(op=None) == api.FL_ERR_NULL
    assert f(lse=P(0x10002)) == api.FL_ERR_ALIGN
    assert f(rows=0, op=None, lp=None, o=None) == api.FL_OK


def test_bwd_validation(lib):
    f = lambda p=None, **kw: lib.fl_attn_bwd(
        *[kw.get(n, FAKE) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws")],
        kw.get("B", 1), kw.get("Hq", 2), kw.get("Hkv", 2), kw.get("Sq", 8), kw.get("Sk", 8),
        kw.get("D", 64), kw.get("dt", api.FL_BF16), None if p is None else ctypes.byref(p), None)
    assert f() == api.FL_ERR_NULL
    assert f(params(), ws=None) == api.FL_ERR_NULL
    assert f(params(), do=None) == api.FL_ERR_NULL
    assert f(params(), D=128) == api.FL_ERR_UNSUPPORTED
    assert f(params(), dt=api.FL_F32) == api.FL_ERR_UNSUPPORTED
    assert f(params(), Hq=3) == api.FL_ERR_SHAPE
    assert f(params(variant=3), Sk=16) == api.FL_ERR_SHAPE
    assert f(params(variant=2, softcap=0.0)) == api.FL_ERR_PARAM
    assert f(params(variant=1, mask=2)) == api.FL_ERR_PARAM
    assert f(params(), dk=MISALIGNED) == api.FL_ERR_ALIGN
    assert f(params(), B=0, q=None, k=None, v=None) == api.FL_OK


def test_span_limits(lib):
    # Byte offsets within one (batch, head) block must stay below 2^31 for
    # every row up to 63 past the last (a partial key tile addresses them):
    # ((rows + 63) * row_elems + width) * 2 < 2^31.  Rejected on the host.
    sk = 16777152  # D = 64: (S_k + 63) * 64 + 64 reaches 2^30
    assert ((sk + 63) * 64 + 64) * 2 >= 1 << 31 and ((sk + 62) * 64 + 64) * 2 < 1 << 31
    assert attn(lib, params(), Sq=8, Sk=sk) == api.FL_ERR_SHAPE
    # DiffAttn with D_v = 128: the V rows set the limit
    sv = 8388544
    assert ((sv + 63) * 128 + 128) * 2 >= 1 << 31 and ((sv + 62) * 128 + 128) * 2 < 1 << 31
    d = lib.fl_diffattn_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1, 2, 8, sv, 64, 128,
                            api.FL_BF16, 0.125, 0.8, 0, None)
    assert d == api.FL_ERR_SHAPE
    # Evoformer column form: a row of the transposed problem is N_res*H*C apart
    n_res, H, C = 16, 2, 32
    ns = ((1 << 30) - C) // (n_res * H * C) - 63 + 1
    assert ((ns + 63) * n_res * H * C + C) * 2 >= 1 << 31
    e = lib.fl_evoformer_gated_attn_fwd(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ns, n_res, H, C,
                                        1, api.FL_BF16, 0.17, None)
    assert e == api.FL_ERR_SHAPE
    # decode: the cache capacity sets the block
    assert decode(lib, params(), S_cap=sk, max_len=256) == api.FL_ERR_SHAPE
    # backward: either length
    b = lambda Sq, Sk: lib.fl_attn_bwd(*([FAKE] * 10), 1, 2, 2, Sq, Sk, 64, api.FL_BF16,
                                       ctypes.byref(params()), None)
    assert b(8, sk) == api.FL_ERR_SHAPE and b(sk, 8) == api.FL_ERR_SHAPE


def test_ipa_validation(lib):
    names = ("q", "k", "v", "q_pts", "k_pts", "v_pts", "rot", "trans", "gamma")

    def f(**kw):
        return lib.fl_ipa_attn_fwd(*[kw.get(n, FAKE) for n in names], kw.get("bias"), kw.get("z"),
                                   kw.get("mask"), kw.get("o", FAKE), kw.get("o_pts", FAKE),
                                   kw.get("o_pair"), kw.get("B", 1), kw.get("L", 16), kw.get("H", 12),
                                   kw.get("C", 16), kw.get("Pq", 4), kw.get("Pv", 8),
                                   kw.get("Cz", 0), kw.get("dt", api.FL_BF16), None)
    assert f(gamma=None) == api.FL_ERR_NULL
    assert f(o_pts=None) == api.FL_ERR_NULL
    assert f(z=FAKE, Cz=128) == api.FL_ERR_NULL             # z without o_pair
    assert f(o_pair=FAKE, Cz=128) == api.FL_ERR_NULL        # o_pair without z
    assert f(L=-1) == api.FL_ERR_SHAPE
    assert f(H=0) == api.FL_ERR_SHAPE
    assert f(C=32) == api.FL_ERR_UNSUPPORTED
    assert f(Pq=3) == api.FL_ERR_UNSUPPORTED
    assert f(z=FAKE, o_pair=FAKE, Cz=96) == api.FL_ERR_UNSUPPORTED
    assert f(dt=api.FL_F32) == api.FL_ERR_UNSUPPORTED
    assert f(k_pts=MISALIGNED) == api.FL_ERR_ALIGN
    assert f(rot=P(0x10002)) == api.FL_ERR_ALIGN
    assert f(z=FAKE, o_pair=MISALIGNED, Cz=128) == api.FL_ERR_ALIGN
    # one residue's pair rows stay below 2^31 bytes
    assert f(z=FAKE, o_pair=FAKE, Cz=128, L=1 << 23) == api.FL_ERR_SHAPE
    assert f(B=0, q=None, o=None) == api.FL_OK


def test_decode_noalloc_validation(lib):
    """The no-allocation decode validates like fl_attn_decode_fwd and rejects,
    before touching the runtime, a call whose partial results would not fit
    the static buffer."""
    def f(p, **kw):
        return lib.fl_attn_decode_fwd_noalloc(
            kw.get("q", FAKE), FAKE, FAKE, kw.get("seqlens", FAKE), kw.get("o", FAKE), None,
            kw.get("B", 2), kw.get("Hq", 8), 2, 1, kw.get("S_cap", 256), kw.get("max_len", 256), 64,
            0, api.FL_BF16, None if p is None else ctypes.byref(p), kw.get("splits", 1), None)
    assert f(None) == api.FL_ERR_NULL
    assert f(params(), seqlens=None) == api.FL_ERR_NULL
    assert f(params(), o=MISALIGNED) == api.FL_ERR_ALIGN
    assert f(params(variant=4, window=0)) == api.FL_ERR_PARAM
    # 256 key ranges of 2048 rows x 65 floats: 136 MB, past the 32 MiB buffer
    big = dict(B=64, Hq=32, S_cap=65536, max_len=65536, splits=256)
    need = lib.fl_attn_decode_workspace_size(64, 32, 2, 1, 65536, 64, None, 256)
    assert need > (32 << 20)
    assert f(params(), **big) == api.FL_ERR_SCRATCH
    assert lib.fl_status_str(api.FL_ERR_SCRATCH)
    assert f(params(), B=0, q=None, o=None) == api.FL_OK
