"""fl_attn_decode_fwd_noalloc (the decode entry point for callers that cannot
allocate) against fl_attn_decode_fwd on the same inputs, through the C ABI:
the same kernels and the same split choice, so the outputs must agree bit
for bit; both are also held to the bf16 bar against the oracle.  Two calls
in a row share the GPU's static buffer, the second with a smaller problem
whose partial results cover less of it."""
import numpy as np
import pytest
import torch

import oracle
from flashattention_attention_variants_amd import api, inputs
from tests._gpu_common import check, errors, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    oracle.build()
    api.load_library()


CASES = [  # B, Hq, Hkv, Sq, S_cap, splits, variant: the second smaller than the first
    (16, 32, 8, 1, 4096, 0, dict(variant="causal")),
    (3, 8, 2, 2, 900, 3, dict(variant="alibi", alibi_max_bias=8.0)),
]


def test_noalloc_matches_workspace_entry_point():
    for n, (B, Hq, Hkv, Sq, S_cap, splits, kw) in enumerate(CASES):
        q, kc, vc = inputs.decode_inputs(B, Hq, Hkv, Sq, S_cap, 64, seed=1500 + n)
        seqlens = inputs.cache_lengths(B, max(Sq, S_cap // 8), S_cap, seed=1510 + n)
        g = [t.to(DEV) for t in (q, kc, vc, seqlens)]
        assert api.fl_attn_decode_num_splits(B, Hq, Hkv, Sq, S_cap, splits, variant=kw["variant"]) > 1
        o_ref, l_ref = api.fl_attn_decode_fwd(*g, num_splits=splits, return_lse=True, **kw)
        o_na = torch.full_like(o_ref, float("nan"))
        l_na = torch.full_like(l_ref, float("nan"))
        api.fl_attn_decode_fwd_noalloc(*g, out=o_na, lse=l_na, num_splits=splits, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_na) and torch.equal(l_ref, l_na), "case %d" % n
        ro, rl = oracle.decode(np64(q), np64(kc), np64(vc), seqlens.numpy(), **kw)
        check(np64(o_na), ro, "bf16", "noalloc case %d" % n)
        mx, _, _ = errors(np64(l_na), rl)
        assert mx <= 2e-2, mx


def test_noalloc_rejects_oversized_call():
    B, Hq, Hkv, S_cap = 64, 32, 2, 65536
    q = torch.zeros(B, Hq, 1, 64, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, Hkv, 64, 64, dtype=torch.bfloat16, device=DEV)  # never read
    seqlens = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    with pytest.raises(api.FlError) as e:
        # a cache that large is not allocated: the size check comes first
        api.load_library()
        st = api.load_library().fl_attn_decode_fwd_noalloc(
            api._ptr(q), api._ptr(kc), api._ptr(kc), api._ptr(seqlens), api._ptr(o), None, B, Hq,
            Hkv, 1, S_cap, S_cap, 64, 0, api.FL_BF16, __import__("ctypes").byref(
                api._params("vanilla", None, None, 64, 50.0, 8.0, 256, True, 512)), 256, None)
        api._check("fl_attn_decode_fwd_noalloc", st)
    assert e.value.status == api.FL_ERR_SCRATCH
