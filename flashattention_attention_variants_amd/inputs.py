"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module holds no attention arithmetic: it only draws tensors.  Every
tensor is drawn on the CPU with ``torch.Generator().manual_seed(seed)`` as
float32 ``randn`` in a fixed order and then rounded to the compute dtype
(bfloat16 rounding is round-to-nearest-even), so the GPU and the oracle see
the same bytes.

Shapes follow the workloads the pages evaluate: sequence lengths 512-16k with
head dimension 64 (papers.lqhl.me wiki, "设计取舍", evaluation conditions) and
AlphaFold2-style Evoformer blocks at 256 residues (same page, "实验与结果").
The pages' own workloads (a LLaMa serving trace, OpenFold inputs) are not
available; these iid N(0,1) tensors stand in for their shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn(g: torch.Generator, shape, dtype: str) -> torch.Tensor:
    """float32 N(0,1) draw rounded to ``dtype`` ("bf16" or "f32")."""
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(DTYPES[dtype]).contiguous()


def doc_offsets(B: int, S: int, n_docs: int, seed: int) -> torch.Tensor:
    """Document boundaries [B, n_docs+1] int32: 0 = o_0 < o_1 < ... < o_n = S.

    Per batch element, n_docs-1 distinct cut points are drawn uniformly without
    replacement from {1, ..., S-1} and sorted: a uniform random composition of
    S into n_docs positive lengths.
    """
    if not 1 <= n_docs <= S:
        raise ValueError("need 1 <= n_docs <= S")
    g = _gen(seed)
    rows = []
    for _ in range(B):
        cuts = torch.randperm(S - 1, generator=g)[: n_docs - 1] + 1
        cuts, _ = torch.sort(cuts)
        rows.append(torch.cat([torch.tensor([0]), cuts, torch.tensor([S])]))
    return torch.stack(rows).to(torch.int32).contiguous()


def attn_inputs(B, Hq, Hkv, S_q, S_k, D, dtype="bf16", seed=0, Dv=None):
    """q [B,Hq,S_q,D], k [B,Hkv,S_k,D], v [B,Hkv,S_k,Dv], drawn in that order."""
    g = _gen(seed)
    q = randn(g, (B, Hq, S_q, D), dtype)
    k = randn(g, (B, Hkv, S_k, D), dtype)
    v = randn(g, (B, Hkv, S_k, Dv or D), dtype)
    return q, k, v


def bias_inputs(Hq, S_q, S_k, dtype="bf16", seed=0):
    """Additive score bias [Hq, S_q, S_k], N(0,1)."""
    return randn(_gen(seed), (Hq, S_q, S_k), dtype)


def diffattn_inputs(B, H, S, Dqk, Dv, dtype="bf16", seed=0):
    """q1, q2, k1, k2 [B,H,S,Dqk] and v [B,H,S,Dv], drawn in that order."""
    g = _gen(seed)
    q1 = randn(g, (B, H, S, Dqk), dtype)
    q2 = randn(g, (B, H, S, Dqk), dtype)
    k1 = randn(g, (B, H, S, Dqk), dtype)
    k2 = randn(g, (B, H, S, Dqk), dtype)
    v = randn(g, (B, H, S, Dv), dtype)
    return q1, q2, k1, k2, v


def evoformer_inputs(N_seq, N_res, H, C, dtype="bf16", seed=0, masked_frac=0.05):
    """MSA-shaped q, k, v, gate [N_seq,N_res,H,C]; pair bias [H,N_res,N_res];
    key mask [N_seq,N_res] uint8 (1 keep, 0 excluded) with each position
    excluded independently with probability ``masked_frac``.  Drawn in the
    order q, k, v, gate, bias, mask."""
    g = _gen(seed)
    q = randn(g, (N_seq, N_res, H, C), dtype)
    k = randn(g, (N_seq, N_res, H, C), dtype)
    v = randn(g, (N_seq, N_res, H, C), dtype)
    gate = randn(g, (N_seq, N_res, H, C), dtype)
    bias = randn(g, (H, N_res, N_res), dtype)
    u = torch.rand(N_seq, N_res, generator=g, dtype=torch.float32)
    key_mask = (u >= masked_frac).to(torch.uint8).contiguous()
    return q, k, v, gate, bias, key_mask


def cache_lengths(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Tokens held by each of B KV caches, int32 uniform on [lo, hi]."""
    return torch.randint(lo, hi + 1, (B,), generator=_gen(seed), dtype=torch.int64).to(torch.int32)


def decode_inputs(B, Hq, Hkv, S_q, S_cap, D, dtype="bf16", seed=0, layout="bhsd"):
    """q [B,Hq,S_q,D] (the newest tokens) and a KV cache of S_cap slots per
    sequence, drawn in the order q, k, v as [B,Hkv,S_cap,D]; for layout
    "bshd" the same values are returned as [B,S_cap,Hkv,D]."""
    g = _gen(seed)
    q = randn(g, (B, Hq, S_q, D), dtype)
    k = randn(g, (B, Hkv, S_cap, D), dtype)
    v = randn(g, (B, Hkv, S_cap, D), dtype)
    if layout == "bshd":
        k, v = k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous()
    return q, k, v


def rotations(n: int, g: torch.Generator) -> torch.Tensor:
    """n rotation matrices [n, 3, 3] (float32, row-major), uniform over the
    rotation group: unit quaternions from normalised 4-d Gaussian draws,
    written out as matrices."""
    u = torch.randn(n, 4, generator=g, dtype=torch.float64)
    w, x, y, z = (u / u.norm(dim=1, keepdim=True)).unbind(1)
    R = torch.stack([
        1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y),
        2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x),
        2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], 1)
    return R.reshape(n, 3, 3).to(torch.float32)


def ipa_inputs(B, L, H, C, Pq, Pv, Cz, dtype="bf16", seed=0, masked_frac=0.0, step=3.8):
    """Invariant Point Attention inputs, drawn in this order:
    q, k, v [B,L,H,C] (N(0,1), dtype); q_pts, k_pts [B,L,H,Pq,3] and v_pts
    [B,L,H,Pv,3] (N(0,1) float32, local coordinates); rot [B,L,3,3] (uniform
    random rotations, float32); trans [B,L,3] (a chain: each residue
    ``step`` apart from the previous one in a uniformly random direction,
    like a protein's C-alpha trace, float32); gamma [H] (softplus of N(0,1),
    float32); pair_bias [B,H,L,L] and z [B,L,L,Cz] (N(0,1), dtype);
    key_mask [B,L] uint8 with each residue excluded with probability
    ``masked_frac``."""
    g = _gen(seed)
    q = randn(g, (B, L, H, C), dtype)
    k = randn(g, (B, L, H, C), dtype)
    v = randn(g, (B, L, H, C), dtype)
    q_pts = randn(g, (B, L, H, Pq, 3), "f32")
    k_pts = randn(g, (B, L, H, Pq, 3), "f32")
    v_pts = randn(g, (B, L, H, Pv, 3), "f32")
    rot = rotations(B * L, g).reshape(B, L, 3, 3).contiguous()
    d = torch.randn(B, L, 3, generator=g, dtype=torch.float64)
    d = d / d.norm(dim=2, keepdim=True) * step
    trans = d.cumsum(1).to(torch.float32).contiguous()
    gamma = torch.nn.functional.softplus(torch.randn(H, generator=g, dtype=torch.float32)).contiguous()
    pair_bias = randn(g, (B, H, L, L), dtype)
    z = randn(g, (B, L, L, Cz), dtype)
    u = torch.rand(B, L, generator=g, dtype=torch.float32)
    key_mask = (u >= masked_frac).to(torch.uint8).contiguous()
    return dict(q=q, k=k, v=v, q_pts=q_pts, k_pts=k_pts, v_pts=v_pts, rot=rot, trans=trans,
                gamma=gamma, pair_bias=pair_bias, z=z, key_mask=key_mask)


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: shapes, dtype, variants and seeds."""

    name: str
    kind: str                    # "attn", "diffattn", "evoformer" or "decode"
    dtype: str
    shape: dict
    variants: tuple
    seed: int
    params: dict = field(default_factory=dict)


ALL_MASK_VARIANTS = ("vanilla", "alibi", "softcap", "causal", "sliding_window",
                     "prefix_lm", "document")

WORKLOADS = {
    # fp32 MHA at a size the oracle finishes in well under a second; returns LSE
    "mha_f32_b1_h2_s128_d64": Workload(
        "mha_f32_b1_h2_s128_d64", "attn", "f32",
        dict(B=1, Hq=2, Hkv=2, S=128, D=64), ("vanilla",), seed=1),
    # FlexAttention-expressible sweep, MHA, S=2048
    "mha_bf16_b4_h16_s2048_d64": Workload(
        "mha_bf16_b4_h16_s2048_d64", "attn", "bf16",
        dict(B=4, Hq=16, Hkv=16, S=2048, D=64), ALL_MASK_VARIANTS, seed=2,
        params=dict(softcap=50.0, alibi_max_bias=8.0, window=256, window_causal=True,
                    prefix=512, n_docs=8, doc_seed=2002)),
    # the same sweep at S=4096: the throughput headline
    "mha_bf16_b4_h16_s4096_d64": Workload(
        "mha_bf16_b4_h16_s4096_d64", "attn", "bf16",
        dict(B=4, Hq=16, Hkv=16, S=4096, D=64), ALL_MASK_VARIANTS, seed=6,
        params=dict(softcap=50.0, alibi_max_bias=8.0, window=256, window_causal=True,
                    prefix=512, n_docs=8, doc_seed=6006)),
    # grouped-query long context
    "gqa_bf16_b1_hq32_hkv8_s16384_d64": Workload(
        "gqa_bf16_b1_hq32_hkv8_s16384_d64", "attn", "bf16",
        dict(B=1, Hq=32, Hkv=8, S=16384, D=64), ("causal", "sliding_window"), seed=3,
        params=dict(window=1024, window_causal=True)),
    # differential attention
    "diffattn_bf16_b4_h16_s4096_dqk64_dv128": Workload(
        "diffattn_bf16_b4_h16_s4096_dqk64_dv128", "diffattn", "bf16",
        dict(B=4, H=16, S=4096, Dqk=64, Dv=128), ("noncausal", "causal"), seed=4,
        params=dict(lam=0.8)),
    # Evoformer MSA gated self-attention, row-wise and column-wise
    "evoformer_bf16_nseq128_nres256_h8_c32": Workload(
        "evoformer_bf16_nseq128_nres256_h8_c32", "evoformer", "bf16",
        dict(N_seq=128, N_res=256, H=8, C=32), ("row", "col"), seed=5,
        params=dict(masked_frac=0.05)),
    # Invariant Point Attention at AlphaFold2's structure-module shape: 256
    # residues, 12 heads of 16 channels, 4 query/key points and 8 value
    # points per head, a 128-channel pair representation
    "ipa_bf16_nres256_h12": Workload(
        "ipa_bf16_nres256_h12", "ipa", "bf16",
        dict(B=1, L=256, H=12, C=16, Pq=4, Pv=8, Cz=128), ("ipa",), seed=8,
        params=dict(masked_frac=0.0)),
    # decode against a KV cache: one new token per sequence, GQA 32/8 with head
    # dim 64 (the shape of the small LLM the pages serve), cache lengths mixed
    # uniformly between 512 and 8192 tokens in place of a serving trace
    "decode_bf16_b64_hq32_hkv8_cap8192_d64": Workload(
        "decode_bf16_b64_hq32_hkv8_cap8192_d64", "decode", "bf16",
        dict(B=64, Hq=32, Hkv=8, Sq=1, S_cap=8192, D=64),
        ("causal", "softcap", "alibi", "sliding_window"), seed=7,
        params=dict(softcap=50.0, alibi_max_bias=8.0, window=1024, window_causal=True,
                    len_lo=512, len_hi=8192, len_seed=7007)),
}


def make(wl: Workload, S: int | None = None):
    """Draw the tensors of workload ``wl`` (optionally at another sequence length)."""
    s = dict(wl.shape)
    if S is not None:
        s["S"] = S
    if wl.kind == "attn":
        q, k, v = attn_inputs(s["B"], s["Hq"], s["Hkv"], s["S"], s["S"], s["D"], wl.dtype, wl.seed)
        out = dict(q=q, k=k, v=v)
        if "n_docs" in wl.params:
            out["doc_offsets"] = doc_offsets(s["B"], s["S"], wl.params["n_docs"],
                                             wl.params["doc_seed"])
        return out
    if wl.kind == "diffattn":
        q1, q2, k1, k2, v = diffattn_inputs(s["B"], s["H"], s["S"], s["Dqk"], s["Dv"],
                                            wl.dtype, wl.seed)
        return dict(q1=q1, q2=q2, k1=k1, k2=k2, v=v)
    if wl.kind == "evoformer":
        q, k, v, gate, bias, km = evoformer_inputs(s["N_seq"], s["N_res"], s["H"], s["C"],
                                                   wl.dtype, wl.seed, wl.params["masked_frac"])
        return dict(q=q, k=k, v=v, gate=gate, pair_bias=bias, key_mask=km)
    if wl.kind == "ipa":
        return ipa_inputs(s["B"], s["L"], s["H"], s["C"], s["Pq"], s["Pv"], s["Cz"], wl.dtype,
                          wl.seed, wl.params["masked_frac"])
    if wl.kind == "decode":
        q, k, v = decode_inputs(s["B"], s["Hq"], s["Hkv"], s["Sq"], s["S_cap"], s["D"], wl.dtype,
                                wl.seed)
        L = cache_lengths(s["B"], wl.params["len_lo"], wl.params["len_hi"], wl.params["len_seed"])
        return dict(q=q, k_cache=k, v_cache=v, seqlens=L)
    raise ValueError(wl.kind)
