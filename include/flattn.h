/*
 * flattn.h -- C ABI of the fused attention-variant forward for AMD MI355X
 * (gfx950).
 *
 * One entry point per operation family.  Each computes, in one kernel launch,
 * the single-pass tiled attention forward softmax(score_mod(Q K^T) + bias) V
 * with an online softmax: a running maximum and sum per query row, rescaled
 * whenever the maximum grows (gist.science explainer of Flashlight, arXiv
 * 2511.02043, "Technical Summary: Methodology", semantic fusion paragraph;
 * papers.lqhl.me wiki, "核心方法").  Scores are never written to memory.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or synchronises; the call enqueues one
 *     kernel on `stream` (a hipStream_t; NULL = the default stream) and
 *     returns.  Inputs are read-only; outputs must not alias inputs.
 *   - Argument errors are detected on the host before anything is launched
 *     and are returned synchronously (FL_ERR_*); nothing is written then.
 *     A failed launch returns FL_ERR_LAUNCH.  Faults inside the kernel
 *     surface at the caller's next synchronisation.
 *   - Tensor pointers must be 16-byte aligned (the kernels move 128-bit
 *     words); lse pointers 4-byte aligned.
 *   - dtype FL_BF16: bfloat16 inputs and outputs, float32 accumulation,
 *     probabilities rounded to bfloat16 (round to nearest even) before the
 *     P.V product.  dtype FL_F32: float32 throughout.
 *   - Every output element is written, including rows that no key may
 *     attend to: such a row gets O = 0 and LSE = -inf.
 *   - The library holds no state and is safe to call from several threads.
 */
#ifndef FLATTN_H
#define FLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FL_ABI_VERSION 5

typedef enum {
  FL_OK = 0,
  FL_ERR_NULL = 1,        /* a required pointer is NULL */
  FL_ERR_SHAPE = 2,       /* sizes inconsistent, negative or too large */
  FL_ERR_ALIGN = 3,       /* a pointer or row is not aligned as required */
  FL_ERR_UNSUPPORTED = 4, /* head dimension / dtype combination not built */
  FL_ERR_PARAM = 5,       /* a variant parameter is out of range */
  FL_ERR_LAUNCH = 6,      /* the kernel launch failed */
  FL_ERR_SCRATCH = 7      /* the call needs more scratch than the library's static
                             buffer holds (fl_attn_decode_fwd_noalloc) */
} fl_status;

typedef enum { FL_BF16 = 0, FL_F32 = 1 } fl_dtype;

/*
 * The FlexAttention-expressible variants the pages evaluate (gist.science
 * explainer, "Technical Summary: Results"; papers.lqhl.me wiki, "实验与结果").
 * The pages name them without formulas; the definitions used are:
 *   FL_VANILLA         every key.
 *   FL_ALIBI           s -= slope_h * |i - j|, slope_h = 2^(-alibi_max_bias*(h+1)/H_q).
 *   FL_SOFTCAP         s = softcap * tanh(s / softcap).
 *   FL_CAUSAL          j <= i (top-left aligned).
 *   FL_SLIDING_WINDOW  window_causal = 1: i - window < j <= i (window keys
 *                      including the query itself); 0: |i - j| < window.
 *   FL_PREFIX_LM       j < prefix or j <= i.
 *   FL_DOCUMENT        query and key lie in the same document of
 *                      doc_offsets (block diagonal, not causal).
 * s is the scaled score scale * q.k; the score modification acts on s, the
 * bias is added after it, and masked keys are excluded.  A score
 * modification composes with any mask through fl_attn_params.mask (the
 * pages' premise that variants compose freely: gist.science explainer,
 * "Technical Summary: Methodology"; papers.lqhl.me wiki, "核心方法").
 */
typedef enum {
  FL_VANILLA = 0,
  FL_ALIBI = 1,
  FL_SOFTCAP = 2,
  FL_CAUSAL = 3,
  FL_SLIDING_WINDOW = 4,
  FL_PREFIX_LM = 5,
  FL_DOCUMENT = 6
} fl_variant;

typedef struct {
  int32_t variant;         /* fl_variant */
  float scale;             /* multiplies q.k; usually 1/sqrt(D) */
  float softcap;           /* FL_SOFTCAP: > 0 */
  float alibi_max_bias;    /* FL_ALIBI: >= 0 */
  int32_t window;          /* FL_SLIDING_WINDOW: >= 1 */
  int32_t window_causal;   /* FL_SLIDING_WINDOW: 1 causal, 0 two-sided */
  int32_t prefix;          /* FL_PREFIX_LM: >= 0 */
  int32_t n_docs;          /* FL_DOCUMENT: >= 1 */
  const int32_t* doc_offsets; /* FL_DOCUMENT: device [B][n_docs+1] int32,
                                 0 = o_0 < o_1 < ... < o_n = S.  Not checked
                                 on the host (it is device memory); offsets
                                 outside [0, S] are clamped, never followed
                                 out of bounds. */
  int32_t mask;            /* A mask composed with the score modification of
                              `variant` (FL_VANILLA, FL_ALIBI or FL_SOFTCAP):
                              FL_VANILLA for none, or FL_CAUSAL,
                              FL_SLIDING_WINDOW, FL_PREFIX_LM, FL_DOCUMENT with
                              their parameters above.  The score is modified,
                              the bias added, then the mask applied.  Must be
                              FL_VANILLA when `variant` is itself a mask
                              (FL_ERR_PARAM otherwise).  Added in ABI 2. */
} fl_attn_params;

/*
 * Attention forward with a FlexAttention-class variant, MHA or GQA.
 *   q    [B, H_q,  S_q, D]   contiguous
 *   k    [B, H_kv, S_k, D]   contiguous; query head h uses K/V head
 *   v    [B, H_kv, S_k, D]   h / (H_q / H_kv) (contiguous groups)
 *   bias NULL or [H_q, S_q, S_k] additive score bias, shared by all B,
 *        same dtype as q (FL_BF16 requires S_k % 8 == 0 with a bias)
 *   o    [B, H_q, S_q, D]    output, same dtype as q
 *   lse  NULL or [B, H_q, S_q] float32 natural-log logsumexp of the scores
 * Requires H_q % H_kv == 0; S_q == S_k for the positional masks (causal,
 * sliding window, PrefixLM, document), as variants or composed.  D: 64 for FL_BF16; 32, 64 or 128
 * for FL_F32.  FL_BF16 also requires S_k * D * 2 < 2^31 (one K/V head block
 * is addressed with 32-bit byte offsets); larger S_k returns FL_ERR_SHAPE.
 */
fl_status fl_attn_fwd(const void* q, const void* k, const void* v, const void* bias,
                      void* o, float* lse, int B, int H_q, int H_kv, int S_q, int S_k,
                      int D, fl_dtype dtype, const fl_attn_params* params, void* stream);

/*
 * Differential attention: two softmax maps over the same values combined as
 *   O = softmax(scale Q1 K1^T) V - lambda * softmax(scale Q2 K2^T) V
 * with the same (optional causal, top-left) mask on both maps; MHA only.
 * The pages name it as a variant FlexAttention cannot express (gist.science
 * explainer, "Technical Summary: Problem Statement" and "Results") without a
 * formula; this is the plain combination with a scalar lambda.
 *   q1, q2 [B, H, S_q, D_qk]; k1, k2 [B, H, S_k, D_qk]; v [B, H, S_k, D_v]
 *   o      [B, H, S_q, D_v]
 *   lse1, lse2  NULL or [B, H, S_q] float32, one per map
 * D_qk = 64 and D_v = 128 for FL_BF16 (64/64 also built); FL_F32 the same.
 * causal requires S_q == S_k.
 */
fl_status fl_diffattn_fwd(const void* q1, const void* q2, const void* k1, const void* k2,
                          const void* v, void* o, float* lse1, float* lse2, int B, int H,
                          int S_q, int S_k, int D_qk, int D_v, fl_dtype dtype, float scale,
                          float lambda, int causal, void* stream);

typedef enum { FL_EVO_ROW = 0, FL_EVO_COL = 1 } fl_evo_axis;

/*
 * Evoformer gated self-attention on MSA tensors (AlphaFold2 layout), named on
 * the pages as a data-dependent variant with a bias broadcast over an extra
 * dimension (papers.lqhl.me wiki, "设计取舍"; gist.science explainer,
 * "Technical Summary: Results").
 *   q, k, v, gate, o  [N_seq, N_res, H, C] contiguous
 *   axis FL_EVO_ROW: each MSA row attends along residues (N_res keys);
 *        pair_bias NULL or [H, N_res(query), N_res(key)], shared by all rows;
 *        key_mask NULL or [N_seq, N_res] uint8, 0 excludes that key.
 *   axis FL_EVO_COL: each residue column attends along sequences (N_seq
 *        keys) of the same tensors, read in place (no transpose); pair_bias
 *        must be NULL; key_mask NULL or [N_seq, N_res], 0 excludes that key.
 *   O[s, r, h, :] = sigmoid(gate[s, r, h, :]) * attention output.
 * scale multiplies q.k only (usually 1/sqrt(C)).  C = 32 (the AlphaFold2
 * head width; other widths return FL_ERR_UNSUPPORTED), FL_BF16 or FL_F32.
 * With a pair bias and FL_BF16, N_res % 8 == 0.  An empty tensor (N_seq or
 * N_res 0) returns FL_OK without launching.
 */
fl_status fl_evoformer_gated_attn_fwd(const void* q, const void* k, const void* v,
                                      const void* gate, const void* pair_bias,
                                      const uint8_t* key_mask, void* o, int N_seq, int N_res,
                                      int H, int C, fl_evo_axis axis, fl_dtype dtype,
                                      float scale, void* stream);

/*
 * Decode-phase attention against a KV cache, with the keys of each sequence
 * split over several work-groups and their partial results merged (the
 * serving path the pages leave untested: papers.lqhl.me wiki, "假设压力测试",
 * serving-path paragraph; the merge is the online-softmax rescaling identity
 * applied to whole key ranges: gist.science explainer, "Technical Summary:
 * Methodology", semantic fusion).
 *   q        [B, H_q, S_q, D] contiguous: the S_q newest tokens of each
 *            sequence (S_q = 1 for plain decoding; more for speculative or
 *            chunked steps)
 *   k_cache, v_cache  the cache, S_cap token slots per sequence:
 *            layout FL_KV_BHSD: [B, H_kv, S_cap, D]; FL_KV_BSHD: [B, S_cap, H_kv, D]
 *   cache_seqlens  device int32 [B]: tokens held by each sequence's cache,
 *            the new ones included (they were appended before the call).
 *            Values are clamped to [0, max_seqlen] on the device.
 *   o        [B, H_q, S_q, D] bf16 output; lse NULL or [B, H_q, S_q] float32
 * Query i of sequence b sits at position L_b - S_q + i (L_b its clamped
 * length) and sees the keys 0 .. L_b - 1 that its variant allows, with masks
 * and ALiBi distances taken between positions (a causal mask is therefore
 * bottom-right aligned).  Variants: vanilla, ALiBi, softcap, causal, sliding
 * window, PrefixLM, and a mask composed with a score modification
 * (fl_attn_params.mask); FL_DOCUMENT returns FL_ERR_UNSUPPORTED.  There is
 * no bias.  GQA: the G = H_q / H_kv query heads of a K/V head are handled
 * together, so each cached key is read once per K/V head.
 *   max_seqlen  an upper bound of cache_seqlens, 0 <= max_seqlen <= S_cap:
 *            the keys are cut into ranges up to it
 *   num_splits  key ranges per (sequence, K/V head): 0 lets the library
 *            choose from the shape; 1 computes each row in one pass with no
 *            workspace; more are capped at the number of 64-key tiles.  Each
 *            work-group's ranges cut the keys its rows need into near-equal
 *            parts, so every sequence's work spreads over its work-groups
 *   workspace  device memory, 16-byte aligned, of at least
 *            fl_attn_decode_workspace_size(...) bytes for the same arguments
 *            (may be NULL when that size is 0); it holds the partial results
 *            between the two kernels this call enqueues
 * FL_BF16 with D = 64 only.  Errors: FL_ERR_NULL (q, caches, seqlens, o, or
 * a needed workspace missing), FL_ERR_SHAPE, FL_ERR_ALIGN, FL_ERR_PARAM (bad
 * variant parameters, max_seqlen outside [0, S_cap], workspace too small),
 * FL_ERR_UNSUPPORTED.
 */
typedef enum { FL_KV_BHSD = 0, FL_KV_BSHD = 1 } fl_kv_layout;

fl_status fl_attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cache_seqlens, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, int B, int H_q, int H_kv, int S_q, int S_cap,
                             int max_seqlen, int D, fl_kv_layout layout, fl_dtype dtype,
                             const fl_attn_params* params, int num_splits, void* stream);

/* Workspace bytes fl_attn_decode_fwd needs for the same arguments (0 when
 * it runs one key range per row); -1 for invalid sizes.  params may be NULL
 * (no sliding window); the split choice depends only on the sizes and, for
 * a sliding window, its width. */
int64_t fl_attn_decode_workspace_size(int B, int H_q, int H_kv, int S_q, int max_seqlen, int D,
                                      const fl_attn_params* params, int num_splits);

/* Key ranges per (sequence, K/V head) that fl_attn_decode_fwd uses for the
 * same arguments; -1 for invalid sizes. */
int fl_attn_decode_num_splits(int B, int H_q, int H_kv, int S_q, int max_seqlen,
                              const fl_attn_params* params, int num_splits);

/*
 * Merge of partial attention results over disjoint key sets (the same
 * identity as above): for each of n_rows rows,
 *   LSE = ln sum_p e^(LSE_p),  O = sum_p e^(LSE_p - LSE) O_p,
 * parts with LSE_p = -inf weigh nothing, and a row with no non-empty part
 * gets O = 0, LSE = -inf.
 *   o_parts   device float32 [n_parts][n_rows][D], each part normalised
 *   lse_parts device float32 [n_parts][n_rows], natural log
 *   o         [n_rows][D] of out_dtype; lse NULL or float32 [n_rows]
 * 1 <= n_parts; any D >= 1.  The same exchange merges results computed on
 * different devices over shards of the keys.
 */
fl_status fl_attn_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                        int n_parts, int64_t n_rows, int D, fl_dtype out_dtype, void* stream);

/*
 * Backward of fl_attn_fwd: the gradients of a loss L with dO = dL/dO,
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 *   dS = P * (dO V^T - D) * mod',  D_i = sum_d dO_id O_id,
 * where P is recomputed from the scores and the saved LSE (never stored)
 * and mod' is the derivative of the score modification (1 for vanilla and
 * ALiBi, 1 - tanh^2(s / softcap) for softcap).  The pages name training as
 * future work (gist.science explainer, "Significance and Claims";
 * papers.lqhl.me wiki, "局限与 Future Work"); this is the plain gradient of
 * the forward above.
 *   q, k, v, params   as given to fl_attn_fwd (no bias)
 *   o, lse            its outputs: o [B, H_q, S_q, D], lse [B, H_q, S_q] float32
 *   d_o               [B, H_q, S_q, D], the gradient of the loss w.r.t. o
 *   dq                [B, H_q, S_q, D] output
 *   dk, dv            [B, H_kv, S_k, D] outputs (query heads of a group add
 *                     into their K/V head)
 *   workspace         device float32 [2, B, H_q, S_q] (32 KiB per 4096 rows):
 *                     holds D and the LSE in log2 units between the two
 *                     kernels the call enqueues (twice the size of ABI 4's)
 * FL_BF16 with D = 64 only; every variant and composed mask of
 * fl_attn_fwd; positional masks need S_q == S_k.  Errors as fl_attn_fwd.
 */
fl_status fl_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                      const float* lse, void* dq, void* dk, void* dv, float* workspace, int B,
                      int H_q, int H_kv, int S_q, int S_k, int D, fl_dtype dtype,
                      const fl_attn_params* params, void* stream);

/*
 * fl_attn_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The float32 partial results of
 * a split call go to a static device buffer of FL_DECODE_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the
 * call itself allocates nothing.  Arguments, split choice, results and
 * errors are those of fl_attn_decode_fwd, plus FL_ERR_SCRATCH (returned
 * before anything is launched) when fl_attn_decode_workspace_size for the
 * same arguments exceeds FL_DECODE_SCRATCH_BYTES.  Every call on one GPU
 * shares that GPU's buffer: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  Added in ABI 4.
 */
#define FL_DECODE_SCRATCH_BYTES (32u << 20)
fl_status fl_attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* cache_seqlens, void* o, float* lse, int B,
                                     int H_q, int H_kv, int S_q, int S_cap, int max_seqlen, int D,
                                     fl_kv_layout layout, fl_dtype dtype,
                                     const fl_attn_params* params, int num_splits, void* stream);

/*
 * Attention core of Invariant Point Attention.  The pages name IPA among the
 * data-dependent variants a score_mod/block_mask template cannot express
 * (gist.science explainer, "Technical Summary: Problem Statement";
 * papers.lqhl.me wiki, "问题与动机") but give no formula; the form computed
 * is AlphaFold2's.  Per batch entry b, query residue i, head h, with frames
 * T_r = (R_r, t_r) mapping local to global coordinates (x -> R x + t):
 *   logit_ij = w_L ( q_i.k_j / sqrt(C) + pair_bias_hij
 *                    - gamma_h w_C / 2 sum_p |T_i q_ip - T_j k_jp|^2 ),
 *   w_L = sqrt(1/3), w_C = sqrt(2 / (9 P_q));
 *   a_ij = softmax over the keys key_mask keeps;
 *   o_i = sum_j a_ij v_j;  o_pts_ip = T_i^-1 sum_j a_ij T_j v_jp;
 *   o_pair_i = sum_j a_ij z_ij.
 *   q, k, v        [B, L, H, C] (dtype)
 *   q_pts, k_pts   [B, L, H, P_q, 3] float32, local coordinates
 *   v_pts          [B, L, H, P_v, 3] float32, local coordinates
 *   rot, trans     [B, L, 3, 3] (row-major) and [B, L, 3] float32
 *   gamma          [H] float32 per-head point weight (AlphaFold2 passes a
 *                  softplus, so >= 0)
 *   pair_bias      nullable [B, H, L, L] (query i, key j) (dtype)
 *   z              nullable [B, L, L, C_z] pair representation (dtype);
 *                  o_pair is computed exactly when it is given
 *   key_mask       nullable [B, L] uint8, 0 = the residue is no key
 *   o              [B, L, H, C] output (dtype)
 *   o_pts          [B, L, H, P_v, 3] float32 output, in the query's frame
 *   o_pair         [B, L, H, C_z] output (dtype), NULL exactly when z is
 * A query with no key gets zero outputs.  Points and frames stay float32
 * (absolute coordinates of tens of angstroms would lose the distances in
 * bfloat16).  Supported: FL_BF16 with C = 16, P_q = 4, P_v = 8, C_z in
 * {64, 128} (or no z), 1 <= H; q/k/v/point/output pointers 16-byte
 * aligned, rot/trans/gamma 4-byte aligned.  Errors as fl_attn_fwd.
 */
fl_status fl_ipa_attn_fwd(const void* q, const void* k, const void* v, const float* q_pts,
                          const float* k_pts, const float* v_pts, const float* rot,
                          const float* trans, const float* gamma, const void* pair_bias,
                          const void* z, const uint8_t* key_mask, void* o, float* o_pts,
                          void* o_pair, int B, int L, int H, int C, int P_q, int P_v, int C_z,
                          fl_dtype dtype, void* stream);

/* Human-readable name of a status code (static string). */
const char* fl_status_str(fl_status status);

/* FL_ABI_VERSION of the library that was loaded. */
int fl_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FLATTN_H */
