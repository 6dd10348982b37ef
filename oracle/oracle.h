/*
 * oracle.h -- plain, slow CPU reference of the fused attention-variant forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library, and neither includes the
 * other.
 *
 * What it computes.  The method on the pages (Flashlight, arXiv 2511.02043)
 * reaches the exact softmax-attention result with a single-pass, tiled,
 * online-softmax kernel; it is not an approximation (Flashlight abstract;
 * gist.science explainer, "Technical Summary: Methodology", semantic fusion
 * paragraph).  So the reference here is the plain definition written out in
 * float64, per query row, in two passes (pass 1: the maximum, pass 2: the sum
 * of exponentials and the weighted sum of values), with no tiling, no fusion
 * and no reordering.  A second routine, the "online twin", walks the keys in
 * blocks and carries a running (max, sum, accumulator) that is rescaled with
 * e^(x-y) = e^x / e^y whenever the max grows -- the single-pass algorithm the
 * pages describe -- and exists only so tests can check that the two agree.
 *
 * Variants (gist.science explainer, "Technical Summary: Results", the
 * FlexAttention-supported list; papers.lqhl.me wiki, "实验与结果"): vanilla,
 * ALiBi, softcap, causal, sliding window, PrefixLM, document mask, each with
 * MHA or GQA heads; and the two variants the pages say FlexAttention cannot
 * express: differential attention and the Evoformer row/column gated
 * self-attention with a broadcast pair bias (same pages, same sections;
 * papers.lqhl.me wiki, "设计取舍", bias broadcast over an extra dimension).
 *
 * Every routine takes float64 row-major arrays and writes float64 outputs.
 * Rows can be restricted to a list so that large problems can be sampled.
 * Return value: 0 on success, a negative number on a bad argument.
 */
#ifndef FLASHLIGHT_ORACLE_H
#define FLASHLIGHT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_VANILLA = 0,
  ORACLE_ALIBI = 1,
  ORACLE_SOFTCAP = 2,
  ORACLE_CAUSAL = 3,
  ORACLE_SLIDING_WINDOW = 4,
  ORACLE_PREFIX_LM = 5,
  ORACLE_DOCUMENT = 6
};

typedef struct {
  int variant;              /* ORACLE_* */
  double scale;             /* multiplies q.k before the score modification */
  double softcap;           /* ORACLE_SOFTCAP: s -> cap * tanh(s / cap) */
  double alibi_max_bias;    /* ORACLE_ALIBI: slope_h = 2^(-max_bias*(h+1)/H_q) */
  int window;               /* ORACLE_SLIDING_WINDOW: W >= 1 keys */
  int window_causal;        /* 1: i-W < j <= i ; 0: |i-j| < W */
  int prefix;               /* ORACLE_PREFIX_LM: j < P or j <= i */
  const int32_t* doc_offsets; /* ORACLE_DOCUMENT: [B][n_docs+1], 0 = o_0 < ... < o_n = S */
  int n_docs;
  int mask;                 /* ORACLE_VANILLA (none) or a mask kind (CAUSAL, SLIDING_WINDOW,
                               PREFIX_LM, DOCUMENT) applied together with the score
                               modification of `variant` (VANILLA, ALIBI, SOFTCAP); must be
                               VANILLA when `variant` is itself a mask */
} oracle_attn_params;

/*
 * Attention rows.  q [B,Hq,Sq,D], k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv],
 * bias NULL or [Hq,Sq,Sk] (added after the score modification, shared by
 * every batch element).  rows: NULL for every row in (b, h, i) order, else a
 * list of flat indices (b*Hq + h)*Sq + i.  o [n_rows, Dv], lse [n_rows]
 * (natural log; may be NULL).  block_keys = 0 selects the two-pass reference,
 * block_keys > 0 the online twin with that many keys per block.
 */
int oracle_attn_rows(const double* q, const double* k, const double* v,
                     const double* bias, double* o, double* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                     const oracle_attn_params* p,
                     const int64_t* rows, int64_t n_rows,
                     int block_keys, int nthreads);

/*
 * Decode rows against a KV cache.  q [B,Hq,Sq,D] holds the Sq newest tokens
 * of each batch entry; k_cache [B,Hkv,S_cap,D], v_cache [B,Hkv,S_cap,Dv]
 * hold seqlens[b] valid tokens (clamped to [0, S_cap]; the new tokens are
 * the last Sq of them), so query i sits at position seqlens[b] - Sq + i and
 * keys j >= seqlens[b] do not exist.  Masks and ALiBi distances use these
 * positions.  Variants: vanilla, ALiBi, softcap, causal, sliding window,
 * PrefixLM, and a mask composed with a score modification; no bias, no
 * document mask.  Rows, outputs and block_keys as for oracle_attn_rows.
 */
int oracle_decode_rows(const double* q, const double* k_cache, const double* v_cache,
                       const int32_t* seqlens, double* o, double* lse,
                       int B, int Hq, int Hkv, int Sq, int S_cap, int D, int Dv,
                       const oracle_attn_params* p, const int64_t* rows,
                       int64_t n_rows, int block_keys, int nthreads);

/*
 * Merge of partial results over disjoint key sets: o_parts [n_parts][n_rows][Dv]
 * (each normalised over its own keys), lse_parts [n_parts][n_rows] (natural
 * log, -inf for a part with no key).  o [n_rows][Dv]; lse [n_rows] or NULL.
 */
int oracle_merge_rows(const double* o_parts, const double* lse_parts, double* o, double* lse,
                      int n_parts, int64_t n_rows, int Dv);

/*
 * Differential attention rows: O = softmax(s(Q1,K1)) V - lambda * softmax(s(Q2,K2)) V
 * with the same scale, the same V and the same (optional causal) mask on both
 * maps.  q1,q2 [B,H,Sq,Dqk]; k1,k2 [B,H,Sk,Dqk]; v [B,H,Sk,Dv]; o [n_rows,Dv];
 * lse1, lse2 [n_rows] or NULL.
 */
int oracle_diffattn_rows(const double* q1, const double* q2,
                         const double* k1, const double* k2, const double* v,
                         double* o, double* lse1, double* lse2,
                         int B, int H, int Sq, int Sk, int Dqk, int Dv,
                         double scale, double lambda, int causal,
                         const int64_t* rows, int64_t n_rows, int nthreads);

/*
 * Evoformer gated self-attention, row-wise form, on the AlphaFold2 layout.
 * q,k,v,gate [N_rows, N_len, H, C]; pair_bias NULL or [H, N_len, N_len]
 * (query i, key j), shared by every row; key_mask NULL or [N_rows, N_len]
 * (1 = keep, 0 = excluded key).  O[r,i,h,:] = sigmoid(G[r,i,h,:]) * attn.
 * rows: NULL for all, else flat indices (r*N_len + i)*H + h.  o [n_rows, C].
 */
int oracle_evoformer_row(const double* q, const double* k, const double* v,
                         const double* gate, const double* pair_bias,
                         const uint8_t* key_mask, double* o,
                         int N_rows, int N_len, int H, int C, double scale,
                         const int64_t* rows, int64_t n_rows, int nthreads);

/*
 * Column-wise form: the same MSA tensors [N_seq, N_res, H, C] attend along
 * the sequence axis within each residue column.  The oracle transposes the
 * tensors to [N_res, N_seq, H, C] itself (and key_mask [N_seq, N_res] to
 * [N_res, N_seq]) and runs the row routine with no pair bias.  rows index the
 * transposed problem: (r*N_seq + s)*H + h with r a residue and s a sequence.
 */
int oracle_evoformer_col(const double* q, const double* k, const double* v,
                         const double* gate, const uint8_t* key_mask, double* o,
                         int N_seq, int N_res, int H, int C, double scale,
                         const int64_t* rows, int64_t n_rows, int nthreads);

/*
 * Invariant Point Attention, attention core (ipa.c; the definition is
 * AlphaFold2's, the pages only name the variant).  Per batch entry b, query
 * residue i and head h:
 *   q, k, v [B, L, H, C]; q_pts, k_pts [B, L, H, Pq, 3] and v_pts
 *   [B, L, H, Pv, 3] in the residues' local frames; rot [B, L, 3, 3]
 *   (row-major) and trans [B, L, 3] map local to global (R x + t);
 *   gamma [H] (the per-head point weight, >= 0); pair_bias NULL or
 *   [B, H, L, L] (query i, key j); z NULL or [B, L, L, Cz] (the pair
 *   representation, query i, key j); key_mask NULL or [B, L] (0 = excluded).
 * rows: NULL for all, else flat indices (b*L + i)*H + h.  Outputs per row:
 *   o [n_rows, C], o_pts [n_rows, Pv, 3] (in the query residue's frame),
 *   o_pair [n_rows, Cz] (NULL exactly when z is NULL).
 */
int oracle_ipa_rows(const double* q, const double* k, const double* v, const double* q_pts,
                    const double* k_pts, const double* v_pts, const double* rot,
                    const double* trans, const double* gamma, const double* pair_bias,
                    const double* z, const uint8_t* key_mask, double* o, double* o_pts,
                    double* o_pair, int B, int L, int H, int C, int Pq, int Pv, int Cz,
                    const int64_t* rows, int64_t n_rows, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
