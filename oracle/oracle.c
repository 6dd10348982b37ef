/*
 * oracle.c -- plain float64 CPU reference of the fused attention-variant
 * forward.  TEST INFRASTRUCTURE ONLY (see oracle.h): nothing on the product
 * path may call it.
 *
 * Per query row the reference is the textbook definition of softmax
 * attention with a score modification, an additive bias and a mask:
 *
 *   s_j  = mod(scale * q.k_j) + bias_j        for every allowed key j
 *   m    = max_j s_j                          (pass 1)
 *   l    = sum_j exp(s_j - m)                 (pass 2)
 *   o    = sum_j exp(s_j - m) v_j / l,  lse = m + ln l
 *
 * A row with no allowed key gets o = 0 and lse = -inf.
 *
 * The stable two-pass softmax (maximum, then the sum of exponentials) is the
 * form the pages start from before the single-pass rewrite (gist.science
 * explainer, "Technical Summary: Methodology", semantic fusion paragraph;
 * papers.lqhl.me wiki, "关键观察", observation 2).
 *
 * Rows are split over host threads; each row is computed start to finish by
 * one thread, so threading changes no arithmetic.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Masks.  Which key j may query i see?  (gist.science explainer, "Technical
 * Summary: Results", FlexAttention-supported block_mask variants; the pages
 * name them without formulas, the readings below are the plain ones.)       */

static int doc_of(const int32_t* off, int n_docs, int x) {
  /* document d holds positions off[d] <= x < off[d+1] */
  for (int d = 0; d < n_docs; ++d)
    if (x >= off[d] && x < off[d + 1]) return d;
  return -1;
}

/* The mask in force: the variant's own, or the one composed with a score
 * modification.  The pages' point is that variants compose freely (the
 * gist.science explainer, "Technical Summary: Methodology": arbitrary
 * attention programs; papers.lqhl.me wiki, "核心方法"); a composed variant
 * modifies the scores and then masks them, the same order as a single one. */
static int mask_kind(const oracle_attn_params* p) {
  return p->variant >= ORACLE_CAUSAL ? p->variant : p->mask;
}

static int allowed(const oracle_attn_params* p, int b, int i, int j) {
  switch (mask_kind(p)) {
    case ORACLE_CAUSAL:
      /* top-left aligned: a query sees itself and everything before it */
      return j <= i;
    case ORACLE_SLIDING_WINDOW:
      if (p->window_causal) return j <= i && j > i - p->window; /* W keys incl. self */
      return abs(i - j) < p->window;                            /* two-sided */
    case ORACLE_PREFIX_LM:
      /* bidirectional inside the prefix, causal after it */
      return j < p->prefix || j <= i;
    case ORACLE_DOCUMENT: {
      const int32_t* off = p->doc_offsets + (size_t)b * (p->n_docs + 1);
      return doc_of(off, p->n_docs, i) == doc_of(off, p->n_docs, j);
    }
    default:
      return 1; /* vanilla, ALiBi and softcap see every key */
  }
}

/* ------------------------------------------------------------------------ */
/* Score modification (FlexAttention's score_mod class: ALiBi, softcap).     */

static double alibi_slope(const oracle_attn_params* p, int h, int Hq) {
  /* geometric head slopes 2^(-max_bias*(h+1)/H) */
  return pow(2.0, -p->alibi_max_bias * (double)(h + 1) / (double)Hq);
}

static double score(const oracle_attn_params* p, const double* qi,
                    const double* kj, int D, int h, int Hq, int i, int j,
                    const double* bias_row) {
  double dot = 0.0;
  for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
  double s = p->scale * dot;
  if (p->variant == ORACLE_ALIBI) s -= alibi_slope(p, h, Hq) * fabs((double)(i - j));
  if (p->variant == ORACLE_SOFTCAP) s = p->softcap * tanh(s / p->softcap);
  if (bias_row) s += bias_row[j];
  return s;
}

/* ------------------------------------------------------------------------ */
/* One query row, two passes.                                               */

typedef struct {
  const double *q, *k, *v, *bias;
  double *o, *lse;
  int B, Hq, Hkv, Sq, Sk, D, Dv;
  const oracle_attn_params* p;
  const int64_t* rows;
  int64_t n_rows;
  int block_keys;
  const int32_t* seqlens; /* decode: tokens held in each batch entry's cache */
} attn_job;

/* Where a query row sits and how many keys it may look at.  In a prefill
 * call query i is position i and all S_k keys exist.  In a decode call the
 * cache of batch entry b holds L_b tokens (0 <= L_b <= S_k), the S_q new
 * queries are its last S_q tokens, so query i sits at position L_b - S_q + i,
 * and keys at or past L_b do not exist.  The pages name decode-phase
 * KV-cache attention only as serving work they leave untested (papers.lqhl.me
 * wiki, "假设压力测试", serving path); the cache convention taken is the
 * usual one, the new tokens appended before they attend. */
static void row_geometry(const attn_job* J, int b, int i, int* pos, int* n_keys) {
  if (!J->seqlens) {
    *pos = i;
    *n_keys = J->Sk;
    return;
  }
  int L = J->seqlens[b];
  if (L < 0) L = 0;
  if (L > J->Sk) L = J->Sk;
  *pos = L - J->Sq + i;
  *n_keys = L;
}

static void attn_row_two_pass(const attn_job* J, int64_t flat, double* out,
                              double* lse_out, double* s_buf,
                              unsigned char* ok) {
  const int Hq = J->Hq, Sq = J->Sq, Sk = J->Sk, D = J->D, Dv = J->Dv;
  const int i = (int)(flat % Sq);
  const int h = (int)((flat / Sq) % Hq);
  const int b = (int)(flat / ((int64_t)Sq * Hq));
  /* grouped-query heads: H_q/H_kv consecutive query heads share one K/V head */
  const int hk = h / (Hq / J->Hkv);
  const double* qi = J->q + flat * D;
  const double* kb = J->k + ((int64_t)b * J->Hkv + hk) * Sk * D;
  const double* vb = J->v + ((int64_t)b * J->Hkv + hk) * Sk * Dv;
  const double* bias_row = J->bias ? J->bias + ((int64_t)h * Sq + i) * Sk : NULL;
  int pos, nk;
  row_geometry(J, b, i, &pos, &nk);

  /* pass 1: scores of the allowed keys and their maximum */
  double m = -INFINITY;
  int any = 0;
  for (int j = 0; j < nk; ++j) {
    ok[j] = (unsigned char)allowed(J->p, b, pos, j);
    if (!ok[j]) continue;
    s_buf[j] = score(J->p, qi, kb + (int64_t)j * D, D, h, Hq, pos, j, bias_row);
    if (s_buf[j] > m) m = s_buf[j];
    any = 1;
  }
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  if (!any || m == -INFINITY) {
    /* no key allowed, or every allowed score is -inf (a -inf bias row) */
    if (lse_out) *lse_out = -INFINITY;
    return;
  }
  /* pass 2: sum of exponentials and the weighted sum of values */
  double l = 0.0;
  for (int j = 0; j < nk; ++j) {
    if (!ok[j]) continue;
    const double e = exp(s_buf[j] - m);
    l += e;
    const double* vj = vb + (int64_t)j * Dv;
    for (int d = 0; d < Dv; ++d) out[d] += e * vj[d];
  }
  for (int d = 0; d < Dv; ++d) out[d] /= l;
  if (lse_out) *lse_out = m + log(l);
}

/*
 * The online twin: keys in blocks of nb; after each block the running max
 * moves to m' = max(m, block max), and the running sum and accumulator are
 * rescaled by e^(m - m') before the block's terms e^(s - m') are added
 * (gist.science explainer, "Technical Summary: Methodology", semantic fusion
 * with algebraic transformation; papers.lqhl.me wiki, "核心方法").
 */
static void attn_row_online(const attn_job* J, int64_t flat, double* out,
                            double* lse_out, double* s_buf, unsigned char* ok) {
  const int Hq = J->Hq, Sq = J->Sq, Sk = J->Sk, D = J->D, Dv = J->Dv;
  const int nb = J->block_keys;
  const int i = (int)(flat % Sq);
  const int h = (int)((flat / Sq) % Hq);
  const int b = (int)(flat / ((int64_t)Sq * Hq));
  const int hk = h / (Hq / J->Hkv);
  const double* qi = J->q + flat * D;
  const double* kb = J->k + ((int64_t)b * J->Hkv + hk) * Sk * D;
  const double* vb = J->v + ((int64_t)b * J->Hkv + hk) * Sk * Dv;
  const double* bias_row = J->bias ? J->bias + ((int64_t)h * Sq + i) * Sk : NULL;
  int pos, nk;
  row_geometry(J, b, i, &pos, &nk);

  double m = -INFINITY, l = 0.0;
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  for (int j0 = 0; j0 < nk; j0 += nb) {
    const int j1 = j0 + nb < nk ? j0 + nb : nk;
    double mb = -INFINITY;
    for (int j = j0; j < j1; ++j) {
      ok[j] = (unsigned char)allowed(J->p, b, pos, j);
      if (!ok[j]) continue;
      s_buf[j] = score(J->p, qi, kb + (int64_t)j * D, D, h, Hq, pos, j, bias_row);
      if (s_buf[j] > mb) mb = s_buf[j];
    }
    if (mb == -INFINITY) continue; /* nothing allowed in this block */
    const double m_new = mb > m ? mb : m;
    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
    l *= alpha;
    for (int d = 0; d < Dv; ++d) out[d] *= alpha;
    for (int j = j0; j < j1; ++j) {
      if (!ok[j]) continue;
      const double e = exp(s_buf[j] - m_new);
      l += e;
      const double* vj = vb + (int64_t)j * Dv;
      for (int d = 0; d < Dv; ++d) out[d] += e * vj[d];
    }
    m = m_new;
  }
  if (m == -INFINITY) {
    if (lse_out) *lse_out = -INFINITY;
    return;
  }
  for (int d = 0; d < Dv; ++d) out[d] /= l;
  if (lse_out) *lse_out = m + log(l);
}

/* ------------------------------------------------------------------------ */
/* Thread pool over rows.                                                   */

typedef struct {
  const attn_job* J;
  int64_t begin, end;
} attn_slice;

static void* attn_worker(void* arg) {
  const attn_slice* S = (const attn_slice*)arg;
  const attn_job* J = S->J;
  double* s_buf = (double*)malloc(sizeof(double) * (size_t)(J->Sk > 0 ? J->Sk : 1));
  unsigned char* ok = (unsigned char*)malloc((size_t)(J->Sk > 0 ? J->Sk : 1));
  for (int64_t r = S->begin; r < S->end; ++r) {
    const int64_t flat = J->rows ? J->rows[r] : r;
    double* out = J->o + r * J->Dv;
    double* lo = J->lse ? J->lse + r : NULL;
    if (J->block_keys > 0)
      attn_row_online(J, flat, out, lo, s_buf, ok);
    else
      attn_row_two_pass(J, flat, out, lo, s_buf, ok);
  }
  free(s_buf);
  free(ok);
  return NULL;
}

static void run_rows(const attn_job* J, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > J->n_rows) nthreads = J->n_rows > 0 ? (int)J->n_rows : 1;
  pthread_t tid[256];
  attn_slice sl[256];
  const int64_t per = (J->n_rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    sl[t].J = J;
    sl[t].begin = per * t < J->n_rows ? per * t : J->n_rows;
    sl[t].end = per * (t + 1) < J->n_rows ? per * (t + 1) : J->n_rows;
  }
  if (nthreads == 1) {
    attn_worker(&sl[0]);
    return;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&tid[t], NULL, attn_worker, &sl[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(tid[t], NULL);
}

static int check_rows(const int64_t* rows, int64_t n_rows, int64_t total) {
  if (!rows) return n_rows == total ? 0 : -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return -1;
  return 0;
}

int oracle_attn_rows(const double* q, const double* k, const double* v,
                     const double* bias, double* o, double* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D, int Dv,
                     const oracle_attn_params* p, const int64_t* rows,
                     int64_t n_rows, int block_keys, int nthreads) {
  if (!q || !k || !v || !o || !p) return -1;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 0 || Sk < 0 || D < 1 || Dv < 1) return -2;
  if (p->variant < ORACLE_VANILLA || p->variant > ORACLE_DOCUMENT) return -3;
  if (p->mask != ORACLE_VANILLA &&
      (p->variant >= ORACLE_CAUSAL || p->mask < ORACLE_CAUSAL || p->mask > ORACLE_DOCUMENT))
    return -3;
  if (mask_kind(p) == ORACLE_DOCUMENT && (!p->doc_offsets || p->n_docs < 1)) return -3;
  if (p->variant == ORACLE_SOFTCAP && !(p->softcap > 0.0)) return -3;
  if (mask_kind(p) == ORACLE_SLIDING_WINDOW && p->window < 1) return -3;
  const int64_t total = (int64_t)B * Hq * Sq;
  if (check_rows(rows, n_rows, total)) return -4;
  attn_job J = {q, k, v, bias, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, p, rows, n_rows, block_keys,
               NULL};
  run_rows(&J, nthreads);
  return 0;
}

int oracle_decode_rows(const double* q, const double* k_cache, const double* v_cache,
                       const int32_t* seqlens, double* o, double* lse,
                       int B, int Hq, int Hkv, int Sq, int S_cap, int D, int Dv,
                       const oracle_attn_params* p, const int64_t* rows,
                       int64_t n_rows, int block_keys, int nthreads) {
  if (!q || !k_cache || !v_cache || !seqlens || !o || !p) return -1;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || Sq < 0 || S_cap < 0 || D < 1 || Dv < 1)
    return -2;
  if (p->variant < ORACLE_VANILLA || p->variant > ORACLE_PREFIX_LM) return -3;
  if (p->mask != ORACLE_VANILLA &&
      (p->variant >= ORACLE_CAUSAL || p->mask < ORACLE_CAUSAL || p->mask > ORACLE_PREFIX_LM))
    return -3;
  if (p->variant == ORACLE_SOFTCAP && !(p->softcap > 0.0)) return -3;
  if (mask_kind(p) == ORACLE_SLIDING_WINDOW && p->window < 1) return -3;
  const int64_t total = (int64_t)B * Hq * Sq;
  if (check_rows(rows, n_rows, total)) return -4;
  attn_job J = {q, k_cache, v_cache, NULL, o, lse, B, Hq, Hkv, Sq, S_cap, D, Dv, p, rows,
               n_rows, block_keys, seqlens};
  run_rows(&J, nthreads);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Merge of partial results over disjoint key sets.  Each part p carries the */
/* softmax-normalised output O_p and log-sum-exp LSE_p of its keys; the      */
/* whole is LSE = ln sum_p e^LSE_p and O = sum_p e^(LSE_p - LSE) O_p: the    */
/* rescaling identity the single-pass rewrite rests on (gist.science         */
/* explainer, "Technical Summary: Methodology", semantic fusion; papers.     */
/* lqhl.me wiki, "关键观察", observation 2), applied to whole parts.  Parts  */
/* with LSE = -inf hold no key and weigh nothing; if every part is empty the */
/* row gets O = 0 and LSE = -inf.                                            */

int oracle_merge_rows(const double* o_parts, const double* lse_parts, double* o, double* lse,
                      int n_parts, int64_t n_rows, int Dv) {
  if (!o_parts || !lse_parts || !o || n_parts < 1 || n_rows < 0 || Dv < 1) return -1;
  for (int64_t r = 0; r < n_rows; ++r) {
    double m = -INFINITY;
    for (int p = 0; p < n_parts; ++p) {
      const double x = lse_parts[(int64_t)p * n_rows + r];
      if (x > m) m = x;
    }
    double* out = o + r * Dv;
    for (int d = 0; d < Dv; ++d) out[d] = 0.0;
    if (m == -INFINITY) {
      if (lse) lse[r] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int p = 0; p < n_parts; ++p) l += exp(lse_parts[(int64_t)p * n_rows + r] - m);
    const double whole = m + log(l);
    for (int p = 0; p < n_parts; ++p) {
      const double w = exp(lse_parts[(int64_t)p * n_rows + r] - whole);
      const double* op = o_parts + ((int64_t)p * n_rows + r) * Dv;
      for (int d = 0; d < Dv; ++d) out[d] += w * op[d];
    }
    if (lse) lse[r] = whole;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Differential attention: two softmax maps over the same values, combined  */
/* as map1 - lambda * map2 (named on the pages as a variant FlexAttention   */
/* cannot express: gist.science explainer, "Technical Summary: Problem       */
/* Statement" and "Results"; the pages give no formula, the combination is   */
/* the plain one).                                                           */

int oracle_diffattn_rows(const double* q1, const double* q2, const double* k1,
                         const double* k2, const double* v, double* o,
                         double* lse1, double* lse2, int B, int H, int Sq,
                         int Sk, int Dqk, int Dv, double scale, double lambda,
                         int causal, const int64_t* rows, int64_t n_rows,
                         int nthreads) {
  if (!q1 || !q2 || !k1 || !k2 || !v || !o) return -1;
  const int64_t total = (int64_t)B * H * Sq;
  if (check_rows(rows, n_rows, total)) return -4;
  oracle_attn_params p;
  memset(&p, 0, sizeof p);
  p.variant = causal ? ORACLE_CAUSAL : ORACLE_VANILLA;
  p.scale = scale;
  double* o2 = (double*)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * Dv);
  if (!o2) return -5;
  int rc = oracle_attn_rows(q1, k1, v, NULL, o, lse1, B, H, H, Sq, Sk, Dqk, Dv, &p,
                            rows, n_rows, 0, nthreads);
  if (!rc)
    rc = oracle_attn_rows(q2, k2, v, NULL, o2, lse2, B, H, H, Sq, Sk, Dqk, Dv, &p,
                          rows, n_rows, 0, nthreads);
  if (!rc)
    for (int64_t r = 0; r < n_rows * Dv; ++r) o[r] -= lambda * o2[r];
  free(o2);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Evoformer gated self-attention (row-wise) on [N_rows, N_len, H, C]:      */
/* scores get the pair bias for (head, query, key), shared by all rows, and */
/* excluded keys; the output is gated elementwise by sigmoid(G).  The pages */
/* name this variant and its broadcast bias (papers.lqhl.me wiki, "设计取舍";*/
/* gist.science explainer, "Technical Summary: Results") without formulas;  */
/* the form used is AlphaFold2's MSA row attention with pair bias.          */

typedef struct {
  const double *q, *k, *v, *gate, *bias;
  const uint8_t* key_mask;
  double* o;
  int N_rows, N_len, H, C;
  double scale;
  const int64_t* rows;
  int64_t n_rows;
} evo_job;

typedef struct {
  const evo_job* J;
  int64_t begin, end;
} evo_slice;

static void* evo_worker(void* arg) {
  const evo_slice* S = (const evo_slice*)arg;
  const evo_job* J = S->J;
  const int L = J->N_len, H = J->H, C = J->C;
  double* s_buf = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  unsigned char* ok = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
  for (int64_t t = S->begin; t < S->end; ++t) {
    const int64_t flat = J->rows ? J->rows[t] : t;
    const int h = (int)(flat % H);
    const int i = (int)((flat / H) % L);
    const int r = (int)(flat / ((int64_t)H * L));
    const double* qi = J->q + flat * C;
    double* out = J->o + t * C;
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < L; ++j) {
      ok[j] = J->key_mask ? (J->key_mask[(int64_t)r * L + j] != 0) : 1;
      if (!ok[j]) continue;
      const double* kj = J->k + (((int64_t)r * L + j) * H + h) * C;
      double dot = 0.0;
      for (int c = 0; c < C; ++c) dot += qi[c] * kj[c];
      double s = J->scale * dot;
      if (J->bias) s += J->bias[((int64_t)h * L + i) * L + j];
      s_buf[j] = s;
      if (s > m) m = s;
      any = 1;
    }
    for (int c = 0; c < C; ++c) out[c] = 0.0;
    if (!any || m == -INFINITY) continue; /* every key excluded: the row is 0 */
    double l = 0.0;
    for (int j = 0; j < L; ++j) {
      if (!ok[j]) continue;
      const double e = exp(s_buf[j] - m);
      l += e;
      const double* vj = J->v + (((int64_t)r * L + j) * H + h) * C;
      for (int c = 0; c < C; ++c) out[c] += e * vj[c];
    }
    const double* gi = J->gate + flat * C;
    for (int c = 0; c < C; ++c) out[c] = (out[c] / l) * (1.0 / (1.0 + exp(-gi[c])));
  }
  free(s_buf);
  free(ok);
  return NULL;
}

int oracle_evoformer_row(const double* q, const double* k, const double* v,
                         const double* gate, const double* pair_bias,
                         const uint8_t* key_mask, double* o, int N_rows,
                         int N_len, int H, int C, double scale,
                         const int64_t* rows, int64_t n_rows, int nthreads) {
  if (!q || !k || !v || !gate || !o) return -1;
  if (N_rows < 0 || N_len < 0 || H < 1 || C < 1) return -2;
  const int64_t total = (int64_t)N_rows * N_len * H;
  if (check_rows(rows, n_rows, total)) return -4;
  evo_job J = {q, k, v, gate, pair_bias, key_mask, o, N_rows, N_len, H, C, scale, rows, n_rows};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n_rows) nthreads = n_rows > 0 ? (int)n_rows : 1;
  pthread_t tid[256];
  evo_slice sl[256];
  const int64_t per = (n_rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    sl[t].J = &J;
    sl[t].begin = per * t < n_rows ? per * t : n_rows;
    sl[t].end = per * (t + 1) < n_rows ? per * (t + 1) : n_rows;
  }
  if (nthreads == 1) {
    evo_worker(&sl[0]);
    return 0;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&tid[t], NULL, evo_worker, &sl[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(tid[t], NULL);
  return 0;
}

int oracle_evoformer_col(const double* q, const double* k, const double* v,
                         const double* gate, const uint8_t* key_mask, double* o,
                         int N_seq, int N_res, int H, int C, double scale,
                         const int64_t* rows, int64_t n_rows, int nthreads) {
  if (!q || !k || !v || !gate || !o) return -1;
  if (N_seq < 0 || N_res < 0 || H < 1 || C < 1) return -2;
  const size_t n = (size_t)N_seq * N_res * H * C;
  double* t[4];
  const double* src[4] = {q, k, v, gate};
  uint8_t* mt = NULL;
  for (int a = 0; a < 4; ++a) {
    t[a] = (double*)malloc(sizeof(double) * (n ? n : 1));
    if (!t[a]) return -5;
    /* [s, r, h, c] -> [r, s, h, c] */
    for (int s = 0; s < N_seq; ++s)
      for (int r = 0; r < N_res; ++r)
        memcpy(t[a] + (((size_t)r * N_seq + s) * H) * C,
               src[a] + (((size_t)s * N_res + r) * H) * C, sizeof(double) * (size_t)H * C);
  }
  if (key_mask) {
    mt = (uint8_t*)malloc((size_t)N_seq * N_res + 1);
    for (int s = 0; s < N_seq; ++s)
      for (int r = 0; r < N_res; ++r) mt[(size_t)r * N_seq + s] = key_mask[(size_t)s * N_res + r];
  }
  const int rc = oracle_evoformer_row(t[0], t[1], t[2], t[3], NULL, mt, o, N_res, N_seq, H, C,
                                      scale, rows, n_rows, nthreads);
  for (int a = 0; a < 4; ++a) free(t[a]);
  free(mt);
  return rc;
}
