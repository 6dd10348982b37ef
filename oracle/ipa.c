/*
 * ipa.c -- plain float64 CPU reference of the attention core of Invariant
 * Point Attention.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): only the tests, the smoke check
 * and the benchmark's CPU baseline leg load it; it shares nothing with the
 * GPU library.
 *
 * The pages name Invariant Point Attention only as one of the data-dependent
 * variants a score_mod/block_mask template cannot express (gist.science
 * explainer, "Technical Summary: Problem Statement"; papers.lqhl.me wiki,
 * "问题与动机"); they give no formula.  The definition written out here is
 * AlphaFold2's (Jumper et al., Nature 2021, supplementary section on the
 * structure module, "Invariant point attention"), restricted to its
 * attention core: the projections that produce q, k, v and the points, and
 * the output projection after it, are ordinary dense layers outside it.
 *
 * Per batch entry b, query residue i and head h, with frames T = (R, t)
 * mapping local to global coordinates (x_global = R x + t):
 *
 *   logit_ij = w_L * ( (1/sqrt(C)) q_i . k_j  +  bias_hij
 *                      - (gamma_h w_C / 2) sum_p |T_i q_ip - T_j k_jp|^2 )
 *   w_L = sqrt(1/3),  w_C = sqrt(2 / (9 P_q))
 *   a_ij = softmax over the keys j the key mask keeps
 *   o_i      = sum_j a_ij v_j                                 (C values)
 *   o_pts_ip = T_i^-1 ( sum_j a_ij T_j v_jp )                 (P_v points, local to i)
 *   o_pair_i = sum_j a_ij z_ij                                (C_z values)
 *
 * written as the plain definition in two passes (maximum, then the sums),
 * no tiling or reordering.  A query whose every key is excluded gets zero
 * outputs.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#include "oracle.h"

typedef struct {
  const double *q, *k, *v, *q_pts, *k_pts, *v_pts, *rot, *trans, *gamma, *bias, *z;
  const uint8_t* key_mask;
  double *o, *o_pts, *o_pair;
  int B, L, H, C, Pq, Pv, Cz;
  const int64_t* rows;
  int64_t n_rows;
} ipa_job;

typedef struct {
  const ipa_job* J;
  int64_t begin, end;
} ipa_slice;

/* x_global = R x + t for frame (b, r) */
static void to_global(const ipa_job* J, int b, int r, const double* x, double* y) {
  const double* R = J->rot + ((int64_t)b * J->L + r) * 9;
  const double* t = J->trans + ((int64_t)b * J->L + r) * 3;
  for (int a = 0; a < 3; ++a) y[a] = R[3 * a] * x[0] + R[3 * a + 1] * x[1] + R[3 * a + 2] * x[2] + t[a];
}

/* x_local = R^T (y - t) for frame (b, r) */
static void to_local(const ipa_job* J, int b, int r, const double* y, double* x) {
  const double* R = J->rot + ((int64_t)b * J->L + r) * 9;
  const double* t = J->trans + ((int64_t)b * J->L + r) * 3;
  const double d[3] = {y[0] - t[0], y[1] - t[1], y[2] - t[2]};
  for (int a = 0; a < 3; ++a) x[a] = R[a] * d[0] + R[3 + a] * d[1] + R[6 + a] * d[2];
}

static void* ipa_worker(void* arg) {
  const ipa_slice* S = (const ipa_slice*)arg;
  const ipa_job* J = S->J;
  const int L = J->L, H = J->H, C = J->C, Pq = J->Pq, Pv = J->Pv, Cz = J->Cz;
  const double w_l = sqrt(1.0 / 3.0), w_c = sqrt(2.0 / (9.0 * Pq));
  double* logit = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  unsigned char* ok = (unsigned char*)malloc((size_t)(L > 0 ? L : 1));
  double* qg = (double*)malloc(sizeof(double) * 3 * (size_t)Pq);
  double* og = (double*)malloc(sizeof(double) * 3 * (size_t)(Pv > 0 ? Pv : 1));
  for (int64_t t = S->begin; t < S->end; ++t) {
    const int64_t flat = J->rows ? J->rows[t] : t; /* (b*L + i)*H + h */
    const int h = (int)(flat % H);
    const int i = (int)((flat / H) % L);
    const int b = (int)(flat / ((int64_t)H * L));
    const double* qi = J->q + flat * C;
    for (int p = 0; p < Pq; ++p) to_global(J, b, i, J->q_pts + (flat * Pq + p) * 3, qg + 3 * p);
    /* pass 1: logits of the allowed keys and their maximum */
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
      ok[j] = J->key_mask ? (J->key_mask[(int64_t)b * L + j] != 0) : 1;
      if (!ok[j]) continue;
      const int64_t kf = ((int64_t)b * L + j) * H + h;
      double dot = 0.0;
      for (int c = 0; c < C; ++c) dot += qi[c] * J->k[kf * C + c];
      double d2 = 0.0;
      for (int p = 0; p < Pq; ++p) {
        double kg[3];
        to_global(J, b, j, J->k_pts + (kf * Pq + p) * 3, kg);
        for (int a = 0; a < 3; ++a) d2 += (qg[3 * p + a] - kg[a]) * (qg[3 * p + a] - kg[a]);
      }
      double s = dot / sqrt((double)C) - 0.5 * J->gamma[h] * w_c * d2;
      if (J->bias) s += J->bias[(((int64_t)b * H + h) * L + i) * L + j];
      s *= w_l;
      logit[j] = s;
      if (s > m) m = s;
    }
    double* o = J->o + t * C;
    double* op = J->o_pts + t * Pv * 3;
    double* oz = J->o_pair ? J->o_pair + t * Cz : NULL;
    for (int c = 0; c < C; ++c) o[c] = 0.0;
    for (int e = 0; e < 3 * Pv; ++e) op[e] = og[e] = 0.0;
    if (oz)
      for (int n = 0; n < Cz; ++n) oz[n] = 0.0;
    if (m == -INFINITY) continue; /* no key allowed: zero outputs */
    /* pass 2: weights e^(logit - m), their sum and the weighted sums */
    double l = 0.0;
    for (int j = 0; j < L; ++j) {
      if (!ok[j]) continue;
      const double w = exp(logit[j] - m);
      l += w;
      const int64_t kf = ((int64_t)b * L + j) * H + h;
      for (int c = 0; c < C; ++c) o[c] += w * J->v[kf * C + c];
      for (int p = 0; p < Pv; ++p) {
        double vg[3];
        to_global(J, b, j, J->v_pts + (kf * Pv + p) * 3, vg);
        for (int a = 0; a < 3; ++a) og[3 * p + a] += w * vg[a];
      }
      if (oz) {
        const double* zij = J->z + (((int64_t)b * L + i) * L + j) * Cz;
        for (int n = 0; n < Cz; ++n) oz[n] += w * zij[n];
      }
    }
    for (int c = 0; c < C; ++c) o[c] /= l;
    for (int p = 0; p < Pv; ++p) {
      double g[3] = {og[3 * p] / l, og[3 * p + 1] / l, og[3 * p + 2] / l};
      to_local(J, b, i, g, op + 3 * p);
    }
    if (oz)
      for (int n = 0; n < Cz; ++n) oz[n] /= l;
  }
  free(logit);
  free(ok);
  free(qg);
  free(og);
  return NULL;
}

int oracle_ipa_rows(const double* q, const double* k, const double* v, const double* q_pts,
                    const double* k_pts, const double* v_pts, const double* rot,
                    const double* trans, const double* gamma, const double* pair_bias,
                    const double* z, const uint8_t* key_mask, double* o, double* o_pts,
                    double* o_pair, int B, int L, int H, int C, int Pq, int Pv, int Cz,
                    const int64_t* rows, int64_t n_rows, int nthreads) {
  if (!q || !k || !v || !q_pts || !k_pts || !v_pts || !rot || !trans || !gamma || !o || !o_pts)
    return -1;
  if (B < 0 || L < 0 || H < 1 || C < 1 || Pq < 1 || Pv < 0 || Cz < 0) return -2;
  if ((z == NULL) != (o_pair == NULL)) return -3;
  const int64_t total = (int64_t)B * L * H;
  if (rows) {
    for (int64_t t = 0; t < n_rows; ++t)
      if (rows[t] < 0 || rows[t] >= total) return -4;
  } else if (n_rows != total) {
    return -4;
  }
  ipa_job J = {q, k, v, q_pts, k_pts, v_pts, rot, trans, gamma, pair_bias, z, key_mask,
               o, o_pts, o_pair, B, L, H, C, Pq, Pv, Cz, rows, n_rows};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n_rows) nthreads = n_rows > 0 ? (int)n_rows : 1;
  pthread_t tid[256];
  ipa_slice sl[256];
  const int64_t per = (n_rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    sl[t].J = &J;
    sl[t].begin = per * t < n_rows ? per * t : n_rows;
    sl[t].end = per * (t + 1) < n_rows ? per * (t + 1) : n_rows;
  }
  if (nthreads == 1) {
    ipa_worker(&sl[0]);
    return 0;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&tid[t], NULL, ipa_worker, &sl[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(tid[t], NULL);
  return 0;
}
