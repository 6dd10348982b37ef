// attn_f32.hpp -- float32 fused attention forward (vector ALU, gfx950).
//
// The float32 dtype exists for accuracy, not throughput: one lane per query
// row, 64 rows per work-group (one wave), K/V tiles of 32 keys staged in LDS
// and read back as broadcasts.  Per tile the lane computes its 32 scores,
// moves the running max, rescales the running sum and accumulator by
// 2^(m_old - m_new), and adds the tile's terms -- the same single-pass online
// softmax as the matrix-core kernel, in float32 throughout (gist.science
// explainer of Flashlight, "Technical Summary: Methodology", semantic fusion).
// DiffAttn runs its two streams one after the other: the first stream's
// normalised output is parked in the output row, the second subtracts
// lambda times its own.
#pragma once

#include "fl_common.hpp"

namespace fl {

// Bias, key mask and gate are runtime switches here (a null pointer turns
// them off); head dims, stream count and score modification are compiled in.
template <int DQK_, int DV_, int NS_, int MOD_>
struct F32Cfg {
  static constexpr int DQK = DQK_, DV = DV_, NS = NS_, MOD = MOD_;
  static constexpr int BM = 64;  // query rows per work-group (one per lane)
  static constexpr int BN = 32;  // keys per tile
};

template <class C>
__global__ __launch_bounds__(64) void attn_f32_kernel(KernelArgs a) {
  constexpr int BN = C::BN, DQK = C::DQK, DV = C::DV;
  __shared__ float ks[BN][DQK];
  __shared__ float vs[BN][DV];
  __shared__ float kms[BN];

  const int lane = threadIdx.x;
  int bh, qt;
  decode_tile(a, blockIdx.x, bh, qt);
  const int b = bh / a.nh, h = bh % a.nh, hk = h / a.group;
  const int q0 = qt * C::BM;
  const int qi = q0 + lane;
  const bool valid = qi < a.sq;
  const int qlast = min(q0 + C::BM, a.sq) - 1;

  int lo_first, hi_first, lo_last, hi_last, lo, hi;
  key_interval(a, b, q0, lo_first, hi_first);
  key_interval(a, b, qlast, lo_last, hi_last);
  key_interval(a, b, min(qi, a.sq - 1), lo, hi);
  const int kt_lo = lo_first / BN;
  const int kt_hi = hi_last >= lo_first ? (hi_last + BN) / BN : kt_lo;
  const float alibi_l2 = C::MOD == MOD_ALIBI ? alibi_slope_log2(a, h) : 0.0f;

  float* op = (float*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)min(qi, a.sq - 1) * a.o_si;

  for (int s = 0; s < C::NS; ++s) {
    float q[DQK];
    const float* qp = (const float*)a.q[s] + b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_si;
#pragma unroll
    for (int d = 0; d < DQK; ++d) q[d] = valid ? qp[d] : 0.0f;
    const float* kb = (const float*)a.k[s] + b * a.k_sb + hk * a.k_sh;
    const float* vb = (const float*)a.v + b * a.v_sb + hk * a.v_sh;

    float acc[DV];
#pragma unroll
    for (int d = 0; d < DV; ++d) acc[d] = 0.0f;
    float m = kNegInf, l = 0.0f;

    for (int kt = kt_lo; kt < kt_hi; ++kt) {
      const int j0 = kt * BN;
      __syncthreads();
      for (int e = lane; e < BN * DQK; e += 64) {
        const int j = e / DQK, d = e % DQK;
        ks[j][d] = j0 + j < a.sk ? kb[(int64_t)(j0 + j) * a.k_si + d] : 0.0f;
      }
      for (int e = lane; e < BN * DV; e += 64) {
        const int j = e / DV, d = e % DV;
        vs[j][d] = j0 + j < a.sk ? vb[(int64_t)(j0 + j) * a.v_si + d] : 0.0f;
      }
      if (lane < BN) {
        const int j = j0 + lane;
        kms[lane] = (j < a.sk && (!a.kmask || a.kmask[b * a.km_sb + (int64_t)j * a.km_sj] != 0))
                        ? 0.0f
                        : kNegInf;
      }
      __syncthreads();

      // scores of this tile, base 2
      float x[BN];
      float xm = kNegInf;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const int key = j0 + j;
        float dot = 0.0f;
#pragma unroll
        for (int d = 0; d < DQK; ++d) dot = __builtin_fmaf(q[d], ks[j][d], dot);
        float xv;
        if constexpr (C::MOD == MOD_SOFTCAP) {
          xv = softcap_log2(a, dot);
        } else {
          xv = dot * a.scale_log2;
          if constexpr (C::MOD == MOD_ALIBI) xv -= alibi_l2 * __builtin_fabsf((float)(qi - key));
        }
        if (a.bias) {
          if (key < a.sk)
            xv += ((const float*)a.bias)[h * a.bias_sh + (int64_t)min(qi, a.sq - 1) * a.bias_si + key] *
                  kLog2e;
        }
        xv += kms[j];
        xv = (key >= lo && key <= hi) ? xv : kNegInf;
        x[j] = xv;
        xm = fmaxf(xm, xv);
      }
      const float m_new = fmaxf(m, xm);
      if (m_new == kNegInf) continue;  // nothing allowed for this row yet
      const float alpha = m == kNegInf ? 0.0f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < DV; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < BN; ++j) {
        const float p = fast_exp2(x[j] - m_new);
        l += p;
#pragma unroll
        for (int d = 0; d < DV; ++d) acc[d] = __builtin_fmaf(p, vs[j][d], acc[d]);
      }
      m = m_new;
    }

    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (a.lse[s] && valid)
      a.lse[s][b * a.lse_sb + h * a.lse_sh + qi] = l > 0.0f ? (m + __builtin_log2f(l)) * kLn2 : kNegInf;
    if (!valid) continue;
    if (s == 0) {
#pragma unroll
      for (int d = 0; d < DV; ++d) op[d] = acc[d] * inv;
    } else {
#pragma unroll
      for (int d = 0; d < DV; ++d) op[d] = op[d] - a.lambda * (acc[d] * inv);
    }
  }
  if (a.gate && valid) {
    const float* gp = (const float*)a.gate + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si;
#pragma unroll
    for (int d = 0; d < DV; ++d) op[d] = op[d] * sigmoid(gp[d]);
  }
}

}  // namespace fl
