// attn_f32.hpp -- float32 fused attention forward on the matrix cores (gfx950).
//
// The float32 dtype exists for accuracy; its products run on the float32
// matrix instruction v_mfma_f32_32x32x2_f32 (exact float32 products, float32
// accumulation), the same single-pass online softmax as the bf16 kernel in
// float32 throughout (gist.science explainer of Flashlight, "Technical
// Summary: Methodology", semantic fusion).  Two waves per work-group, 32
// query rows each; K and V tiles of 32 keys staged in LDS.
//
// Per tile a wave computes S^T = K Q^T (rows = keys in the accumulator
// registers, columns = its queries in the lanes) in DQK / 2 steps of k = 2.
// Any pairing of head-dimension entries between the two operands gives the
// same sum, so lane (c, g) takes dims g DQK/2 + t at step t: its Q operand
// is one contiguous half of its query row (registers) and its K operand one
// contiguous half of key c's row (16-byte LDS reads).  Then O^T += V^T P^T
// in 16 steps per 32 keys: step t pairs keys 8(t/4) + 4g + t%4, exactly the
// keys of accumulator register t in lane half g, so each lane's B operand is
// its own register t and no value crosses lanes.
//
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
  static constexpr int NW = 2;        // waves per work-group
  static constexpr int BM = 32 * NW;  // query rows per work-group
  static constexpr int BN = 32;       // keys per tile
  // LDS row strides in floats: K rows shifted by 4 banks each (16 rows of
  // one 16-byte read hit distinct banks), V rows by 8 (the two key rows of
  // one read step, 4 apart, fall in opposite bank halves)
  static constexpr int KS = DQK + 4, VS = DV + 8;
  static_assert(DQK % 8 == 0 && DV % 32 == 0, "head dims");
};

template <class C>
__global__ __launch_bounds__(C::NW * 64) void attn_f32_kernel(KernelArgs a) {
  constexpr int BN = C::BN, DQK = C::DQK, DV = C::DV, KS = C::KS, VS = C::VS;
  constexpr int NT = C::NW * 64;
  constexpr int HQ = DQK / 2;  // S^T steps; also this lane's share of a query row
  __shared__ __attribute__((aligned(16))) float ks[BN * KS];
  __shared__ __attribute__((aligned(16))) float vs[BN * VS];
  __shared__ float kms[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  int bh, qt;
  decode_tile(a, blockIdx.x, bh, qt);
  const int b = bh / a.nh, h = bh % a.nh, hk = h / a.group;
  const int q0 = qt * C::BM;
  const int qi = q0 + 32 * w + c;  // this lane's query (the column it holds)
  const bool valid = qi < a.sq;
  const int qr = min(qi, a.sq - 1);
  const int qlast = min(q0 + C::BM, a.sq) - 1;

  int lo_first, hi_first, lo_last, hi_last, lo, hi;
  key_interval(a, b, q0, lo_first, hi_first);
  key_interval(a, b, qlast, lo_last, hi_last);
  key_interval(a, b, qr, lo, hi);
  const int kt_lo = lo_first / BN;
  const int kt_hi = hi_last >= lo_first ? (hi_last + BN) / BN : kt_lo;
  const float alibi_l2 = C::MOD == MOD_ALIBI ? alibi_slope_log2(a, h) : 0.0f;

  float* op = (float*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qr * a.o_si;

  for (int s = 0; s < C::NS; ++s) {
    // B operand of S^T: dims g HQ .. g HQ + HQ - 1 of this lane's query
    float q[HQ];
    {
      const float* qp = (const float*)a.q[s] + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_si + g * HQ;
#pragma unroll
      for (int t = 0; t < HQ; t += 4) {
        const f32x4 v4 = *(const f32x4*)(qp + t);
#pragma unroll
        for (int e = 0; e < 4; ++e) q[t + e] = v4[e];
      }
    }
    const float* kb = (const float*)a.k[s] + b * a.k_sb + hk * a.k_sh;
    const float* vb = (const float*)a.v + b * a.v_sb + hk * a.v_sh;

    f32x16 acc[DV / 32];  // O^T: lane (c, g) holds dims 32db + 8(r/4) + 4g + r%4 of query c
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) acc[db] = f32x16{};
    float m = kNegInf, l = 0.0f;

    for (int kt = kt_lo; kt < kt_hi; ++kt) {
      const int j0 = kt * BN;
      __syncthreads();
      // stage the tile: rows past S_k read as zeros
      for (int e = tid; e < BN * DQK / 4; e += NT) {
        const int j = e / (DQK / 4), d4 = e % (DQK / 4);
        f32x4 v4 = {};
        if (j0 + j < a.sk) v4 = *(const f32x4*)(kb + (int64_t)(j0 + j) * a.k_si + 4 * d4);
        *(f32x4*)(ks + j * KS + 4 * d4) = v4;
      }
      for (int e = tid; e < BN * DV / 4; e += NT) {
        const int j = e / (DV / 4), d4 = e % (DV / 4);
        f32x4 v4 = {};
        if (j0 + j < a.sk) v4 = *(const f32x4*)(vb + (int64_t)(j0 + j) * a.v_si + 4 * d4);
        *(f32x4*)(vs + j * VS + 4 * d4) = v4;
      }
      if (tid < BN) {
        const int j = j0 + tid;
        kms[tid] = (j < a.sk && (!a.kmask || a.kmask[b * a.km_sb + (int64_t)j * a.km_sj] != 0))
                       ? 0.0f
                       : kNegInf;
      }
      __syncthreads();

      // S^T for the tile: A = K (row c, dims g HQ + t), B = Q
      f32x16 sc = {};
#pragma unroll
      for (int t = 0; t < HQ; t += 4) {
        const f32x4 k4 = *(const f32x4*)(ks + c * KS + g * HQ + t);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc = __builtin_amdgcn_mfma_f32_32x32x2f32(k4[e], q[t + e], sc, 0, 0, 0);
      }

      // scores of this lane's query against keys j0 + 8(r/4) + 4g + r%4, base 2
      float xm = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jj = 8 * (r >> 2) + 4 * g + (r & 3);
        const int key = j0 + jj;
        float xv;
        if constexpr (C::MOD == MOD_SOFTCAP) {
          xv = softcap_log2(a, sc[r]);
        } else {
          xv = sc[r] * a.scale_log2;
          if constexpr (C::MOD == MOD_ALIBI) xv -= alibi_l2 * __builtin_fabsf((float)(qi - key));
        }
        if (a.bias) {
          if (key < a.sk)
            xv += ((const float*)a.bias)[h * a.bias_sh + (int64_t)qr * a.bias_si + key] * kLog2e;
        }
        xv += kms[jj];
        xv = (key >= lo && key <= hi) ? xv : kNegInf;
        sc[r] = xv;
        xm = fmaxf(xm, xv);
      }
      xm = fmaxf(xm, __shfl_xor(xm, 32));  // both halves of the query's keys
      const float m_new = fmaxf(m, xm);
      // a query with nothing allowed yet keeps m = -inf and adds nothing
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = m == kNegInf ? 0.0f : fast_exp2(m - m_use);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) acc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = fast_exp2(sc[r] - m_use);
        l += sc[r];
      }
      m = m_new;

      // O^T += V^T P^T: step t takes keys 8(t/4) + 4g + t%4 (register t)
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int jj = 8 * (t >> 2) + 4 * g + (t & 3);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[jj * VS + 32 * db + c], sc[t], acc[db], 0, 0, 0);
        }
    }

    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (a.lse[s] && valid && g == 0)
      a.lse[s][b * a.lse_sb + h * a.lse_sh + qi] = lt > 0.0f ? (m + __builtin_log2f(lt)) * kLn2 : kNegInf;
    if (!valid) continue;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float* p4 = op + 32 * db + 8 * r4 + 4 * g;
        f32x4 v4 = {acc[db][4 * r4] * inv, acc[db][4 * r4 + 1] * inv, acc[db][4 * r4 + 2] * inv,
                    acc[db][4 * r4 + 3] * inv};
        if (s == 1) v4 = *(const f32x4*)p4 - a.lambda * v4;
        *(f32x4*)p4 = v4;
      }
  }
  if (a.gate && valid) {
    const float* gp = (const float*)a.gate + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * g;
        const f32x4 g4 = *(const f32x4*)(gp + d);
        f32x4 v4 = *(const f32x4*)(op + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] *= sigmoid(g4[e]);
        *(f32x4*)(op + d) = v4;
      }
  }
}

}  // namespace fl
