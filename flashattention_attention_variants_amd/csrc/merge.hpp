// merge.hpp -- merge of partial attention results over disjoint key ranges.
//
// Part p of a row carries O_p, normalised over its own keys, and its
// log-sum-exp LSE_p.  The row over all keys is
//
//   LSE = ln sum_p e^(LSE_p),   O = sum_p e^(LSE_p - LSE) O_p
//
// the rescaling identity that lets the single-pass softmax visit keys in
// pieces (gist.science explainer of Flashlight, "Technical Summary:
// Methodology", semantic fusion), applied to whole key ranges.  Parts with
// LSE = -inf held no key and weigh nothing; a row whose parts are all empty
// gets O = 0 and LSE = -inf.
//
// One wave per row: the lanes reduce the parts' maximum and sum, then each
// lane owns head-dimension columns lane, lane + 64, ...  The traffic is the
// parts' outputs read once and the row written once; the kernel is bound by
// HBM bandwidth and is small next to the attention that produced the parts.
#pragma once

#include "fl_common.hpp"

namespace fl {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int n_parts,
                                                    int64_t n_rows, int D, OutT* __restrict__ o,
                                                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  float m = kNegInf;
  for (int p = lane; p < n_parts; p += 64) m = fmaxf(m, lse_part[(int64_t)p * n_rows + row]);
  m = wave_max(m);
  OutT* out = o + row * D;
  if (m == kNegInf) {
    for (int d = lane; d < D; d += 64) out[d] = (OutT)0.0f;
    if (lse && lane == 0) lse[row] = kNegInf;
    return;
  }
  float l = 0.0f;
  for (int p = lane; p < n_parts; p += 64)
    l += fast_exp2((lse_part[(int64_t)p * n_rows + row] - m) * kLog2e);
  l = wave_sum(l);
  const float whole = m + __builtin_log2f(l) * kLn2;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.0f;
    for (int p = 0; p < n_parts; ++p) {
      const float w = fast_exp2((lse_part[(int64_t)p * n_rows + row] - whole) * kLog2e);
      acc = fmaf(w, o_part[((int64_t)p * n_rows + row) * D + d], acc);
    }
    out[d] = (OutT)acc;
  }
  if (lse && lane == 0) lse[row] = whole;
}

}  // namespace fl
