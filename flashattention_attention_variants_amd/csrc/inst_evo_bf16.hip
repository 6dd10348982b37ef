// Template instances of the bf16 matrix-core kernel for Evoformer gated
// attention: C = 32, optional pair bias, per-key mask, sigmoid gate.
#include "attn_mfma.hpp"
#include "evo.hpp"
#include "fl_launch.hpp"

namespace fl {

template <class C>
static hipError_t go(const KernelArgs& a, hipStream_t st) {
  // each work-group walks rows_per_wg batch entries of one head and query tile
  const int groups = (a.nb + a.rows_per_wg - 1) / a.rows_per_wg;
  const int nwg = groups * a.nh * a.n_qt;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_mfma_kernel<C>, dim3(nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_evo_bf16(const KernelArgs& a, int c, int qb, bool bias, hipStream_t st) {
  (void)c;  // C = 32 only
  if (qb == 1) {
    if (bias) return go<MfmaCfg<32, 32, 1, 1, MOD_NONE, true, true, true>>(a, st);
    return go<MfmaCfg<32, 32, 1, 1, MOD_NONE, false, true, true>>(a, st);
  }
  if (bias) return go<MfmaCfg<32, 32, 1, 2, MOD_NONE, true, true, true>>(a, st);
  return go<MfmaCfg<32, 32, 1, 2, MOD_NONE, false, true, true>>(a, st);
}

// Short rows: one work-group per (entry, head) at a time, walking
// rows_per_wg entries of one head.  Work-groups per compute unit: 8 waves
// (two per SIMD; with a bias) or 12 (three per SIMD; without) over NKU
// waves each, which the LDS stages also allow.
// The grid aims at filling every compute unit once (head pairs to XCDs:
// see the kernel's work-group decode).
#ifndef FL_EVO_SHORT_FILL
#define FL_EVO_SHORT_FILL 1
#endif
template <int NKU, bool BIAS>
static hipError_t go_short(KernelArgs& a, hipStream_t st) {
  using K = EvoCfg<NKU, BIAS>;
  const int per_cu = (BIAS ? 8 : 12) / NKU;
  const int target = 256 * per_cu * FL_EVO_SHORT_FILL;
  const int per_head = max(1, target / a.nh);
  a.rows_per_wg = (a.nb + per_head - 1) / per_head;
  const int64_t groups = (a.nb + a.rows_per_wg - 1) / a.rows_per_wg;
  // two work-groups (the heads of a pair) per unit, units dealt 8 at a time
  const int64_t units = groups * ((a.nh + 1) / 2);
  const int64_t nwg = 16 * ((units + 7) / 8);
  (void)hipGetLastError();
  hipLaunchKernelGGL(evo_kernel<K>, dim3((unsigned)nwg), dim3(K::NW * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_evo_short_bf16(KernelArgs& a, hipStream_t st) {
  const int L = a.sq;
  const bool bias = a.bias != nullptr;
  if (L <= 64) return bias ? go_short<2, true>(a, st) : go_short<2, false>(a, st);
  if (L <= 128) return bias ? go_short<4, true>(a, st) : go_short<4, false>(a, st);
  if (L <= 256) return bias ? go_short<8, true>(a, st) : go_short<8, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace fl
