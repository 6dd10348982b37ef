// Template instances of the bf16 matrix-core kernel for Evoformer gated
// attention: C = 32, optional pair bias, per-key mask, sigmoid gate.
#include "attn_mfma.hpp"
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

}  // namespace fl
