// Template instances of the bf16 matrix-core kernel with two softmax streams
// (differential attention).
#include "attn_mfma.hpp"
#include "fl_launch.hpp"

namespace fl {

template <class C>
static hipError_t go(const KernelArgs& a, hipStream_t st) {
  const int nwg = a.nb * a.nh * a.n_qt;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_mfma_kernel<C>, dim3(nwg), dim3(C::NW * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_diff_bf16(const KernelArgs& a, int dqk, int dv, hipStream_t st) {
  if (dqk == 64 && dv == 64) return go<MfmaCfg<64, 64, 2, 1, MOD_NONE, false, false, false>>(a, st);
  return go<MfmaCfg<64, 128, 2, 1, MOD_NONE, false, false, false>>(a, st);
}

}  // namespace fl
