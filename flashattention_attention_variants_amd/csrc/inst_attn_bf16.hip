// Template instances of the bf16 matrix-core attention kernel, D = 64.
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

template <int QB, int MOD>
static hipError_t pick_bias(const KernelArgs& a, bool bias, hipStream_t st) {
  if (bias) return go<MfmaCfg<64, 64, 1, QB, MOD, true, false, false>>(a, st);
  return go<MfmaCfg<64, 64, 1, QB, MOD, false, false, false>>(a, st);
}

template <int QB>
static hipError_t pick_mod(const KernelArgs& a, int mod, bool bias, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI:
      // ALiBi with a bias takes one query block per wave (its two-block
      // form would spill); that instance is not built
      if (QB == 2 && bias) return hipErrorInvalidConfiguration;
      if constexpr (QB == 1) return pick_bias<QB, MOD_ALIBI>(a, bias, st);
      return go<MfmaCfg<64, 64, 1, QB, MOD_ALIBI, false, false, false>>(a, st);
    case MOD_SOFTCAP: return pick_bias<QB, MOD_SOFTCAP>(a, bias, st);
    case MOD_SOFTCAP_BOUNDED:  // chosen only without a bias
      return go<MfmaCfg<64, 64, 1, QB, MOD_SOFTCAP_BOUNDED, false, false, false>>(a, st);
    default: return pick_bias<QB, MOD_NONE>(a, bias, st);
  }
}

hipError_t launch_attn_bf16(const KernelArgs& a, int qb, int mod, bool bias, hipStream_t st) {
  if (qb == 1) return pick_mod<1>(a, mod, bias, st);
  return pick_mod<2>(a, mod, bias, st);
}

}  // namespace fl
