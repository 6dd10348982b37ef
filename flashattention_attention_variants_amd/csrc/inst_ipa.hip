// Template instances of the Invariant Point Attention core: C = 16 scalar
// channels, 4 query/key points and 8 value points per head (AlphaFold2's
// structure module), pair representation of 64 or 128 channels or none.
#include "fl_launch.hpp"
#include "ipa.hpp"

namespace fl {

template <int CZ>
static hipError_t go_ipa(const IpaArgs& a, hipStream_t st) {
  using K = IpaCfg<16, 4, 8, CZ>;
  const int64_t nwg = (int64_t)a.B * a.L * ((a.H + K::HW - 1) / K::HW);
  (void)hipGetLastError();
  hipLaunchKernelGGL(ipa_kernel<K>, dim3((unsigned)nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ipa_bf16(const IpaArgs& a, int cz, hipStream_t st) {
  switch (cz) {
    case 0: return go_ipa<0>(a, st);
    case 64: return go_ipa<64>(a, st);
    case 128: return go_ipa<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fl
