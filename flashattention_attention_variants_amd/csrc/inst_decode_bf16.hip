// Template instances of the bf16 matrix-core kernel in its decode form, D = 64.
#include "attn_mfma.hpp"
#include "fl_launch.hpp"

namespace fl {

template <int MOD>
static hipError_t go_dec(const KernelArgs& a, hipStream_t st) {
  using C = MfmaCfg<64, 64, 1, 1, MOD, false, false, false, true>;
  const int64_t nwg = (int64_t)a.nb * a.nh * a.n_qt * a.n_split;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_mfma_kernel<C>, dim3((unsigned)nwg), dim3(C::NW * 64), 0, st, a);
  return hipGetLastError();
}

int decode_rows_per_wg() { return MfmaCfg<64, 64, 1, 1, MOD_NONE, false, false, false, true>::BM; }

hipError_t launch_decode_bf16(const KernelArgs& a, int mod, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return go_dec<MOD_ALIBI>(a, st);
    case MOD_SOFTCAP: return go_dec<MOD_SOFTCAP>(a, st);
    case MOD_SOFTCAP_BOUNDED: return go_dec<MOD_SOFTCAP_BOUNDED>(a, st);
    default: return go_dec<MOD_NONE>(a, st);
  }
}

}  // namespace fl
