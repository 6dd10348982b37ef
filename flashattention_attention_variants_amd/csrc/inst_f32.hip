// Template instances of the float32 attention kernel (matrix cores).
#include "attn_f32.hpp"
#include "fl_launch.hpp"

namespace fl {

template <class C>
static hipError_t go(const KernelArgs& a, hipStream_t st) {
  const int nwg = a.nb * a.nh * a.n_qt;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_f32_kernel<C>, dim3(nwg), dim3(C::NW * 64), 0, st, a);
  return hipGetLastError();
}

template <int DQK, int DV, int NS>
static hipError_t pick_mod(const KernelArgs& a, int mod, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return go<F32Cfg<DQK, DV, NS, MOD_ALIBI>>(a, st);
    case MOD_SOFTCAP: return go<F32Cfg<DQK, DV, NS, MOD_SOFTCAP>>(a, st);
    default: return go<F32Cfg<DQK, DV, NS, MOD_NONE>>(a, st);
  }
}

hipError_t launch_f32(const KernelArgs& a, int dqk, int dv, int ns, int mod, hipStream_t st) {
  if (ns == 2) {
    if (dqk == 64 && dv == 64) return go<F32Cfg<64, 64, 2, MOD_NONE>>(a, st);
    return go<F32Cfg<64, 128, 2, MOD_NONE>>(a, st);
  }
  if (dqk == 32 && dv == 32) return pick_mod<32, 32, 1>(a, mod, st);
  if (dqk == 128 && dv == 128) return pick_mod<128, 128, 1>(a, mod, st);
  return pick_mod<64, 64, 1>(a, mod, st);
}

}  // namespace fl
