// Template instances of the bf16 attention backward, D = 64.
#include "attn_bwd.hpp"
#include "fl_launch.hpp"

namespace fl {

template <int ROLE, int MOD>
static hipError_t go_bwd(const KernelArgs& a, const BwdArgs& g, hipStream_t st) {
  using C = BwdCfg<ROLE, MOD>;
  const int n_rows = ROLE == BWD_DQ ? a.sq : a.sk;
  const int nh = ROLE == BWD_DQ ? a.nh : a.nh / a.group;
  const int64_t nwg = (int64_t)a.nb * nh * ((n_rows + C::BM - 1) / C::BM);
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_bwd_kernel<C>, dim3((unsigned)nwg), dim3(C::NW * 64), 0, st, a, g);
  return hipGetLastError();
}

template <int MOD>
static hipError_t both(const KernelArgs& a, const BwdArgs& g, hipStream_t st) {
  // dQ first: it also writes the row statistic D that dK, dV read.  With no
  // query (or no batch) only dK, dV remain, and the second launch, seeing
  // no query tile, writes them as zeros.
  hipError_t e = hipSuccess;
  if ((int64_t)a.nb * a.sq > 0) e = go_bwd<BWD_DQ, MOD>(a, g, st);
  if (e != hipSuccess || (int64_t)a.nb * a.sk == 0) return e;
  return go_bwd<BWD_DKDV, MOD>(a, g, st);
}

hipError_t launch_bwd_bf16(const KernelArgs& a, const BwdArgs& g, int mod, hipStream_t st) {
  switch (mod) {
    case MOD_ALIBI: return both<MOD_ALIBI>(a, g, st);
    case MOD_SOFTCAP: return both<MOD_SOFTCAP>(a, g, st);
    default: return both<MOD_NONE>(a, g, st);
  }
}

}  // namespace fl
