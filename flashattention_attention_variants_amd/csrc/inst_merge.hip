// Launcher of the (O, LSE) merge kernel.
#include "fl_launch.hpp"
#include "merge.hpp"

namespace fl {

hipError_t launch_merge(const float* o_part, const float* lse_part, int n_parts, int64_t n_rows,
                        int D, void* o, bool out_bf16, float* lse, hipStream_t st) {
  const int64_t nwg = (n_rows + 3) / 4;
  (void)hipGetLastError();
  if (out_bf16)
    hipLaunchKernelGGL(merge_kernel<bf16>, dim3((unsigned)nwg), dim3(256), 0, st, o_part, lse_part,
                       n_parts, n_rows, D, (bf16*)o, lse);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)nwg), dim3(256), 0, st, o_part,
                       lse_part, n_parts, n_rows, D, (float*)o, lse);
  return hipGetLastError();
}

}  // namespace fl
