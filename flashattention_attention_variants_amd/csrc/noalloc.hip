// noalloc.hip -- fl_attn_decode_fwd_noalloc: split-key decode whose float32
// partial results live in the library's own static device buffer instead of
// a caller workspace, for callers that cannot allocate device memory (code
// under graph capture, tight serving loops).
#include <stdint.h>

#include <mutex>

#include "fl_launch.hpp"
#include "flattn.h"

namespace {

// The scratch buffer: FL_DECODE_SCRATCH_BYTES of device memory that every
// GPU the library runs on holds until the process ends.  In host code its
// name is only a stand-in: host code uses the device address found below.
static __device__ __align__(256) unsigned char scratch[FL_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU

// Workspace supplier of the no-allocation decode: rejects a call that needs
// more than the buffer holds before touching the runtime; on the first call
// on a device that needs it, looks the buffer's address up with that device
// current and keeps it.
fl_status scratch_workspace(int64_t need, void* ctx, void** ws) {
  (void)ctx;
  *ws = nullptr;
  if (need > (int64_t)FL_DECODE_SCRATCH_BYTES) return FL_ERR_SCRATCH;
  if (need == 0) return FL_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FL_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FL_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *ws = g_scratch[dev];
  return FL_OK;
}

}  // namespace

extern "C" fl_status fl_attn_decode_fwd_noalloc(const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* cache_seqlens,
                                                void* o, float* lse, int B, int H_q, int H_kv,
                                                int S_q, int S_cap, int max_seqlen, int D,
                                                fl_kv_layout layout, fl_dtype dtype,
                                                const fl_attn_params* p, int num_splits,
                                                void* stream) {
  return fl::decode_fwd(q, k_cache, v_cache, cache_seqlens, o, lse, scratch_workspace, nullptr, B,
                        H_q, H_kv, S_q, S_cap, max_seqlen, D, layout, dtype, p, num_splits, stream);
}
