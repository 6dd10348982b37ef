// fl_launch.hpp -- host-side launchers of the kernel families, one per
// translation unit so the template instances compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "fl_common.hpp"
#include "flattn.h"

namespace fl {

// bf16 attention, D = 64: qb = 32-query blocks per wave (1 or 2), mod =
// ModKind, bias = additive [H_q, S_q, S_k] bias present.
hipError_t launch_attn_bf16(const KernelArgs& a, int qb, int mod, bool bias, hipStream_t st);

// bf16 differential attention: (dqk, dv) = (64, 128) or (64, 64).
hipError_t launch_diff_bf16(const KernelArgs& a, int dqk, int dv, hipStream_t st);

// bf16 Evoformer gated attention, C = 32: qb = 1 or 2, bias = pair bias.
hipError_t launch_evo_bf16(const KernelArgs& a, int c, int qb, bool bias, hipStream_t st);

// bf16 Evoformer gated attention with a pair bias, C = 32, rows of at most
// 256 positions (evo.hpp): a.sq = a.sk = L; sets a.rows_per_wg, the
// entries each work-group walks.
hipError_t launch_evo_short_bf16(KernelArgs& a, hipStream_t st);
constexpr int kEvoShortMax = 256;  // longest row of the short-row kernel

// bf16 decode against a KV cache, D = 64 (KernelArgs' decode fields set):
// grid = B * H_kv * n_qt * n_split work-groups.
hipError_t launch_decode_bf16(const KernelArgs& a, int mod, hipStream_t st);
int decode_rows_per_wg();  // packed query rows per decode work-group

// Merge of n_parts partial results per row (merge.hpp) into o (bf16 or
// float32) and lse (may be NULL).
hipError_t launch_merge(const float* o_part, const float* lse_part, int n_parts, int64_t n_rows,
                        int D, void* o, bool out_bf16, float* lse, hipStream_t st);

// bf16 attention backward, D = 64 (attn_bwd.hpp): the dQ launch, then the
// dK, dV launch.
hipError_t launch_bwd_bf16(const KernelArgs& a, const BwdArgs& g, int mod, hipStream_t st);

// Invariant Point Attention core (ipa.hpp), C = 16, 4 query/key points,
// 8 value points; cz = pair channels (0: no pair output, 64 or 128).
struct IpaArgs;
hipError_t launch_ipa_bf16(const IpaArgs& a, int cz, hipStream_t st);

// float32 path: (dqk, dv, ns, mod) as built in inst_f32.hip.
hipError_t launch_f32(const KernelArgs& a, int dqk, int dv, int ns, int mod, hipStream_t st);

// Decode against a KV cache with the workspace from a supplier: once the
// call is validated, get_ws(bytes, ctx, &ptr) provides `bytes` of device
// memory (0 when the call uses one key range) or returns the error status.
typedef fl_status (*DecodeWorkspaceFn)(int64_t bytes, void* ctx, void** ws);
fl_status decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cache_seqlens, void* o, float* lse, DecodeWorkspaceFn get_ws,
                     void* ws_ctx, int B, int H_q, int H_kv, int S_q, int S_cap, int max_seqlen,
                     int D, fl_kv_layout layout, fl_dtype dtype, const fl_attn_params* p,
                     int num_splits, void* stream);

// Query rows per work-group of each family.
constexpr int mfma_rows_per_wg(int qb) { return 4 * 32 * qb; }
#ifndef FL_FWD_WAVES
#define FL_FWD_WAVES 4
#endif
// fl_attn_fwd's work-groups: FL_FWD_WAVES waves of 32 qb rows each
constexpr int attn_rows_per_wg(int qb) { return FL_FWD_WAVES * 32 * qb; }
constexpr int f32_rows_per_wg() { return 64; }

}  // namespace fl
