// fl_common.hpp -- types, launch arguments and per-row key intervals shared
// by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Score modification applied to every score (FlexAttention's score_mod class).
// MOD_SOFTCAP_BOUNDED is softcap without a bias or key mask and with
// cap * log2(e) <= 100: every base-2 score lies in [-100, 100], so the
// exponentials need no running reference at all.
enum ModKind { MOD_NONE = 0, MOD_ALIBI = 1, MOD_SOFTCAP = 2, MOD_SOFTCAP_BOUNDED = 3 };

// Every mask variant on the pages allows, for query i, one contiguous run of
// keys [lo(i), hi(i)], and both ends never decrease as i grows.  That is
// what lets a tile's fate (all allowed / none allowed / mixed) follow from
// index arithmetic on its first and last query, with no mask tensor.
enum IntervalKind {
  IV_FULL = 0,              // vanilla, ALiBi, softcap: [0, S_k-1]
  IV_CAUSAL = 1,            // [0, i]
  IV_WINDOW_CAUSAL = 2,     // [i-W+1, i]
  IV_WINDOW_TWO_SIDED = 3,  // [i-W+1, i+W-1]
  IV_PREFIX = 4,            // [0, max(i, P-1)]
  IV_DOCUMENT = 5           // [start(doc(i)), end(doc(i))-1]
};

// Everything a launch needs.  Strides are in elements; the head dimension is
// always contiguous.  "b" is the batch index (the MSA row or column for the
// Evoformer), "h" the query head, "i"/"j" query/key positions.
struct KernelArgs {
  const void* q[2];
  const void* k[2];
  const void* v;
  const void* bias;        // [h][i][j], j contiguous
  const void* gate;        // same layout and strides as o
  const uint8_t* kmask;    // [b][j]
  void* o;
  float* lse[2];           // [b][h][i]
  int64_t q_sb, q_sh, q_si;
  int64_t k_sb, k_sh, k_si;  // head index is the K/V head
  int64_t v_sb, v_sh, v_si;
  int64_t o_sb, o_sh, o_si;
  int64_t lse_sb, lse_sh;
  int64_t bias_sh, bias_si;
  int64_t km_sb, km_sj;
  int nb, nh, group, sq, sk;  // group = H_q / H_kv
  int n_qt;                   // query tiles per (b, h)
  int iv_kind, window, prefix, n_docs;
  const int32_t* doc_offsets;  // [b][n_docs+1]
  float scale_log2;            // scale * log2(e)
  float softcap_arg;           // 2 * scale * log2(e) / cap
  float softcap_log2;          // cap * log2(e)
  float alibi_max_bias;
  float lambda;
  int heavy_first;             // schedule the most expensive query tiles first
  int doc_order;               // document mask: deal query tiles longest first
  int head_major;              // deal a head's query tiles to its XCD consecutively
  int alibi_nh;                // query heads in the ALiBi slope formula
  int rows_per_wg;             // gated launches: batch entries per work-group
  // Decode against a KV cache.  The rows of K/V head hk are the G*S_new
  // query rows of its G query heads, packed: row r is new token r % S_new of
  // query head hk*G + r / S_new (contiguous in [B, H_q, S_new, D]).  Batch
  // entry b's cache holds seqlens[b] tokens (clamped to [0, max_len]) and
  // the new tokens are its last S_new, so row r sits at position
  // len - S_new + r % S_new.  The key tiles a work-group's rows need are
  // cut into n_split near-equal ranges; with n_split > 1 each range writes
  // its normalised output and log-sum-exp to o_part / lse_part in float32
  // ([n_split][B*H_q*S_new][D] and [n_split][B*H_q*S_new]) for a merge.
  const int32_t* seqlens;
  int max_len, sq_new, grp;
  int n_split;
  float* o_part;
  float* lse_part;
};

// Tensors of the backward beyond the forward's arguments; all [B, H, S, D]
// with the strides of q (o, dout, dq) or of k (dk, dv).
struct BwdArgs {
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  // [B, H_q, S_q] each, written by the dQ launch and read by the dK, dV
  // launch: D, and the LSE in log2 units (+inf for a query with no key)
  float* delta;
  float* lse2;
};

// Document mask: the document holding row i (the largest d < n_docs with
// off[d] <= i, by binary search over the n_docs + 1 offsets of one batch
// entry) and its run of keys [off[d], off[d+1] - 1], unclamped.  `off`
// points at global memory or at an LDS copy.
template <class P>
__device__ __forceinline__ void doc_run(P off, int n_docs, int i, int& lo, int& hi) {
  int dlo = 0, dhi = n_docs - 1;
  while (dlo < dhi) {
    const int mid = (dlo + dhi + 1) >> 1;
    if (off[mid] <= i) dlo = mid; else dhi = mid - 1;
  }
  lo = off[dlo];
  hi = off[dlo + 1] - 1;
}

// Key interval [lo, hi] of query i, clamped to [0, S_k-1] (empty: lo > hi).
__device__ __forceinline__ void key_interval(const KernelArgs& a, int b, int i, int& lo,
                                             int& hi) {
  switch (a.iv_kind) {
    case IV_CAUSAL:
      lo = 0;
      hi = i;
      break;
    case IV_WINDOW_CAUSAL:
      lo = i - a.window + 1;
      hi = i;
      break;
    case IV_WINDOW_TWO_SIDED:
      lo = i - a.window + 1;
      hi = i + a.window - 1;
      break;
    case IV_PREFIX:
      lo = 0;
      hi = i > a.prefix - 1 ? i : a.prefix - 1;
      break;
    case IV_DOCUMENT:
      doc_run(a.doc_offsets + (int64_t)b * (a.n_docs + 1), a.n_docs, i, lo, hi);
      break;
    default:
      lo = 0;
      hi = a.sk - 1;
      break;
  }
  lo = lo < 0 ? 0 : lo;
  hi = hi > a.sk - 1 ? a.sk - 1 : hi;
}

// Queries that may see key j, [lo, hi] clamped to [0, S_q-1] (empty: lo > hi):
// every interval kind has both ends of [lo(i), hi(i)] non-decreasing in i,
// so {i : lo(i) <= j <= hi(i)} is one run of queries.
__device__ __forceinline__ void query_interval(const KernelArgs& a, int b, int j, int& lo,
                                               int& hi) {
  switch (a.iv_kind) {
    case IV_CAUSAL:
      lo = j;
      hi = a.sq - 1;
      break;
    case IV_WINDOW_CAUSAL:
      lo = j;
      hi = j + a.window - 1;
      break;
    case IV_WINDOW_TWO_SIDED:
      lo = j - a.window + 1;
      hi = j + a.window - 1;
      break;
    case IV_PREFIX:
      lo = j < a.prefix ? 0 : j;
      hi = a.sq - 1;
      break;
    case IV_DOCUMENT:
      doc_run(a.doc_offsets + (int64_t)b * (a.n_docs + 1), a.n_docs, j, lo, hi);
      break;
    default:
      lo = 0;
      hi = a.sq - 1;
      break;
  }
  lo = lo < 0 ? 0 : lo;
  hi = hi > a.sq - 1 ? a.sq - 1 : hi;
}

// Work-group id -> (b*H + h, query tile).  Work-groups are dealt to the 8
// XCDs round-robin by id, and each XCD has its own L2.  When the number of
// K/V heads (b, hk) is a multiple of 8, XCD x takes K/V heads x, x+8, x+16,
// ... with every query tile of every query head that reads them, so their
// K/V reads share one L2 and heads of different cost (ALiBi slopes, batch
// entries) spread over all XCDs.  Dense rows (equal work per tile) go out
// head-major within an XCD, so the work-groups resident at one time cover
// few heads and stream the same K/V tiles together.  Masked rows go out
// tile-index-major, which balances unequal tiles better; with heavy_first
// the most expensive tiles of every head start first and the grid's tail is
// made of cheap ones.
__device__ __forceinline__ void decode_tile(const KernelArgs& a, int bid, int& bh, int& qt) {
  const int nbh = a.nb * a.nh;
  const int G = a.group, nkv = nbh / G;
  int order;
  if ((nkv & 7) == 0) {
    const int kpx = nkv >> 3;  // K/V heads per XCD
    const int xcd = bid & 7, slot = bid >> 3;
    int kv_local, r;
    if (a.head_major) {
      kv_local = slot / (G * a.n_qt);
      const int rem = slot % (G * a.n_qt);
      r = rem / a.n_qt;
      order = rem % a.n_qt;
    } else {
      order = slot / (kpx * G);
      const int hi = slot % (kpx * G);
      kv_local = hi / G;
      r = hi % G;
    }
    bh = (kv_local * 8 + xcd) * G + r;
  } else {
    bh = bid % nbh;
    order = bid / nbh;
  }
  qt = a.heavy_first ? a.n_qt - 1 - order : order;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(x) = 1 / (1 + e^-x)
__device__ __forceinline__ float sigmoid(float x) {
  return fast_rcp(1.0f + fast_exp2(-x * kLog2e));
}

// ALiBi slope of query head h: 2^(-max_bias * (h+1) / H), in log2 units of
// the exponent (times log2 e) so it can be applied to base-2 scores.
__device__ __forceinline__ float alibi_slope_log2(const KernelArgs& a, int h) {
  return fast_exp2(-a.alibi_max_bias * (float)(h + 1) / (float)a.alibi_nh) * kLog2e;
}

// cap * tanh(y) in log2 units, from t = 2*y*log2(e):
// tanh(y) = 1 - 2 / (e^(2y) + 1).
__device__ __forceinline__ float softcap_log2(const KernelArgs& a, float raw) {
  const float e = fast_exp2(raw * a.softcap_arg);
  return a.softcap_log2 - 2.0f * a.softcap_log2 * fast_rcp(e + 1.0f);
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16*l (lds is wave-uniform).  Issued from assembly: the compiler's
// wait-count pass cannot tell which LDS bytes such a load writes, and would
// make every later LDS read wait for all tiles still in flight (the next
// tiles' loads included), which serialises the tile pipeline.  The pipeline
// waits for these loads itself (s_waitcnt vmcnt before the barrier that
// publishes a tile).  The load writes no register; M0, which carries the LDS
// address, is restored before the statement ends.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, void* lds, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(byte_off), "s"(rs));
#else
  (void)rs;
  (void)lds;
  (void)byte_off;
#endif
}

// 4 bytes per lane, the same way: lane l's dword lands at lds + 4*l, and a
// lane whose offset lies past the resource's end writes 0.
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, void* lds, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(byte_off), "s"(rs));
#else
  (void)rs;
  (void)lds;
  (void)byte_off;
#endif
}

// Buffer resource over [base, base + bytes); 0x00020000 is the raw 32-bit
// data-format word of gfx9 buffer descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

}  // namespace fl
