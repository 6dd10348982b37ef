// fl_api.hip -- the C ABI: argument validation on the host, then one kernel
// launch on the caller's stream.  No allocation, no synchronisation.
#include <math.h>
#include <stdint.h>

#include "flattn.h"
#include "fl_launch.hpp"
#include "ipa.hpp"

using namespace fl;

namespace {

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }

constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;
constexpr int kMaxSeq = 1 << 30;

fl_status launch_status(hipError_t e) { return e == hipSuccess ? FL_OK : FL_ERR_LAUNCH; }

void init_args(KernelArgs& a) {
  a = KernelArgs{};
  a.scale_log2 = 0.0f;
  a.lambda = 0.0f;
  a.iv_kind = IV_FULL;
}

// Contiguous [B, H, S, D] strides.
void bhsd(int64_t H, int64_t S, int64_t D, int64_t& sb, int64_t& sh, int64_t& si) {
  si = D;
  sh = S * D;
  sb = H * S * D;
}

int grid_qtiles(int S_q, int rows_per_wg) { return (S_q + rows_per_wg - 1) / rows_per_wg; }

// The matrix-core kernels address one (batch, K/V head) block of K and of V
// through 32-bit byte offsets.
// Byte offsets within one (batch, head) block of bf16 rows stay below 2^31
// (32-bit buffer offsets), for the rows given and for the 64 rows past them
// that a partial key tile addresses (and reads as zeros).
bool span_ok(int64_t rows, int64_t row_stride, int64_t width) {
  return rows <= 0 || ((rows + 63) * row_stride + width) * 2 < ((int64_t)1 << 31);
}

// Decode: key ranges per (sequence, K/V head).  Enough work-groups to give
// every compute unit sixteen (256 units; measured 3-4% faster than eight on
// mixed cache lengths, where short and long ranges then even out), but no
// range shorter than sixteen 64-key tiles: a work-group pays a fixed
// start-up (the length, the Q rows, the first tiles in flight) that short
// ranges do not amortise.  A request is capped at the number of tiles.
constexpr int kDecodeTargetWgs = 4096;
constexpr int kDecodeMinTiles = 16;
constexpr int kDecodeMaxSplits = 256;

bool decode_sizes_ok(int B, int H_q, int H_kv, int S_q, int max_seqlen) {
  return B >= 0 && H_q >= 1 && H_kv >= 1 && H_q % H_kv == 0 && S_q >= 0 && max_seqlen >= 0 &&
         S_q <= kMaxSeq && max_seqlen <= kMaxSeq && (int64_t)(H_q / H_kv) * S_q <= kMaxSeq;
}

// keys one row block of a decode call may need: a sliding window bounds
// them whatever the cache length
int64_t decode_span(int S_q, int max_seqlen, const fl_attn_params* p) {
  int64_t span = max_seqlen;
  if (p) {
    const int mask = p->variant >= FL_CAUSAL ? p->variant : p->mask;
    if (mask == FL_SLIDING_WINDOW && p->window >= 1) {
      const int64_t w = p->window_causal ? (int64_t)p->window + S_q - 1
                                         : 2 * (int64_t)p->window + S_q - 2;
      span = w < span ? w : span;
    }
  }
  return span;
}

int decode_split(int B, int H_q, int H_kv, int S_q, int max_seqlen, const fl_attn_params* p,
                 int requested) {
  const int64_t span = decode_span(S_q, max_seqlen, p);
  const int n_tiles = span > 0 ? (int)((span + 63) / 64) : 1;
  const int64_t n_qt = grid_qtiles((H_q / H_kv) * S_q, decode_rows_per_wg());
  int s;
  if (requested > 0) {
    s = requested < n_tiles ? requested : n_tiles;
  } else {
    const int64_t base = (int64_t)B * H_kv * n_qt > 0 ? (int64_t)B * H_kv * n_qt : 1;
    const int64_t want = (kDecodeTargetWgs + base - 1) / base;
    const int64_t cap = n_tiles / kDecodeMinTiles > 1 ? n_tiles / kDecodeMinTiles : 1;
    s = (int)(want < cap ? want : cap);
    s = s < 1 ? 1 : (s > kDecodeMaxSplits ? kDecodeMaxSplits : s);
  }
  return s;
}

int64_t decode_workspace(int B, int H_q, int S_q, int D, int n_split) {
  if (n_split <= 1) return 0;
  const int64_t rows = (int64_t)B * H_q * S_q;
  const int64_t o_bytes = (int64_t)n_split * rows * D * 4;
  return o_bytes + ((int64_t)n_split * rows * 4 + 15) / 16 * 16;
}

// Validation of fl_attn_params shared by the forward and the backward.
fl_status check_params(const fl_attn_params* p, int S_q, int S_k) {
  if (p->variant < FL_VANILLA || p->variant > FL_DOCUMENT) return FL_ERR_PARAM;
  if (!isfinite(p->scale)) return FL_ERR_PARAM;
  // the mask in force: the variant's own, or one composed with a score
  // modification (vanilla, ALiBi, softcap)
  const bool variant_is_mask = p->variant >= FL_CAUSAL;
  if (p->mask != FL_VANILLA && (variant_is_mask || p->mask < FL_CAUSAL || p->mask > FL_DOCUMENT))
    return FL_ERR_PARAM;
  const int mask = variant_is_mask ? p->variant : p->mask;
  if (mask != FL_VANILLA && S_q != S_k) return FL_ERR_SHAPE;
  if (p->variant == FL_SOFTCAP && !(p->softcap > 0.0f && isfinite(p->softcap))) return FL_ERR_PARAM;
  if (p->variant == FL_ALIBI && !(p->alibi_max_bias >= 0.0f && isfinite(p->alibi_max_bias)))
    return FL_ERR_PARAM;
  if (mask == FL_SLIDING_WINDOW && p->window < 1) return FL_ERR_PARAM;
  if (mask == FL_PREFIX_LM && p->prefix < 0) return FL_ERR_PARAM;
  if (mask == FL_DOCUMENT) {
    if (p->n_docs < 1) return FL_ERR_PARAM;
    if (!p->doc_offsets) return FL_ERR_NULL;
  }
  return FL_OK;
}

// Score modification (returned) and key intervals of a variant.
int variant_args(const fl_attn_params* p, int S_k, KernelArgs& a) {
  int mod = MOD_NONE;
  const int mask = p->variant >= FL_CAUSAL ? p->variant : p->mask;
  if (p->variant == FL_ALIBI) {
    mod = MOD_ALIBI;
    a.alibi_max_bias = p->alibi_max_bias;
  } else if (p->variant == FL_SOFTCAP) {
    mod = MOD_SOFTCAP;
    a.softcap_arg = 2.0f * p->scale * kLog2e / p->softcap;
    a.softcap_log2 = p->softcap * kLog2e;
  }
  switch (mask) {
    case FL_CAUSAL:
      a.iv_kind = IV_CAUSAL;
      a.heavy_first = 1;
      break;
    case FL_SLIDING_WINDOW:
      a.iv_kind = p->window_causal ? IV_WINDOW_CAUSAL : IV_WINDOW_TWO_SIDED;
      a.window = p->window > S_k + 1 ? S_k + 1 : p->window;  // wider windows change nothing
      break;
    case FL_PREFIX_LM:
      a.iv_kind = IV_PREFIX;
      a.prefix = p->prefix > S_k ? S_k : p->prefix;
      a.heavy_first = 1;
      break;
    case FL_DOCUMENT:
      a.iv_kind = IV_DOCUMENT;
      a.n_docs = p->n_docs;
      a.doc_offsets = p->doc_offsets;
      a.doc_order = 1;
      break;
    default:
      break;
  }
  return mod;
}

}  // namespace

extern "C" {

const char* fl_status_str(fl_status s) {
  switch (s) {
    case FL_OK: return "ok";
    case FL_ERR_NULL: return "a required pointer is NULL";
    case FL_ERR_SHAPE: return "sizes inconsistent, negative or too large";
    case FL_ERR_ALIGN: return "pointer or row not aligned as required";
    case FL_ERR_UNSUPPORTED: return "head dimension / dtype combination not built";
    case FL_ERR_PARAM: return "variant parameter out of range";
    case FL_ERR_LAUNCH: return "kernel launch failed";
    case FL_ERR_SCRATCH: return "the call needs more than the library's static scratch buffer";
  }
  return "unknown status";
}

int fl_abi_version(void) { return FL_ABI_VERSION; }

fl_status fl_attn_fwd(const void* q, const void* k, const void* v, const void* bias, void* o,
                      float* lse, int B, int H_q, int H_kv, int S_q, int S_k, int D,
                      fl_dtype dtype, const fl_attn_params* p, void* stream) {
  if (!p) return FL_ERR_NULL;
  if (B < 0 || H_q < 1 || H_kv < 1 || S_q < 0 || S_k < 0 || D < 1) return FL_ERR_SHAPE;
  if (H_q % H_kv) return FL_ERR_SHAPE;
  if (S_q > kMaxSeq || S_k > kMaxSeq) return FL_ERR_SHAPE;
  if (dtype != FL_BF16 && dtype != FL_F32) return FL_ERR_UNSUPPORTED;
  const fl_status pv = check_params(p, S_q, S_k);
  if (pv != FL_OK) return pv;
  if (dtype == FL_BF16 && D != 64) return FL_ERR_UNSUPPORTED;
  if (dtype == FL_F32 && D != 32 && D != 64 && D != 128) return FL_ERR_UNSUPPORTED;
  if ((int64_t)B * H_q * S_q == 0) return FL_OK;  // no output element
  if (!q || !o || (S_k > 0 && (!k || !v))) return FL_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(bias, 16) || !aligned(lse, 4))
    return FL_ERR_ALIGN;
  if (bias && dtype == FL_BF16 && S_k % 8) return FL_ERR_ALIGN;

  KernelArgs a;
  init_args(a);
  a.q[0] = q;
  a.k[0] = k;
  a.v = v;
  a.bias = bias;
  a.o = o;
  a.lse[0] = lse;
  bhsd(H_q, S_q, D, a.q_sb, a.q_sh, a.q_si);
  bhsd(H_kv, S_k, D, a.k_sb, a.k_sh, a.k_si);
  bhsd(H_kv, S_k, D, a.v_sb, a.v_sh, a.v_si);
  bhsd(H_q, S_q, D, a.o_sb, a.o_sh, a.o_si);
  a.lse_sh = S_q;
  a.lse_sb = (int64_t)H_q * S_q;
  a.bias_si = S_k;
  a.bias_sh = (int64_t)S_q * S_k;
  a.nb = B;
  a.nh = H_q;
  a.alibi_nh = H_q;
  a.group = H_q / H_kv;
  a.sq = S_q;
  a.sk = S_k;
  a.scale_log2 = p->scale * kLog2e;
  int mod = variant_args(p, S_k, a);
  a.head_major = a.iv_kind == IV_FULL;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FL_F32) {
    a.n_qt = grid_qtiles(S_q, f32_rows_per_wg());
    if ((int64_t)a.n_qt * B * H_q > kMaxGrid) return FL_ERR_SHAPE;
    return launch_status(launch_f32(a, D, D, 1, mod, st));
  }
  if (!span_ok(S_k, D, D)) return FL_ERR_SHAPE;
  // softcap bounds every score by cap, so with a modest cap and no bias the
  // kernel needs no running reference
  if (mod == MOD_SOFTCAP && !bias && p->softcap * kLog2e <= 100.0f) mod = MOD_SOFTCAP_BOUNDED;
  // Two 32-row blocks per wave halve the LDS operand traffic per product.
  // Dense rows take them when that still leaves two work-groups per compute
  // unit (ALiBi too: its two-block form spills a few registers, about one
  // dword per lane per tile of extra traffic, and is still 8% faster).
  // Under a positional mask the taller tiles cross more partial key tiles
  // and balance worse: causal and PrefixLM rows take them from four
  // work-groups per unit (3% faster at B4 H16 S4096), document rows from
  // eight (at four they are 7% slower: short documents leave the taller
  // tiles mostly masked), and a sliding window, whose rows see few keys,
  // never does.
  const int64_t wg2 = (int64_t)grid_qtiles(S_q, attn_rows_per_wg(2)) * B * H_q;
#ifdef FL_FORCE_QB
  const int qb = FL_FORCE_QB;
#else
  int qb;
  if (mod == MOD_ALIBI && bias)
    qb = 1;  // the vector path's ALiBi with a bias: two blocks spill more, unmeasured
  else if (a.iv_kind == IV_FULL)
    qb = wg2 >= 512 ? 2 : 1;
  else if (a.iv_kind == IV_WINDOW_CAUSAL || a.iv_kind == IV_WINDOW_TWO_SIDED)
    qb = 1;
  else if (a.iv_kind == IV_DOCUMENT)
    qb = wg2 >= 2048 ? 2 : 1;
  else
    qb = wg2 >= 1024 ? 2 : 1;
#endif
  a.n_qt = grid_qtiles(S_q, attn_rows_per_wg(qb));
  if ((int64_t)a.n_qt * B * H_q > kMaxGrid) return FL_ERR_SHAPE;
  return launch_status(launch_attn_bf16(a, qb, mod, bias != nullptr, st));
}

fl_status fl_diffattn_fwd(const void* q1, const void* q2, const void* k1, const void* k2,
                          const void* v, void* o, float* lse1, float* lse2, int B, int H,
                          int S_q, int S_k, int D_qk, int D_v, fl_dtype dtype, float scale,
                          float lambda, int causal, void* stream) {
  if (B < 0 || H < 1 || S_q < 0 || S_k < 0 || D_qk < 1 || D_v < 1) return FL_ERR_SHAPE;
  if (S_q > kMaxSeq || S_k > kMaxSeq) return FL_ERR_SHAPE;
  if (causal && S_q != S_k) return FL_ERR_SHAPE;
  if (dtype != FL_BF16 && dtype != FL_F32) return FL_ERR_UNSUPPORTED;
  if (D_qk != 64 || (D_v != 64 && D_v != 128)) return FL_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(lambda)) return FL_ERR_PARAM;
  if ((int64_t)B * H * S_q == 0) return FL_OK;
  if (!q1 || !q2 || !o || (S_k > 0 && (!k1 || !k2 || !v))) return FL_ERR_NULL;
  if (!aligned(q1, 16) || !aligned(q2, 16) || !aligned(k1, 16) || !aligned(k2, 16) ||
      !aligned(v, 16) || !aligned(o, 16) || !aligned(lse1, 4) || !aligned(lse2, 4))
    return FL_ERR_ALIGN;

  KernelArgs a;
  init_args(a);
  a.q[0] = q1;
  a.q[1] = q2;
  a.k[0] = k1;
  a.k[1] = k2;
  a.v = v;
  a.o = o;
  a.lse[0] = lse1;
  a.lse[1] = lse2;
  bhsd(H, S_q, D_qk, a.q_sb, a.q_sh, a.q_si);
  bhsd(H, S_k, D_qk, a.k_sb, a.k_sh, a.k_si);
  bhsd(H, S_k, D_v, a.v_sb, a.v_sh, a.v_si);
  bhsd(H, S_q, D_v, a.o_sb, a.o_sh, a.o_si);
  a.lse_sh = S_q;
  a.lse_sb = (int64_t)H * S_q;
  a.nb = B;
  a.nh = H;
  a.group = 1;
  a.sq = S_q;
  a.sk = S_k;
  a.scale_log2 = scale * kLog2e;
  a.lambda = lambda;
  if (causal) {
    a.iv_kind = IV_CAUSAL;
    a.heavy_first = 1;
  }
  a.head_major = a.iv_kind == IV_FULL;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FL_F32) {
    a.n_qt = grid_qtiles(S_q, f32_rows_per_wg());
    if ((int64_t)a.n_qt * B * H > kMaxGrid) return FL_ERR_SHAPE;
    return launch_status(launch_f32(a, D_qk, D_v, 2, MOD_NONE, st));
  }
  if (!span_ok(S_k, D_v, D_v)) return FL_ERR_SHAPE;
  a.n_qt = grid_qtiles(S_q, mfma_rows_per_wg(1));
  if ((int64_t)a.n_qt * B * H > kMaxGrid) return FL_ERR_SHAPE;
  return launch_status(launch_diff_bf16(a, D_qk, D_v, st));
}

fl_status fl_evoformer_gated_attn_fwd(const void* q, const void* k, const void* v,
                                      const void* gate, const void* pair_bias,
                                      const uint8_t* key_mask, void* o, int N_seq, int N_res,
                                      int H, int C, fl_evo_axis axis, fl_dtype dtype,
                                      float scale, void* stream) {
  if (N_seq < 0 || N_res < 0 || H < 1 || C < 1) return FL_ERR_SHAPE;
  if (N_seq > kMaxSeq || N_res > kMaxSeq) return FL_ERR_SHAPE;
  if (axis != FL_EVO_ROW && axis != FL_EVO_COL) return FL_ERR_PARAM;
  if (axis == FL_EVO_COL && pair_bias) return FL_ERR_PARAM;
  if (dtype != FL_BF16 && dtype != FL_F32) return FL_ERR_UNSUPPORTED;
  if (C != 32) return FL_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FL_ERR_PARAM;
  if ((int64_t)N_seq * N_res == 0) return FL_OK;
  if (!q || !k || !v || !gate || !o) return FL_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(gate, 16) ||
      !aligned(o, 16) || !aligned(pair_bias, 16))
    return FL_ERR_ALIGN;
  if (pair_bias && dtype == FL_BF16 && N_res % 8) return FL_ERR_ALIGN;

  KernelArgs a;
  init_args(a);
  a.q[0] = q;
  a.k[0] = k;
  a.v = v;
  a.gate = gate;
  a.bias = pair_bias;
  a.kmask = key_mask;
  a.o = o;
  const int64_t row = (int64_t)H * C;  // one (sequence, residue) position
  int L;
  if (axis == FL_EVO_ROW) {
    // batch = MSA row s, positions = residues
    a.nb = N_seq;
    L = N_res;
    a.q_sb = (int64_t)N_res * row;
    a.q_si = row;
    a.km_sb = N_res;
    a.km_sj = 1;
  } else {
    // batch = residue column r, positions = sequences
    a.nb = N_res;
    L = N_seq;
    a.q_sb = row;
    a.q_si = (int64_t)N_res * row;
    a.km_sb = 1;
    a.km_sj = N_res;
  }
  a.q_sh = C;
  a.k_sb = a.v_sb = a.o_sb = a.q_sb;
  a.k_si = a.v_si = a.o_si = a.q_si;
  a.k_sh = a.v_sh = a.o_sh = a.q_sh;
  a.bias_si = L;
  a.bias_sh = (int64_t)L * L;
  a.nh = H;
  a.group = 1;
  a.sq = L;
  a.sk = L;
  a.scale_log2 = scale * kLog2e;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FL_F32) {
    a.n_qt = grid_qtiles(L, f32_rows_per_wg());
    if ((int64_t)a.n_qt * a.nb * H > kMaxGrid) return FL_ERR_SHAPE;
    return launch_status(launch_f32(a, C, C, 1, MOD_NONE, st));
  }
  if (!span_ok(L, a.k_si, C)) return FL_ERR_SHAPE;
  // Rows of at most 256 positions: the short-row kernel, which keeps each
  // wave's bias rows in registers across the entries it walks (row form at
  // 128 x 256, H = 8: 41 against 54 us cold) and without a bias runs three
  // waves per SIMD (column form: 31.7 against 32.6 us cold, 22.4 against
  // 24.8 us warm).
  if (L <= kEvoShortMax) {
    if ((int64_t)a.nb * (H + 1) + 16 > kMaxGrid) return FL_ERR_SHAPE;
    return launch_status(launch_evo_short_bf16(a, st));
  }
  const int qb = L > 128 ? 2 : 1;
  a.n_qt = grid_qtiles(L, mfma_rows_per_wg(qb));
  if ((int64_t)a.n_qt * a.nb * H > kMaxGrid) return FL_ERR_SHAPE;
  // A work-group may walk several batch entries (MSA rows or columns) of one
  // head with its tile pipeline running across them.  Measured at the
  // AlphaFold2 sizes: two entries per work-group help the two-block tiles
  // of long key ranges (256 residues), one is best for one-block tiles.
#ifdef FL_EVO_ROWS
  a.rows_per_wg = FL_EVO_ROWS;
#else
  a.rows_per_wg = qb == 2 ? 2 : 1;
#endif
  return launch_status(launch_evo_bf16(a, C, qb, pair_bias != nullptr, st));
}

int fl_attn_decode_num_splits(int B, int H_q, int H_kv, int S_q, int max_seqlen,
                              const fl_attn_params* p, int num_splits) {
  if (!decode_sizes_ok(B, H_q, H_kv, S_q, max_seqlen) || num_splits < 0) return -1;
  const int n_split = decode_split(B, H_q, H_kv, S_q, max_seqlen, p, num_splits);
  return n_split;
}

int64_t fl_attn_decode_workspace_size(int B, int H_q, int H_kv, int S_q, int max_seqlen, int D,
                                      const fl_attn_params* p, int num_splits) {
  if (!decode_sizes_ok(B, H_q, H_kv, S_q, max_seqlen) || D < 1 || num_splits < 0) return -1;
  const int n_split = decode_split(B, H_q, H_kv, S_q, max_seqlen, p, num_splits);
  return decode_workspace(B, H_q, S_q, D, n_split);
}

}  // extern "C"

namespace fl {

fl_status decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* cache_seqlens, void* o, float* lse, DecodeWorkspaceFn get_ws,
                     void* ws_ctx, int B, int H_q, int H_kv, int S_q, int S_cap, int max_seqlen,
                     int D, fl_kv_layout layout, fl_dtype dtype, const fl_attn_params* p,
                     int num_splits, void* stream) {
  if (!p) return FL_ERR_NULL;
  if (!decode_sizes_ok(B, H_q, H_kv, S_q, max_seqlen) || S_cap < 0 || S_cap > kMaxSeq || D < 1)
    return FL_ERR_SHAPE;
  if (layout != FL_KV_BHSD && layout != FL_KV_BSHD) return FL_ERR_PARAM;
  if (dtype != FL_BF16 || D != 64) return FL_ERR_UNSUPPORTED;
  if (p->variant < FL_VANILLA || p->variant > FL_DOCUMENT) return FL_ERR_PARAM;
  if (!isfinite(p->scale) || num_splits < 0) return FL_ERR_PARAM;
  if (max_seqlen > S_cap) return FL_ERR_PARAM;
  const bool variant_is_mask = p->variant >= FL_CAUSAL;
  if (p->mask != FL_VANILLA && (variant_is_mask || p->mask < FL_CAUSAL || p->mask > FL_DOCUMENT))
    return FL_ERR_PARAM;
  const int mask = variant_is_mask ? p->variant : p->mask;
  if (mask == FL_DOCUMENT) return FL_ERR_UNSUPPORTED;
  if (p->variant == FL_SOFTCAP && !(p->softcap > 0.0f && isfinite(p->softcap))) return FL_ERR_PARAM;
  if (p->variant == FL_ALIBI && !(p->alibi_max_bias >= 0.0f && isfinite(p->alibi_max_bias)))
    return FL_ERR_PARAM;
  if (mask == FL_SLIDING_WINDOW && p->window < 1) return FL_ERR_PARAM;
  if (mask == FL_PREFIX_LM && p->prefix < 0) return FL_ERR_PARAM;
  if ((int64_t)B * H_q * S_q == 0) return FL_OK;  // no output element
  if (!q || !o || !cache_seqlens || (S_cap > 0 && (!k_cache || !v_cache))) return FL_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(cache_seqlens, 4))
    return FL_ERR_ALIGN;

  const int G = H_q / H_kv;
  const int n_split = decode_split(B, H_q, H_kv, S_q, max_seqlen, p, num_splits);
  const int64_t ws = decode_workspace(B, H_q, S_q, D, n_split);

  KernelArgs a;
  init_args(a);
  a.q[0] = q;
  a.k[0] = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse[0] = lse;
  // the G query heads of a K/V head are one packed head of G * S_q rows
  a.q_si = D;
  a.q_sh = (int64_t)G * S_q * D;
  a.q_sb = (int64_t)H_q * S_q * D;
  a.o_si = a.q_si;
  a.o_sh = a.q_sh;
  a.o_sb = a.q_sb;
  a.lse_sh = (int64_t)G * S_q;
  a.lse_sb = (int64_t)H_q * S_q;
  if (layout == FL_KV_BHSD) {
    bhsd(H_kv, S_cap, D, a.k_sb, a.k_sh, a.k_si);
  } else {
    a.k_si = (int64_t)H_kv * D;
    a.k_sh = D;
    a.k_sb = (int64_t)S_cap * H_kv * D;
  }
  a.v_sb = a.k_sb;
  a.v_sh = a.k_sh;
  a.v_si = a.k_si;
  if (!span_ok(S_cap, a.k_si, D)) return FL_ERR_SHAPE;
  a.nb = B;
  a.nh = H_kv;
  a.alibi_nh = H_q;
  a.group = 1;
  a.grp = G;
  a.sq = G * S_q;
  a.sq_new = S_q;
  a.sk = S_cap;
  a.max_len = max_seqlen;
  a.seqlens = cache_seqlens;
  a.scale_log2 = p->scale * kLog2e;
  int mod = MOD_NONE;
  if (p->variant == FL_ALIBI) {
    mod = MOD_ALIBI;
    a.alibi_max_bias = p->alibi_max_bias;
  } else if (p->variant == FL_SOFTCAP) {
    mod = p->softcap * kLog2e <= 100.0f ? MOD_SOFTCAP_BOUNDED : MOD_SOFTCAP;
    a.softcap_arg = 2.0f * p->scale * kLog2e / p->softcap;
    a.softcap_log2 = p->softcap * kLog2e;
  }
  // wider windows and prefixes than every distance present change nothing
  const int far = (max_seqlen > S_q ? max_seqlen : S_q) + 1;
  switch (mask) {
    case FL_CAUSAL:
      a.iv_kind = IV_CAUSAL;
      break;
    case FL_SLIDING_WINDOW:
      a.iv_kind = p->window_causal ? IV_WINDOW_CAUSAL : IV_WINDOW_TWO_SIDED;
      a.window = p->window > far ? far : p->window;
      break;
    case FL_PREFIX_LM:
      a.iv_kind = IV_PREFIX;
      a.prefix = p->prefix > max_seqlen ? max_seqlen : p->prefix;
      break;
    default:
      break;
  }
  a.n_qt = grid_qtiles(G * S_q, decode_rows_per_wg());
  a.n_split = n_split;
  if ((int64_t)a.n_qt * B * H_kv * n_split > kMaxGrid) return FL_ERR_SHAPE;
  const int64_t rows = (int64_t)B * H_q * S_q;
  if (n_split > 1 && (rows + 3) / 4 > kMaxGrid) return FL_ERR_SHAPE;
  // everything checked: only now is the workspace asked for
  void* workspace = nullptr;
  const fl_status wrc = get_ws(ws, ws_ctx, &workspace);
  if (wrc != FL_OK) return wrc;
  if (n_split > 1) {
    a.o_part = (float*)workspace;
    a.lse_part = (float*)((char*)workspace + (int64_t)n_split * rows * D * 4);
  }
  hipStream_t st = (hipStream_t)stream;
  const fl_status rc = launch_status(launch_decode_bf16(a, mod, st));
  if (rc != FL_OK || n_split == 1) return rc;
  return launch_status(launch_merge(a.o_part, a.lse_part, n_split, rows, D, o, true, lse, st));
}

}  // namespace fl

namespace {

// the caller's workspace: present when needed, large enough, 16-byte aligned
struct CallerWorkspace {
  void* ptr;
  size_t bytes;
};

fl_status caller_workspace(int64_t need, void* ctx, void** ws) {
  const CallerWorkspace* c = (const CallerWorkspace*)ctx;
  if (need > 0 && !c->ptr) return FL_ERR_NULL;
  if ((int64_t)c->bytes < need) return FL_ERR_PARAM;
  *ws = c->ptr;
  return FL_OK;
}

}  // namespace

extern "C" {

fl_status fl_attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cache_seqlens, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, int B, int H_q, int H_kv, int S_q, int S_cap,
                             int max_seqlen, int D, fl_kv_layout layout, fl_dtype dtype,
                             const fl_attn_params* p, int num_splits, void* stream) {
  if (!aligned(workspace, 16)) return FL_ERR_ALIGN;
  CallerWorkspace cw = {workspace, workspace_bytes};
  return decode_fwd(q, k_cache, v_cache, cache_seqlens, o, lse, caller_workspace, &cw, B, H_q,
                    H_kv, S_q, S_cap, max_seqlen, D, layout, dtype, p, num_splits, stream);
}

fl_status fl_ipa_attn_fwd(const void* q, const void* k, const void* v, const float* q_pts,
                          const float* k_pts, const float* v_pts, const float* rot,
                          const float* trans, const float* gamma, const void* pair_bias,
                          const void* z, const uint8_t* key_mask, void* o, float* o_pts,
                          void* o_pair, int B, int L, int H, int C, int P_q, int P_v, int C_z,
                          fl_dtype dtype, void* stream) {
  if (B < 0 || L < 0 || H < 1 || C < 1 || P_q < 1 || P_v < 1 || C_z < 0) return FL_ERR_SHAPE;
  if (L > kMaxSeq) return FL_ERR_SHAPE;
  if ((z == nullptr) != (o_pair == nullptr)) return FL_ERR_NULL;
  if (z && C_z < 1) return FL_ERR_SHAPE;
  if (dtype != FL_BF16) return FL_ERR_UNSUPPORTED;
  if (C != 16 || P_q != 4 || P_v != 8) return FL_ERR_UNSUPPORTED;
  if (z && C_z != 64 && C_z != 128) return FL_ERR_UNSUPPORTED;
  if ((int64_t)B * L == 0) return FL_OK;
  if (!q || !k || !v || !q_pts || !k_pts || !v_pts || !rot || !trans || !gamma || !o || !o_pts)
    return FL_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_pts, 16) ||
      !aligned(k_pts, 16) || !aligned(v_pts, 16) || !aligned(o, 16) || !aligned(o_pts, 16) ||
      !aligned(z, 16) || !aligned(o_pair, 16) || !aligned(rot, 4) || !aligned(trans, 4) ||
      !aligned(gamma, 4) || !aligned(pair_bias, 2))
    return FL_ERR_ALIGN;
  // one residue's pair rows z[b, i, :, :] go through a 32-bit buffer resource
  if (z && (int64_t)L * C_z * 2 >= ((int64_t)1 << 31)) return FL_ERR_SHAPE;
  const int64_t n_hg = (H + 3) / 4;
  if ((int64_t)B * L * n_hg > kMaxGrid) return FL_ERR_SHAPE;
  IpaArgs a = {};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.q_pts = q_pts;
  a.k_pts = k_pts;
  a.v_pts = v_pts;
  a.rot = rot;
  a.trans = trans;
  a.gamma = gamma;
  a.bias = (const bf16*)pair_bias;
  a.z = (const bf16*)z;
  a.kmask = key_mask;
  a.o = (bf16*)o;
  a.o_pts = o_pts;
  a.o_pair = (bf16*)o_pair;
  a.B = B;
  a.L = L;
  a.H = H;
  // AlphaFold2's weights: w_L = sqrt(1/3) over the three logit terms,
  // w_C = sqrt(2 / (9 P_q)) on the point distances; base-2 units
  const double w_l = sqrt(1.0 / 3.0), w_c = sqrt(2.0 / (9.0 * P_q));
  a.w_scalar = (float)(w_l / sqrt((double)C) * 1.4426950408889634);
  a.w_bias = (float)(w_l * 1.4426950408889634);
  a.w_point = (float)(w_l * w_c * 0.5 * 1.4426950408889634);
  return launch_status(launch_ipa_bf16(a, z ? C_z : 0, (hipStream_t)stream));
}

fl_status fl_attn_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                        int n_parts, int64_t n_rows, int D, fl_dtype out_dtype, void* stream) {
  if (n_parts < 1 || n_rows < 0 || D < 1) return FL_ERR_SHAPE;
  if (out_dtype != FL_BF16 && out_dtype != FL_F32) return FL_ERR_UNSUPPORTED;
  if (n_rows == 0) return FL_OK;
  if ((n_rows + 3) / 4 > kMaxGrid) return FL_ERR_SHAPE;
  if (!o_parts || !lse_parts || !o) return FL_ERR_NULL;
  if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(lse, 4) ||
      !aligned(o, out_dtype == FL_BF16 ? 2 : 4))
    return FL_ERR_ALIGN;
  return launch_status(launch_merge(o_parts, lse_parts, n_parts, n_rows, D, o,
                                    out_dtype == FL_BF16, lse, (hipStream_t)stream));
}

fl_status fl_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                      const float* lse, void* dq, void* dk, void* dv, float* workspace, int B,
                      int H_q, int H_kv, int S_q, int S_k, int D, fl_dtype dtype,
                      const fl_attn_params* p, void* stream) {
  if (!p) return FL_ERR_NULL;
  if (B < 0 || H_q < 1 || H_kv < 1 || S_q < 0 || S_k < 0 || D < 1) return FL_ERR_SHAPE;
  if (H_q % H_kv) return FL_ERR_SHAPE;
  if (S_q > kMaxSeq || S_k > kMaxSeq) return FL_ERR_SHAPE;
  if (dtype != FL_BF16 || D != 64) return FL_ERR_UNSUPPORTED;
  const fl_status pv = check_params(p, S_q, S_k);
  if (pv != FL_OK) return pv;
  const bool no_q = (int64_t)B * H_q * S_q == 0, no_k = (int64_t)B * H_kv * S_k == 0;
  if (no_q && no_k) return FL_OK;
  if ((!no_k && (!k || !v || !dk || !dv)) || (!no_q && (!q || !o || !d_o || !lse || !dq)) ||
      (!no_q && !no_k && !workspace))
    return FL_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(d_o, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 4))
    return FL_ERR_ALIGN;
  if (!span_ok(S_k, D, D) || !span_ok(S_q, D, D)) return FL_ERR_SHAPE;
  hipStream_t st = (hipStream_t)stream;

  KernelArgs a;
  init_args(a);
  a.q[0] = q;
  a.k[0] = k;
  a.v = v;
  a.lse[0] = const_cast<float*>(lse);
  bhsd(H_q, S_q, D, a.q_sb, a.q_sh, a.q_si);
  bhsd(H_kv, S_k, D, a.k_sb, a.k_sh, a.k_si);
  bhsd(H_kv, S_k, D, a.v_sb, a.v_sh, a.v_si);
  bhsd(H_q, S_q, D, a.o_sb, a.o_sh, a.o_si);
  a.lse_sh = S_q;
  a.lse_sb = (int64_t)H_q * S_q;
  a.nb = B;
  a.nh = H_q;
  a.alibi_nh = H_q;
  a.group = H_q / H_kv;
  a.sq = S_q;
  a.sk = S_k;
  a.scale_log2 = p->scale * kLog2e;
  const int mod = variant_args(p, S_k, a);
  const int64_t rows_q = (int64_t)B * H_q * ((S_q + 127) / 128);
  const int64_t rows_k = (int64_t)B * H_kv * ((S_k + 127) / 128);
  if (rows_q > kMaxGrid || rows_k > kMaxGrid) return FL_ERR_SHAPE;
  BwdArgs g;
  g.o = o;
  g.dout = d_o;
  g.dq = dq;
  g.dk = dk;
  g.dv = dv;
  g.delta = workspace;
  g.lse2 = workspace + (int64_t)B * H_q * S_q;
  return launch_status(launch_bwd_bf16(a, g, mod, st));
}

}  // extern "C"
