// attn_mfma.hpp -- the bf16 fused attention forward on gfx950 matrix cores.
//
// One work-group = 4 waves = a tile of BM = 4*32*QB query rows of one (b, h)
// (two softmax streams: 8 waves, four per stream over the same rows).
// Each wave owns 32*QB rows for the whole kernel: its Q rows sit in
// registers, already in matrix-core operand order; K and V stream through
// LDS in tiles of 64 keys, double-buffered, with the next tile's global loads
// in flight while the current one is consumed.  Per tile and per 32-query
// block the wave computes
//
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, one lane per query column
//   score mod / bias / mask in registers (masks only on tiles that need them)
//   online softmax: running max m and sum l per row, rescaled by
//                   2^(m_old - m_new) when m grows
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, P rounded to bf16
//
// and finally O = O^T / l (gated, or differenced for DiffAttn) is stored.
// The score matrix never leaves registers: the key axis is the kernel's inner
// reduction loop and the softmax is single-pass (gist.science explainer of
// Flashlight, "Technical Summary: Methodology", structural fusion with
// dimension demotion and semantic fusion; papers.lqhl.me wiki, "核心方法").
//
// Why S^T rather than S: in the 32x32 accumulator layout a lane holds one
// output column and 16 of its rows (rows 8*(r/4) + 4*g + r%4 of register r in
// lane half g).  With queries as columns every lane owns one query: the row
// max and row sum are reductions inside the lane plus the half held by the
// lane 32 apart, and the rescale factor of a row is a per-lane scalar for the
// O^T accumulator too.  The S^T registers, rounded to bf16, are directly the
// B operand of the P.V product once V^T's key order inside each 16-key step
// is permuted to match: keys 16*st + 4*g + 0..3, then 16*st + 8 + 4*g + 0..3.
// V stays row-major in LDS; ds_read_b64_tr_b16 delivers those transposed
// 4-key groups (16 lanes read a 4 x 16 block and each receives a column).
#pragma once

#include <type_traits>

#include "fl_common.hpp"

namespace fl {

template <int DQK_, int DV_, int NS_, int QB_, int MOD_, bool BIAS_, bool KMASK_, bool GATE_,
          bool DEC_ = false>
struct MfmaCfg {
  static constexpr int DQK = DQK_;   // q/k head dim (multiple of 16)
  static constexpr int DV = DV_;     // v head dim (multiple of 32)
  static constexpr int NS = NS_;     // softmax streams: 1, or 2 for DiffAttn
  static constexpr int QB = QB_;     // 32-query blocks per wave
  static constexpr int MOD = MOD_;
  static constexpr bool BIAS = BIAS_;
  static constexpr bool KMASK = KMASK_;
  static constexpr bool GATE = GATE_;
  // decode against a KV cache: packed GQA rows, per-sequence lengths, key
  // splits (see KernelArgs)
  static constexpr bool DEC = DEC_;
  // gated (Evoformer) launches: a work-group walks rows_per_wg consecutive
  // batch entries (MSA rows) of one head and query tile, its K/V tile
  // pipeline running straight across the entries, so the short per-entry
  // key ranges do not each pay a work-group's start-up
  static constexpr bool PERSIST = GATE_;
  // waves per work-group; decode rows are few (the G query heads of one K/V
  // head), so its work-groups are narrower and more of them fit a unit
#ifndef FL_DEC_WAVES
#define FL_DEC_WAVES 4
#endif
  // Two streams (DiffAttn) split over the waves: eight waves, the first four
  // take stream 0 of the work-group's rows and the last four stream 1; each
  // wave then holds one stream's state, which leaves room for two waves per
  // SIMD, and the streams meet through LDS at the end.
  static constexpr bool SPLIT = NS_ == 2;
  static constexpr int NSU = SPLIT ? 1 : NS_;  // streams per wave
#ifndef FL_FWD_WAVES
#define FL_FWD_WAVES 4
#endif
  static constexpr int NW = DEC ? FL_DEC_WAVES : (SPLIT ? 8 : (GATE ? 4 : FL_FWD_WAVES));
  static constexpr int RW = SPLIT ? NW / NS_ : NW;  // waves per stream (row blocks)
  static constexpr int BM = RW * 32 * QB;    // query rows per work-group
  static constexpr int BN = 64;              // keys per tile
  // K and V tiles sit in LDS row-major without padding; the 16-byte chunks
  // of a row are XOR-swizzled by the row index so that the operand reads
  // hit distinct banks (64 banks of 4 bytes).  A K read serves 16 lanes
  // (16 consecutive rows, one logical chunk) per cycle: the eight rows of
  // each parity share a bank half, so with 128-byte rows the swizzle
  // follows the row pair, (row >> 1) & 7 (row & 7 gave rows 8 apart the
  // same banks, a two-way conflict on every K read); with 64-byte rows,
  // rows 4 apart share banks and it follows (row >> 2) & 3.  A transposed
  // V read serves 32 lanes (four rows x four chunks) per cycle.
  static constexpr int KCPR = DQK / 8;       // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;        // 16-byte chunks per V row
  static constexpr int K_ELEMS = BN * DQK;
  static constexpr int V_ELEMS = BN * DV;
  static constexpr int STAGE = NS * K_ELEMS + V_ELEMS;
  // LDS stages: the tile in use plus STAGES - 1 tiles landed or in flight.
  // Decode streams each cached key once with little work per byte, so it
  // keeps more bytes in flight per work-group.
#ifndef FL_DEC_STAGES
#define FL_DEC_STAGES 3
#endif
#ifndef FL_EVO_STAGES
#define FL_EVO_STAGES 3
#endif
#ifndef FL_FWD_STAGES
#define FL_FWD_STAGES 3
#endif
  static constexpr int STAGES = DEC ? FL_DEC_STAGES : (GATE ? FL_EVO_STAGES : FL_FWD_STAGES);
  __device__ static constexpr int kswz(int row) { return KCPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7; }
  __device__ static constexpr int vswz(int row) { return VCPR == 4 ? 2 * ((row >> 1) & 1) : 2 * (row & 3); }
  static constexpr int KCH = BN * DQK / 8 / (NW * 64);  // 16-byte K chunks per thread
  static constexpr int VCH = BN * DV / 8 / (NW * 64);   // 16-byte V chunks per thread
  // gated launches that walk several entries per work-group (two query
  // blocks per wave): the gate rows of an entry (BM x DV) go to LDS when
  // the entry starts, double-buffered by entry parity.  (With one entry per
  // work-group the gate is read in the epilogue directly: measured faster.)
  static constexpr bool GATE_LDS = GATE && QB == 2;
  static constexpr int G_ELEMS = GATE_LDS ? BM * DV : 0;
  static constexpr int GCH = G_ELEMS / 8 / (NW * 64);  // 16-byte gate chunks per thread
  // Folded scores: the scale, the running reference, the ALiBi distance
  // penalty or the key mask all enter the S^T product itself.
  static constexpr bool FOLD = (MOD == MOD_NONE || MOD == MOD_ALIBI) && !BIAS;
  static constexpr bool ALIBI_FOLD = FOLD && MOD == MOD_ALIBI;
  static_assert(!(ALIBI_FOLD && KMASK), "ALiBi and the key mask share a folded k-slot");
  // bounded softcap: fixed reference 0
  static constexpr bool SCAPB = MOD == MOD_SOFTCAP_BOUNDED;
  // Folded scores without a key mask (plain or ALiBi) and the bounded
  // softcap (one stream per wave; not decode or gated): a first pass keeps a fixed
  // reference (0; c = cap log2(e) for the softcap) with no per-unit test and
  // sums rows on the matrix cores; if any row of the work-group ends with a
  // sum out of range (or not finite) with keys allowed, the pass is
  // discarded and the checked pass (for the softcap: reference 0) runs.
  static constexpr bool FASTP = (FOLD || SCAPB) && !KMASK && !GATE && !DEC && NSU == 1;
  static_assert(!SCAPB || (!BIAS && !KMASK), "bounded softcap takes no bias or key mask");
  static_assert(!DEC || (QB == 1 && NS == 1 && !BIAS && !KMASK && !GATE), "decode form");
  static_assert(STAGES >= 3 && STAGES <= 6, "pipeline depth");
  // one stream fits 2 waves per SIMD; two streams need the whole register file
#ifndef FL_QB1_WAVES
#define FL_QB1_WAVES 2
#endif
  static constexpr int WAVES_PER_EU = NSU == 1 ? (QB == 1 ? FL_QB1_WAVES : 2) : 1;
  static_assert(DQK % 16 == 0 && DV % 32 == 0, "head dims");
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the work-group");
};

// Row of the 32-row block held by accumulator register r in lane half 0
// (lane half g adds 4*g).
__device__ __forceinline__ constexpr int acc_row(int r) { return 8 * (r >> 2) + (r & 3); }

// Bounds-checked 128-bit load: bytes at or past the resource's end read as 0.
__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// One transposed 8-byte LDS read (ds_read_b64_tr_b16) at LDS byte address
// `addr`: the 16 lanes of a block each point at 4 consecutive 16-bit values
// of a 4 x 16 block (row i/4, columns 4(i%4)..+3 for lane i) and lane i
// receives column i, rows 0..3.
__device__ __forceinline__ u32x2 ds_read_tr(uint32_t addr) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)addr));
}

// Cross-lane reads whose lane-address register is formed where it is used
// (the lane index comes from assembly, which the compiler does not hoist):
// left to itself the compiler computes such addresses once, at the top of
// the kernel, and keeps them live across the whole tile loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
// x of lane (this lane & 15)
__device__ __forceinline__ float lane_read16(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute((lane_here() & 15) << 2, __builtin_bit_cast(int, x)));
}
// x of lane (this lane ^ 32)
__device__ __forceinline__ float lane_xor32(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_bpermute((lane_here() ^ 32) << 2, __builtin_bit_cast(int, x)));
}

#ifndef FL_SCHED_INTERLEAVE
#define FL_SCHED_INTERLEAVE 1
#endif
#ifndef FL_SCHED_VALU_PER_MFMA
#define FL_SCHED_VALU_PER_MFMA 5
#endif

// Scheduling shape of one pipeline unit's basic block (the previous unit's
// P.V products, this unit's successor's S^T products, this unit's
// exponentials): operand reads from LDS first, then each matrix instruction
// followed by a few independent vector instructions, so the matrix core runs
// while the wave keeps issuing vector work.
__device__ __forceinline__ void interleave_hint() {
#if FL_SCHED_INTERLEAVE == 1
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, FL_SCHED_VALU_PER_MFMA, 0);  // a few VALU
  }
#elif FL_SCHED_INTERLEAVE == 2
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#endif
}

#ifndef FL_SCAPB_VALU
#define FL_SCAPB_VALU 9
#endif
// One bounded-softcap unit, a single basic block: the K operand reads, then
// each matrix instruction (the successor's S^T products, the predecessor's
// P.V products) followed by a share of this unit's vector work (8 or 9 per
// instruction measured 2.7% faster than 14, 7 slower).
__device__ __forceinline__ void unit_hint_scapb() {
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, FL_SCAPB_VALU, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

#ifndef FL_FAST_VALU
#define FL_FAST_VALU 5
#endif

// One unit of the unchecked first pass on plain folded scores: the K
// operand reads, then each of the ten matrix instructions followed by a
// share of the vector work (5 per instruction measured 1.5% faster on
// vanilla than the compiler's own order, 3 to 5 alike; ALiBi, with its
// folded step, lost 0.8% and keeps the compiler's order).
__device__ __forceinline__ void unit_hint_fast() {
#if FL_FAST_VALU > 0
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, FL_FAST_VALU, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Document mask work order.  A query tile costs as many key tiles as its
// rows' documents span, which varies along the sequence, so the plain order
// can leave a long tile for the end of the grid.  Here the (batch entry,
// query tile) items go out longest first, the heads of one item adjacent
// (work-group id = rank * H + head).  Every work-group ranks all items
// itself in LDS: it needs no buffer and no second launch, and the keys
// (span, index) are unique, so the ranks form a permutation whatever the
// offsets hold.  `ws` holds the offsets of every batch entry (copied by
// the caller) and room for 2 NT ints after kDocOrderMaxOffsets.  Returns
// false (the caller keeps the plain order) when the items outnumber the
// work-group's NT threads.  The caller synchronises before the LDS is
// written again.
constexpr int kDocOrderMaxOffsets = 1024;
template <int NT, int BN>
__device__ bool doc_order_tile(const KernelArgs& a, int bm, int* ws, int& bh, int& qt) {
  const int n = a.nb * a.n_qt;
  if (n > NT) return false;
  const int tid = threadIdx.x;
  const int* off = ws;
  int* key = ws + kDocOrderMaxOffsets;
  int* perm = key + NT;
  if (tid < n) {
    const int b = tid / a.n_qt, t = tid % a.n_qt;
    const int* o = off + b * (a.n_docs + 1);
    // the document of row i: the largest d < n_docs with o[d] <= i
    auto doc_of = [&](int i) {
      int lo = 0, hi = a.n_docs - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (o[mid] <= i) lo = mid; else hi = mid - 1;
      }
      return lo;
    };
    // rows' key intervals are monotone: the tile spans lo(first) .. hi(last)
    const int q0 = t * bm, q1 = min(q0 + bm, a.sq) - 1;
    const int lo = max(o[doc_of(q0)], 0), hi = min(o[doc_of(q1) + 1] - 1, a.sk - 1);
    const int span = lo <= hi ? hi / BN - lo / BN + 1 : 0;
    key[tid] = (min(span, 0x7fff) << 16) | (0xffff - tid);
  }
  // pad the keys to a multiple of 4 with 0, below every real key (those
  // hold 0xffff - tid > 0 in their low half)
  const int n4 = (n + 3) & ~3;
  if (tid >= n && tid < n4) key[tid] = 0;
  __syncthreads();
  if (tid < n) {
    // rank = number of larger keys; the wave reads the same 16 bytes at
    // once (a broadcast), eight reads in flight
    const int mine = key[tid];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < n4; j += 4) {
      const int4 kk = *(const int4*)(key + j);
      rank += (kk.x > mine) + (kk.y > mine) + (kk.z > mine) + (kk.w > mine);
    }
    perm[rank] = tid;
  }
  __syncthreads();
  const int item = perm[blockIdx.x / a.nh];
  bh = (item / a.n_qt) * a.nh + blockIdx.x % a.nh;
  qt = item % a.n_qt;
  return true;
}

template <class C>
__global__ __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU)))
void attn_mfma_kernel(KernelArgs a) {
  constexpr int BN = C::BN, DQK = C::DQK, DV = C::DV, NS = C::NS, QB = C::QB;
  constexpr int NSU = C::NSU;  // streams held by one wave
  __shared__ __attribute__((aligned(16))) bf16 lds[C::STAGES * C::STAGE];
  __shared__ __attribute__((aligned(16))) float kmadd[C::KMASK ? C::STAGES * BN : 4];
  __shared__ __attribute__((aligned(16))) bf16 gbuf[C::GATE_LDS ? 2 * C::G_ELEMS : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;
  // split streams: this wave's stream and row block
  const int ws = C::SPLIT ? w / C::RW : 0, wr = C::SPLIT ? w % C::RW : w;
  auto stream_of = [&](int s) { return C::SPLIT ? ws : s; };

  int bh, qt, split = 0;
  int b_first = 0, n_rep = 1;  // batch entries this work-group walks
  bool doc_lds = false;        // the document offsets sit in LDS (prologue only)
  if constexpr (C::DEC) {
    split = blockIdx.x % a.n_split;
    const int rest = blockIdx.x / a.n_split;
    qt = rest % a.n_qt;
    bh = rest / a.n_qt;
  } else if constexpr (C::PERSIST) {
    // Heads of one position are adjacent in memory (a head's row is 64
    // bytes), so the work-groups of all heads of a batch entry share an
    // XCD, whose L2 then serves each 128-byte line to both of its heads.
    const int n_grp = (a.nb + a.rows_per_wg - 1) / a.rows_per_wg;
    int item = blockIdx.x;  // (row group, query tile, head), head fastest
    int hh, grp;
    // With a pair bias shared by every batch entry, an XCD takes one pair of
    // heads (the two heads of a 128-byte line) for a share of the row
    // groups, so that each XCD's L2 holds only its heads' bias.
    const int n_pair = a.nh >> 1, per_pair = n_pair > 0 && 8 % n_pair == 0 ? 8 / n_pair : 0;
    if (C::BIAS && a.bias && (a.nh & 1) == 0 && per_pair > 0 && n_grp % per_pair == 0) {
      const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
      const int e = slot & 1, rest = slot >> 1;
      qt = rest % a.n_qt;
      grp = (xcd / n_pair) + per_pair * (rest / a.n_qt);
      hh = 2 * (xcd % n_pair) + e;
    } else {
      if ((n_grp & 7) == 0) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int per = a.nh * a.n_qt;  // items of one row group
        item = ((slot / per) * 8 + xcd) * per + slot % per;
      }
      hh = item % a.nh;
      const int rest = item / a.nh;
      qt = rest % a.n_qt;
      grp = rest / a.n_qt;
    }
    b_first = grp * a.rows_per_wg;
    n_rep = min(a.rows_per_wg, a.nb - b_first);
    bh = b_first * a.nh + hh;
  } else {
    // Document mask: the offsets of every batch entry go to LDS once, where
    // the work order and every key interval of the prologue search them
    // (a search through global memory costs a round trip per step).  The
    // K/V tiles overwrite them after the prologue's closing barrier.
    static_assert(sizeof(lds) >= (kDocOrderMaxOffsets + 2 * C::NW * 64) * sizeof(int),
                  "LDS for the document order");
    const int n_off = a.nb * (a.n_docs + 1);
    doc_lds = a.iv_kind == IV_DOCUMENT && n_off <= kDocOrderMaxOffsets;
    if (doc_lds) {
      for (int t = tid; t < n_off; t += C::NW * 64) ((int*)lds)[t] = a.doc_offsets[t];
      __syncthreads();
    }
    if (!(doc_lds && a.doc_order && doc_order_tile<C::NW * 64, BN>(a, C::BM, (int*)lds, bh, qt)))
      decode_tile(a, blockIdx.x, bh, qt);
  }
  // (the work order read from LDS is uniform too)
  bh = __builtin_amdgcn_readfirstlane(bh);
  qt = __builtin_amdgcn_readfirstlane(qt);
  int b = bh / a.nh;  // the batch entry whose rows are in flight
  const int h = bh % a.nh, hk = h / a.group;
  const int q0 = qt * C::BM;
  const int qlast = min(q0 + C::BM, a.sq) - 1;

  // ---- positions of the rows ---------------------------------------------------
  // A row's position is its index, except in decode, where the packed row r
  // is new token r % S_new of its head at position len - S_new + r % S_new.
  int len = a.sk;
  if constexpr (C::DEC) len = min(max(a.seqlens[b], 0), a.max_len);
  auto pos_of = [&](int r) { return C::DEC ? len - a.sq_new + r % a.sq_new : r; };
  // smallest and largest position among rows r0..r1 (r0 <= r1)
  auto pos_range = [&](int r0, int r1, int& pmin, int& pmax) {
    if constexpr (C::DEC) {
      const int n = a.sq_new, i0 = r0 % n, i1 = r1 % n;
      const bool all = r1 - r0 + 1 >= n || i0 > i1;
      pmin = len - n + (all ? 0 : i0);
      pmax = len - n + (all ? n - 1 : i1);
    } else {
      pmin = r0;
      pmax = r1;
    }
  };
  // key interval of the query at position x (only the first len keys exist)
  auto interval = [&](int x, int& lo, int& hi) {
    if (doc_lds) {
      doc_run((const int*)lds + b * (a.n_docs + 1), a.n_docs, x, lo, hi);
      lo = max(lo, 0);
      hi = min(hi, a.sk - 1);
    } else {
      key_interval(a, b, x, lo, hi);
    }
    if constexpr (C::DEC) hi = min(hi, len - 1);
  };

  // ---- key-tile range of the work-group (union over its rows) -------------
  // Every interval kind has both ends non-decreasing in the position, so the
  // union over a set of rows runs from the smallest position's start to the
  // largest position's end.
  int p_first, p_last, lo_first, hi_first, lo_last, hi_last;
  pos_range(q0, qlast, p_first, p_last);
  interval(p_first, lo_first, hi_first);
  interval(p_last, lo_last, hi_last);
  int kt_lo = lo_first / BN;
  int kt_hi = hi_last >= lo_first ? (hi_last + BN) / BN : kt_lo;
  if constexpr (C::DEC) {
    // this work-group's share of the keys: its rows' key tiles cut into
    // n_split near-equal ranges, so every sequence's work spreads evenly over
    // its work-groups whatever its length
    const int per = (kt_hi - kt_lo + a.n_split - 1) / a.n_split;
    const int lo = kt_lo + split * per;
    kt_hi = min(lo + per, kt_hi);
    kt_lo = min(lo, kt_hi);
  }

  // ---- this wave's rows and their key intervals ----------------------------
  // cross-lane reads: walking launches use them inside their loop and keep
  // the plain forms
  auto xor32 = [&](float x) {
    if constexpr (C::PERSIST) return __shfl_xor(x, 32);
    else return lane_xor32(x);
  };
  auto read16 = [&](float x) {
    if constexpr (C::PERSIST) return __shfl(x, c & 15);
    else return lane_read16(x);
  };
  const int wq0 = q0 + wr * 32 * QB;
  // the same in a scalar register, for the epilogue (a vector copy would
  // stay live across the loop); walking launches keep the vector one, which
  // their loop uses anyway
  const int wq0_s = __builtin_amdgcn_readfirstlane(wq0);
  const int wq1 = min(wq0 + 32 * QB, a.sq) - 1;  // last valid row of the wave
  int wp_min, wp_max, w_lo_min, w_hi_min, w_lo_max, w_hi_max;
  pos_range(min(wq0, a.sq - 1), max(wq1, min(wq0, a.sq - 1)), wp_min, wp_max);
  interval(wp_min, w_lo_min, w_hi_min);
  interval(wp_max, w_lo_max, w_hi_max);
  const bool wave_idle = wq0 >= a.sq;

  // ---- Q operands in registers ---------------------------------------------
  // B operand of S^T = K Q^T: lane (c, g) holds Q[row c][16t + 8g .. +7].
  // Folded scores: Q is multiplied by the signed power-of-two part of
  // scale*log2(e) (exact), so S^T is the base-2 score over fold_m; bounded
  // softcap: by that part of the tanh argument 2*scale*log2(e)/cap, so S^T
  // is t / scap_m.
  bf16x8 qreg[NSU][QB][DQK / 16];
  // bounded softcap: tanh argument = scap_m * scap_q, scap_q a power of two
  // Both factors split as x = m * q with m in [0.5, 1) (so a larger S^T is
  // always a larger score) and q = +-2^e carrying the sign (a negative
  // scale flips Q exactly); a zero factor gives q = 0, m = 1.
  auto split_pow2 = [](float x, float& m, float& q) {
    int e = 0;
    const float f = frexpf(x, &e);
    m = x == 0.0f ? 1.0f : __builtin_fabsf(f);
    q = x == 0.0f ? 0.0f : __builtin_copysignf(ldexpf(1.0f, e), x);
  };
  float scap_m = 1.0f, scap_q = 1.0f;
  if constexpr (C::SCAPB) split_pow2(a.softcap_arg, scap_m, scap_q);
  // folded scores: scale*log2(e) = fold_m * fold_q, fold_q a signed power of
  // two.  Q takes fold_q (exact), so S^T, the folded terms and the running
  // reference are in units of 1/fold_m base-2 units; fold_m enters where
  // a term is exponentiated (one fused multiply-add per score).
  float fold_m = 1.0f, fold_q = 1.0f;
  if constexpr (C::FOLD) split_pow2(a.scale_log2, fold_m, fold_q);
  auto load_q = [&](int bb) {
#pragma unroll
    for (int s = 0; s < NSU; ++s) {
      // rows past S_q read as zeros through the bounds-checked resource
      const bf16* qh = (const bf16*)a.q[stream_of(s)] + bb * a.q_sb + h * a.q_sh;
      const int64_t q_row_b = a.q_si * 2;
      const int64_t q_span = (int64_t)(a.sq - 1) * q_row_b + DQK * 2 - (int64_t)wq0 * q_row_b;
      const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qh + (int64_t)wq0 * a.q_si, q_span);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t) {
          qreg[s][qb][t] = load16(qrs, (32 * qb + c) * (int)q_row_b + 32 * t + 16 * g);
          if constexpr (C::FOLD || C::SCAPB) {
            // folded: scale*log2(e); bounded softcap: the power-of-two part
            // of the tanh argument 2*scale*log2(e)/cap (exact in bf16; the
            // mantissa multiplies each score)
            const float qs = C::FOLD ? fold_q : scap_q;
            f32x8 f = __builtin_convertvector(qreg[s][qb][t], f32x8);
            qreg[s][qb][t] = __builtin_convertvector(f * qs, bf16x8);
          }
        }
      }
    }
  };
  load_q(b);

  // ---- global -> LDS tile movement ---------------------------------------------
  // K and V tiles go from global memory straight into LDS (buffer loads with
  // the LDS flag: no registers, no LDS store instructions), two tiles ahead of
  // the one being consumed.  Each (b, K/V head) block is addressed through a
  // bounds-checked buffer resource re-based at every tile, so keys past S_k
  // read as zeros.  One load instruction of a wave fills 1 KiB of LDS in lane
  // order, so the swizzled layout is realised by choosing, per lane, which
  // global 16-byte chunk to fetch.
  auto kblk = [&](int s, int bb) {
    return (const char*)((const bf16*)a.k[s] + bb * a.k_sb + hk * a.k_sh);
  };
  auto vblk = [&](int bb) { return (const char*)((const bf16*)a.v + bb * a.v_sb + hk * a.v_sh); };
  const int64_t k_row_b = a.k_si * 2, v_row_b = a.v_si * 2;
  // (decode: only the first len rows exist; cache slots past them may hold
  // anything, NaN included, and must not reach even a zero-weighted product)
  const int64_t k_span = len > 0 ? (int64_t)(len - 1) * k_row_b + DQK * 2 : 0;
  const int64_t v_span = len > 0 ? (int64_t)(len - 1) * v_row_b + DV * 2 : 0;

  int k_off[C::KCH], v_off[C::VCH];
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int q = (i * C::NW + w) * 64 + lane;  // 16-byte slot in the K tile
    const int row = q / C::KCPR, phys = q % C::KCPR;
    k_off[i] = row * (int)k_row_b + 16 * (phys ^ C::kswz(row));
  }
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int q = (i * C::NW + w) * 64 + lane;
    const int row = q / C::VCPR, phys = q % C::VCPR;
    v_off[i] = row * (int)v_row_b + 16 * (phys ^ C::vswz(row));
  }
  float kmpre = 0.0f;

  // issue the loads of tile kt of batch entry bb into LDS stage `stage`
  auto load_tile = [&](int bb, int kt, int stage) {
    const int64_t j0 = (int64_t)kt * BN;
    if (C::KMASK && tid < BN) {
      const int j = (int)j0 + tid;
      kmpre = (j < a.sk && (!a.kmask || a.kmask[bb * a.km_sb + (int64_t)j * a.km_sj] != 0))
                  ? 0.0f
                  : kNegInf;
    }
    bf16* ks = lds + stage * C::STAGE;
    // one resource over the whole (b, K/V head) block; the tile's offset
    // rides in the per-lane offset, which the launcher keeps below 2^31 for
    // every row up to 63 past S_k
    const int kt_off = (int)j0 * (int)k_row_b, vt_off = (int)j0 * (int)v_row_b;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(kblk(s, bb), k_span);
#pragma unroll
      for (int i = 0; i < C::KCH; ++i)
        lds_load16(rs, ks + s * C::K_ELEMS + (i * C::NW + w) * 512, k_off[i] + kt_off);
    }
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vblk(bb), v_span);
#pragma unroll
    for (int i = 0; i < C::VCH; ++i)
      lds_load16(rs, ks + NS * C::K_ELEMS + (i * C::NW + w) * 512, v_off[i] + vt_off);
  };
  // the key-mask column of a tile travels through a register
  auto store_kmask = [&](int stage) {
    if (C::KMASK && tid < BN) kmadd[stage * BN + tid] = kmpre;
  };

  constexpr int LOADS = NS * C::KCH + C::VCH;  // LDS-bound loads per thread per tile
  constexpr int AHEAD = C::STAGES - 1;          // tiles issued ahead of the one consumed
  // Tile order: ascending keys, except under ALiBi, where the visit starts
  // at the work-group's diagonal tile and wraps round.  The scores of a row
  // peak near its diagonal, so the running reference is set there first
  // instead of climbing (and being moved) tile after tile.
  const int n_kt = kt_hi - kt_lo;
  int kt_start = 0;
  if constexpr (C::MOD == MOD_ALIBI) kt_start = min(max(p_first / BN - kt_lo, 0), max(n_kt - 1, 0));
  auto tile_of = [&](int it) {
    const int x = it + kt_start;
    return kt_lo + (x >= n_kt ? x - n_kt : x);
  };
  // the visit: n_kt tiles of each of the n_rep batch entries, in sequence
  const int n_total = n_rep * n_kt;
  auto issue = [&](int it, int stage) {
    if constexpr (C::PERSIST)
      load_tile(b_first + it / n_kt, tile_of(it % n_kt), stage);
    else
      load_tile(b, tile_of(it), stage);
  };
  // The softcap pass runs against the reference c = cap log2(e): it is
  // tried for c <= 76, where rows of scores near 0 end far above its bound.
  const bool fast_try = !C::SCAPB || a.softcap_log2 <= 76.0f;

  // Folded first pass: Q and the first tiles go out as soon as the
  // work-group's key range is known, so that their latency runs under the
  // rest of the set-up.  (Under a document mask the offsets hold the LDS
  // until the set-up ends; its tiles go out after it.)
  bool pre_issued = false;
  if constexpr (C::FASTP) {
    if (fast_try && !doc_lds && n_total > 0) {
      issue(0, 0);
#pragma unroll
      for (int t = 1; t < AHEAD; ++t)
        if (t < n_total) issue(t, t);
      pre_issued = true;
    }
  }

  int row_lo[QB], row_w[QB];  // first key and number of keys (0: none) of each lane's row
  // positions of this lane's row and of the first and last row of each
  // 32-row block (the block's place against the diagonal)
  int lane_pos[QB], blk_pmin[QB], blk_pmax[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(wq0 + 32 * qb + c, a.sq - 1);  // rows past S_q copy the last row
    interval(pos_of(qi), row_lo[qb], row_w[qb]);   // first and last key
    row_w[qb] = max(row_w[qb] - row_lo[qb] + 1, 0);  // from here on: the number of keys
    if constexpr (C::DEC) {
      lane_pos[qb] = pos_of(qi);
      const int r0 = min(wq0 + 32 * qb, a.sq - 1);
      pos_range(r0, max(min(wq0 + 32 * qb + 31, a.sq - 1), r0), blk_pmin[qb], blk_pmax[qb]);
    } else {
      lane_pos[qb] = wq0 + 32 * qb + c;
      blk_pmin[qb] = wq0 + 32 * qb;
      blk_pmax[qb] = wq0 + 32 * qb + 31;
      if constexpr (C::ALIBI_FOLD) {
        // wave-uniform: the per-unit diagonal tests become scalar compares
        blk_pmin[qb] = __builtin_amdgcn_readfirstlane(blk_pmin[qb]);
        blk_pmax[qb] = __builtin_amdgcn_readfirstlane(blk_pmax[qb]);
      }
    }
  }
  // the prologue's last read of the LDS offsets
  if (doc_lds) __syncthreads();



  // Gate rows of entry bb (rows q0.., DV values each) into gate buffer
  // `buf`, straight from global memory; rows past S_q read as zeros.  They
  // land while the entry's tiles compute: the tile waits retire them (loads
  // return in issue order), and the epilogue of an entry with fewer than two
  // tiles waits for them itself.
  auto issue_gate = [&](int bb, int buf) {
    if constexpr (C::GATE_LDS) {
      const int64_t g_row_b = a.o_si * 2;
      const bf16* gb = (const bf16*)a.gate + bb * a.o_sb + h * a.o_sh + (int64_t)q0 * a.o_si;
      const __amdgpu_buffer_rsrc_t grs =
          make_rsrc(gb, (int64_t)(a.sq - 1 - q0) * g_row_b + DV * 2);
#pragma unroll
      for (int i = 0; i < C::GCH; ++i) {
        const int q = (i * C::NW + w) * 64 + lane;  // 16-byte slot: row q / (DV/8)
        lds_load16(grs, gbuf + buf * C::G_ELEMS + (i * C::NW + w) * 512,
                   (q / (DV / 8)) * (int)g_row_b + 16 * (q % (DV / 8)));
      }
    }
  };
  issue_gate(b, 0);

  // ---- per-row softmax state -------------------------------------------------
  f32x16 oacc[NSU][QB][DV / 32];
  // Bounded softcap: the row sums go through the matrix cores (the path is
  // vector-bound and never needs a unit's sum on its own).  A 16x16x32
  // product with a 0/1 selector as A adds each query's 32 rounded terms of a
  // unit: lane l supplies selector row l % 16 over k-group l / 16, and the
  // B operand (P^T of the unit) puts query n's terms in k-groups 0 and 2 and
  // query n + 16's in k-groups 1 and 3 of column n; rows 0 and 1 of the
  // 16x16 accumulator (registers 0 and 1 of lanes 0..15) collect them.
  f32x4 lacc[NSU][QB];
  bf16x8 lsel = {};
  if constexpr (C::SCAPB || C::FASTP) {
    const int m = lane & 15, kgrp = lane >> 4;
    const bf16 v = (bf16)((m == 0 && (kgrp & 1) == 0) || (m == 1 && (kgrp & 1) == 1) ? 1.0f : 0.0f);
    lsel = bf16x8{v, v, v, v, v, v, v, v};
  }
  float m_run[NSU][QB], l_run[NSU][QB];
  bool m_set[NSU][QB];
  // Folded scores: one more k-step of the S^T product adds the terms of the
  // score that are not q.k.  Only lane half 0 (k-slots 0..7) carries them;
  // half 1 of the key-side operand is zero.  For the tile at key j0, key
  // j = j0 + ck (ck = 32kb + row of the key half) and sigma = +1 on key
  // blocks wholly at or below the diagonal (j <= i), -1 wholly above:
  //   k-slot  0      A = 1    B = -m                     (m kept bf16-exact)
  //   k-slots 1..3   A = 1    B = -sigma*slope*(i - j0)  (3 bf16 parts)
  //   k-slots 4..6   A = ck   B = sigma*slope            (3 parts)
  // so S = q.k*scale*log2(e) - m - sigma*slope*(i - j), slope in base-2
  // units: the running reference and the ALiBi distance penalty.  Each
  // product is exact (ck < 64 is exact in bf16; three bf16 parts carry an
  // fp32 value), so p = 2^S needs no vector arithmetic before the
  // exponential.  The row term is rebuilt once per tile; sigma = -1 flips
  // the sign bits of slots 1..6.  Blocks that straddle the diagonal take
  // sigma = +1 and a vector correction for j > i.  Plain scores use slot 0.
  bf16x8 qext[NSU][QB];
  // Wave-uniform: some row of the wave has a reference m != 0, so S^T needs
  // the folded step (always under ALiBi, whose penalty rides on it).
  bool need_fold = C::ALIBI_FOLD;
  const bf16 one = (bf16)1.0f, zero = (bf16)0.0f;
  auto split3 = [](float x, bf16& hi, bf16& mid, bf16& lo) {
    hi = (bf16)x;
    mid = (bf16)(x - (float)hi);
    lo = (bf16)(x - (float)hi - (float)mid);
  };
  // decode rows of one K/V head belong to G query heads with their own slopes
  const int h_alibi = C::DEC ? hk * a.grp + min(wq0 + c, a.sq - 1) / a.sq_new : h;
  const float alibi_l2 = C::MOD == MOD_ALIBI ? alibi_slope_log2(a, h_alibi) : 0.0f;
  const float alibi_f = alibi_l2 / fold_m;  // the folded slope, in the units of S^T
  bf16 sl0, sl1, sl2;
  split3(alibi_f, sl0, sl1, sl2);
  // k-slots 4..7 of the query-side operand, the same in every lane: held in
  // scalar registers (decode rows of one wave may belong to several heads)
  uint32_t sl01 = __builtin_bit_cast(uint32_t, bf16x2{sl0, sl1});
  uint32_t sl2z = __builtin_bit_cast(uint32_t, bf16x2{sl2, zero});
  if constexpr (C::ALIBI_FOLD && !C::DEC) {
    sl01 = __builtin_amdgcn_readfirstlane(sl01);
    sl2z = __builtin_amdgcn_readfirstlane(sl2z);
  }
  // query-side operand for reference m (bf16-exact) and, under ALiBi, the
  // tile at j0
  auto set_qext = [&](int s, int qb, float m, int j0) {
    const bf16 mt = (bf16)(-m);
    if constexpr (C::ALIBI_FOLD) {
      bf16 x0, x1, x2;
      split3(-alibi_f * (float)(lane_pos[qb] - j0), x0, x1, x2);
      const u32x4 w4 = {__builtin_bit_cast(uint32_t, bf16x2{mt, x0}),
                        __builtin_bit_cast(uint32_t, bf16x2{x1, x2}), sl01, sl2z};
      qext[s][qb] = __builtin_bit_cast(bf16x8, w4);
    } else if constexpr (C::KMASK) {
      qext[s][qb] = bf16x8{mt, one, zero, zero, zero, zero, zero, zero};
    } else {
      qext[s][qb] = bf16x8{mt, zero, zero, zero, zero, zero, zero, zero};
    }
  };
  // key-side operand of key half kb.  With a key mask, k-slot 1 carries the
  // key's additive mask term (0, or -inf for an excluded key) against a
  // query-side 1, so excluded keys come out of the product at -inf.
  int cur_stage = 0;  // LDS stage of the tile being consumed
  auto kext = [&](int kb) {
    if constexpr (C::ALIBI_FOLD) {
      const bf16 ck = (bf16)(float)(32 * kb + c);
      return g == 0 ? bf16x8{one, one, one, one, ck, ck, ck, zero} : bf16x8{};
    } else if constexpr (C::KMASK) {
      const bf16 km = (bf16)kmadd[cur_stage * BN + 32 * kb + c];
      return g == 0 ? bf16x8{one, km, zero, zero, zero, zero, zero, zero} : bf16x8{};
    } else {
      return g == 0 ? bf16x8{one, zero, zero, zero, zero, zero, zero, zero} : bf16x8{};
    }
  };
  // sigma = -1: negate k-slots 1..6 of the query-side operand
  auto flip = [](bf16x8 x) {
    u32x4 w = __builtin_bit_cast(u32x4, x);
    w ^= (u32x4){0x80000000u, 0x80008000u, 0x80008000u, 0x00008000u};
    return __builtin_bit_cast(bf16x8, w);
  };
  auto reset_state = [&]() {
#pragma unroll
    for (int s = 0; s < NSU; ++s)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // folded: m = 0 is a valid reference from the start; it moves only
        // when terms overflow or a row's terms underflow
        m_run[s][qb] = (C::FOLD || C::SCAPB) ? 0.0f : kNegInf;
        m_set[s][qb] = false;
        l_run[s][qb] = 0.0f;
        lacc[s][qb] = f32x4{};
        qext[s][qb] = bf16x8{};
        if constexpr (C::FOLD) set_qext(s, qb, 0.0f, 0);
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) oacc[s][qb][db] = f32x16{};
      }
  };
  reset_state();

  // Scores live in base 2.  Modified scores are converted to base-2 units
  // after the product and use a lazy rescale: the running max used in the
  // exponent only moves when a score exceeds it by more than 8, so p <= 256
  // and most tiles skip the accumulator rescale.  Exact: numerator and
  // denominator share the reference.
  const float thr = 8.0f;


  // LDS element offsets of this lane's operand reads.  K: row 32kb + c,
  // logical 16-byte chunk 2t + g.
  int k_rd[DQK / 16];
#pragma unroll
  for (int t = 0; t < DQK / 16; ++t) k_rd[t] = c * DQK + 8 * ((2 * t + g) ^ C::kswz(c));  // + 32kb*DQK
  // Transposed V read: lane i of each 16-lane block points at row i/4 of a
  // 4-key group and 4 d-columns 4*(i%4) of the block's 16 columns.  The row
  // index mod 4 fixes the swizzle, so it is the same for every 4-key group.
  const int v_row = 4 * g + ((c & 15) >> 2);
  int v_rd[DV / 32];
#pragma unroll
  for (int db = 0; db < DV / 32; ++db) {
    const int d = 32 * db + 16 * (c >> 4) + 4 * (c & 3);
    v_rd[db] = v_row * DV + 8 * ((d >> 3) ^ C::vswz(v_row)) + (d & 7);  // + 16st*DV (+ 8*DV)
  }

  // ---- one key tile: S^T, softmax update, O^T += V^T P^T ---------------------
  // Work units u = (stream s, 32-key half kb, query block qb) run as a
  // three-stage pipeline: while the vector ALUs take the softmax of unit u,
  // the matrix cores run the S^T product of unit u+1 and the P.V product of
  // unit u-1, neither of which depends on it.  (P.V of u-1 is accumulated
  // before u's softmax may rescale the same rows' accumulator.)  The running
  // reference of a row never needs a tile-wide maximum, so the two key halves
  // of a tile are independent units.
  bf16x8 kop[DQK / 16];  // K operands of the current (stream, key half)
  auto read_k = [&](const bf16* ks, int s, int kb) {
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t)
      kop[t] = *(const bf16x8*)(ks + stream_of(s) * C::K_ELEMS + k_rd[t] + 32 * kb * DQK);
  };
  // position of a (key half, query block) unit against the diagonal
  // (wave-uniform): keys wholly above the rows' diagonal, or straddling it
  auto above = [&](int j0, int kb, int qb) { return j0 + 32 * kb >= blk_pmax[qb]; };
  auto straddles = [&](int j0, int kb, int qb) {
    return !above(j0, kb, qb) && j0 + 32 * kb + 31 > blk_pmin[qb];
  };
  // the folded k-step: -m, and the ALiBi penalty with the unit's sign
  auto fold = [&](int j0, int s, int kb, int qb, f32x16& acc) {
    const bf16x8 bq = C::ALIBI_FOLD && above(j0, kb, qb) ? flip(qext[s][qb]) : qext[s][qb];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kext(kb), bq, acc, 0, 0, 0);
  };
  // ALiBi on a straddling unit: the sign was +1, so keys past the row got
  // +slope*(j - i); subtract twice that
  auto alibi_fix = [&](int j0, f32x16& acc, int kb, int qb) {
    if constexpr (C::ALIBI_FOLD) {
      if (straddles(j0, kb, qb)) {
        const int qi = lane_pos[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dj = j0 + 32 * kb + 4 * g + acc_row(r) - qi;
          acc[r] = dj > 0 ? acc[r] - 2.0f * alibi_f * (float)dj : acc[r];
        }
      }
    }
  };
  auto qk = [&](int j0, int s, int kb, int qb, f32x16& acc, auto folded_tag) {
    acc = f32x16{};
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[t], qreg[s][qb][t], acc, 0, 0, 0);
    if constexpr (C::FOLD && decltype(folded_tag)::value) fold(j0, s, kb, qb, acc);
  };

  const float scap_k = C::SCAPB ? 0.5f / a.softcap_log2 : 0.0f;  // 1 / (2c)
  // Consume tile kt from LDS stage `stage`.  Folded scores: FOLDED adds the
  // extra k-step to every S^T product; without it the tile assumes that
  // every row of the wave still has the reference m = 0 (see need_fold).
  auto compute_tile = [&](int stage, int kt, auto masked_tag, auto folded_tag, auto fast_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool FOLDED = decltype(folded_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value;
    constexpr int U = NSU * 2 * QB;
    cur_stage = stage;
    const bf16* ks = lds + stage * C::STAGE;
    const int j0 = kt * BN;

    // V^T operands of one key half (A operands of the P.V products): lane
    // (c, g) holds V^T[d = 32db + c][keys 16st + 4g + 0..3, 16st + 8 + 4g +
    // 0..3] for the 16-key step st = 2kb + h2, from two transposed reads.
    u32x2 vraw[DV / 32 * 4];  // [db][h2][half]
    bf16x8 vop[DV / 32][2];   // [db][h2]
    const uint32_t vbase = lds_addr(ks + NS * C::K_ELEMS);
    // rows v_row + 8i (+ 32 for the second key half) of the V tile
    auto read_v = [&](int kb) {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vraw[4 * db + i] = ds_read_tr(vbase + 2 * v_rd[db] + 2 * (8 * i + 32 * kb) * DV);
    };
    auto take_v = [&]() {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x2 lo = vraw[4 * db + 2 * h2], hi = vraw[4 * db + 2 * h2 + 1];
          vop[db][h2] = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
        }
    };
    read_v(0);

    // One unsigned compare per score: key j is allowed when j - lo, as an
    // unsigned number, is below the row's width (lo >= 0 and the last key
    // <= S_k - 1, so nothing overflows); the offset of register 0 is formed
    // once per unit.
    auto mask = [&](f32x16& acc, int kb, int qb) {
      const int base = j0 + 32 * kb + 4 * g - row_lo[qb];
      const unsigned width = (unsigned)row_w[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[r] = (unsigned)(base + acc_row(r)) < width ? acc[r] : kNegInf;
    };
    // p = 2^(x - shift) of a unit's 16 scores (folded scores: x and shift
    // in the units of S^T, 2^(fold_m (x - shift))), rounded to bf16 in the
    // B-operand order of the P.V product (16-key steps 2kb and 2kb+1);
    // returns this lane's sum of the rounded values.
    auto exp_pack = [&](const f32x16& x, bf16x8 (&pk)[2], float shift) {
      float part[2] = {0.0f, 0.0f};  // two partial sums keep the add chain short
      const float fshift = shift * fold_m;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = fast_exp2(C::FOLD ? fmaf(x[8 * h2 + e], fold_m, -fshift) : x[8 * h2 + e] - shift);
        pk[h2] = __builtin_convertvector(p, bf16x8);
        if constexpr (C::SCAPB || FAST) continue;  // summed by the matrix cores
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pr = {pk[h2][e], pk[h2][e + 1]};
          const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
          part[h2] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, part[h2], false);
        }
      }
      return part[0] + part[1];
    };

    if constexpr (C::ALIBI_FOLD) {
#pragma unroll
      for (int s = 0; s < NSU; ++s)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) set_qext(s, qb, m_run[s][qb], j0);
    }
    f32x16 sacc[2];  // [pipeline slot]
    bf16x8 pkp[2];  // P of the previous unit, whose P.V product is still to come
    auto pv = [&](int s, int qb, const bf16x8 (&p)[2]) {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          oacc[s][qb][db] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db][h2], p[h2], oacc[s][qb][db], 0, 0, 0);
    };
    read_k(ks, 0, 0);
    qk(j0, 0, 0, 0, sacc[0], folded_tag);
    // unit u: key half kb = u / (NSU*QB), stream s = (u / QB) % NSU, block qb = u % QB
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = u / (NSU * QB), s = (u / QB) % NSU, qb = u % QB;
      if (u + 1 < U) {
        const int kb1 = (u + 1) / (NSU * QB), s1 = ((u + 1) / QB) % NSU, qb1 = (u + 1) % QB;
        if (qb1 == 0) read_k(ks, s1, kb1);
        qk(j0, s1, kb1, qb1, sacc[(u + 1) & 1], folded_tag);
      }
      // the previous unit's P.V product, independent of this unit's softmax
      if (u >= 1) {
        if ((u - 1) % (NSU * QB) == 0) take_v();
        pv(((u - 1) / QB) % NSU, (u - 1) % QB, pkp);
        if (u - 1 == NSU * QB - 1) read_v(1);
      }
      f32x16& sc = sacc[u & 1];
      const int qi = wq0 + 32 * qb + c;
      const int jb = j0 + 32 * kb + 4 * g;  // key of register 0 in this lane
      bf16x8 pk[2];

      if constexpr (C::SCAPB && FAST) {
        // first pass, reference c: 2^(score - c) = 2^(-2c / (2^t + 1)) lies in
        // (2^-2c, 1]; 1 / (2c) folds into one fused multiply-add before the
        // reciprocal, and the exponential takes the negation as a modifier
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[r] = -fast_rcp(fmaf(fast_exp2(sc[r] * scap_m), scap_k, scap_k));
        if constexpr (MASKED) mask(x, kb, qb);
        exp_pack(x, pk, 0.0f);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[0], lacc[s][qb], 0, 0, 0);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[1], lacc[s][qb], 0, 0, 0);
      } else if constexpr (C::SCAPB) {
        // With t = 2 y log2(e) for y = scale q.k / cap (S^T holds t / scap_m),
        // the softcapped base-2 score is cap log2(e) tanh(y) = c - 2c / (2^t + 1),
        // where c = cap log2(e) <= 100: the terms 2^score stay within fp32's
        // normal range with the fixed reference 0.
        const float c2 = a.softcap_log2;
        f32x16 x;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          x[r] = fmaf(fast_rcp(fast_exp2(sc[r] * scap_m) + 1.0f), -2.0f * c2, c2);
        if constexpr (MASKED) mask(x, kb, qb);
        exp_pack(x, pk, 0.0f);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[0], lacc[s][qb], 0, 0, 0);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[1], lacc[s][qb], 0, 0, 0);
      } else if constexpr (FAST) {
        // first pass: reference 0 throughout, rows summed by the matrix cores
        alibi_fix(j0, sc, kb, qb);
        if constexpr (MASKED) mask(sc, kb, qb);
        exp_pack(sc, pk, 0.0f);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[0], lacc[s][qb], 0, 0, 0);
        lacc[s][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pk[1], lacc[s][qb], 0, 0, 0);
      } else if constexpr (C::FOLD) {
        // S^T already holds (score - m) in base 2.
        alibi_fix(j0, sc, kb, qb);
        if constexpr (MASKED) mask(sc, kb, qb);
        float lsum = exp_pack(sc, pk, 0.0f);
        // The reference m is revisited only when the unit's terms grew past
        // 2^64 (inf included), or when a row that has allowed keys here has
        // no mass at all yet (its terms underflowed): then both halves of the
        // row agree on a new reference, the accumulator is rescaled and the
        // scores are recomputed and re-exponentiated.  In a tile without the
        // folded step, every unit after a reference moved is recomputed the
        // same way.  Wave-uniform, rarely taken.
        // (Every row has all keys of a full tile.  Bitwise operators keep the
        // test in vector compares, without divergent control flow.)
        bool has_key = true;
        if constexpr (MASKED)
          has_key = (row_lo[qb] + row_w[qb] - 1 >= j0 + 32 * kb) & (row_lo[qb] <= j0 + 32 * kb + 31) &
                    (row_w[qb] > 0);
        const bool redo = (has_key & (l_run[s][qb] + lsum == 0.0f)) | !(lsum <= 0x1p64f);
        interleave_hint();
        if (__builtin_amdgcn_ballot_w64(redo) || (!FOLDED && need_fold)) {
          f32x16 rs = f32x16{};
#pragma unroll
          for (int t = 0; t < DQK / 16; ++t) {
            const bf16x8 ka = *(const bf16x8*)(ks + stream_of(s) * C::K_ELEMS + k_rd[t] + 32 * kb * DQK);
            rs = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[s][qb][t], rs, 0, 0, 0);
          }
          fold(j0, s, kb, qb, rs);
          alibi_fix(j0, rs, kb, qb);
          if constexpr (MASKED) mask(rs, kb, qb);
          float xm = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r) xm = fmaxf(xm, rs[r]);
          xm = fmaxf(xm, xor32(xm));
          // move when the row maximum passes 32 units of S^T (terms of 2^16
          // to 2^32), or when the row (both lane halves, this unit included)
          // has no mass and its maximum is below -32 units; both halves of a
          // row decide alike
          const float lr = l_run[s][qb] + lsum;
          const float l_row = lr + xor32(lr);
          const bool move = xm != kNegInf && (xm > 32.0f || (l_row == 0.0f && xm < -32.0f));
          // the new reference is the row maximum rounded to bf16, so that
          // one k-slot carries it exactly
          const float m_new = move ? (float)(bf16)(m_run[s][qb] + xm) : m_run[s][qb];
          const float shift = m_new - m_run[s][qb];
          // (a row without mass has nothing to rescale; moving its reference
          // down could overflow the factor)
          const float alpha = !move ? 1.0f : (l_run[s][qb] == 0.0f ? 0.0f : fast_exp2(-shift * fold_m));
          l_run[s][qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DV / 32; ++db) oacc[s][qb][db] *= alpha;
          m_run[s][qb] = m_new;
          set_qext(s, qb, m_run[s][qb], j0);
          if (__builtin_amdgcn_ballot_w64(m_run[s][qb] != 0.0f)) need_fold = true;
          // the next unit's scores, already issued, may belong to the same rows
          if (u + 1 < U && (u + 1) % QB == qb && ((u + 1) / QB) % NSU == s) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[(u + 1) & 1][r] -= shift;
          }
          lsum = exp_pack(rs, pk, shift);
        }
        l_run[s][qb] += lsum;
      } else {
        // score modification, bias, key mask, positional mask
        float bias_v[16];
        if constexpr (C::BIAS) {
          // Two 16-byte loads per lane (keys 16r + 8g .. +7 of the unit's 32)
          // and a swap of half of each with the lane 32 apart give every lane
          // its keys 4g + 8 r4 + 0..3 (the accumulator layout).
          const int qi_c = min(qi, a.sq - 1);
          const bf16* bp = (const bf16*)a.bias + h * a.bias_sh + (int64_t)qi_c * a.bias_si;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int j = j0 + 32 * kb + 16 * r + 8 * g;  // S_k % 8 == 0: whole chunk or none
            u32x4 raw = {};
            if (!MASKED || j < a.sk) raw = *(const u32x4*)(bp + j);
            const auto s0 = __builtin_amdgcn_permlane32_swap(raw[0], raw[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(raw[1], raw[3], false, false);
            const bf16x4 lo = __builtin_bit_cast(bf16x4, u32x2{s0[0], s1[0]});  // r4 = 2r
            const bf16x4 hi = __builtin_bit_cast(bf16x4, u32x2{s0[1], s1[1]});  // r4 = 2r + 1
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bias_v[8 * r + e] = (float)lo[e] * kLog2e;
              bias_v[8 * r + 4 + e] = (float)hi[e] * kLog2e;
            }
          }
        }
        float km_v[16];
        if constexpr (C::KMASK) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 kv = *(const f32x4*)(kmadd + stage * BN + 32 * kb + 4 * g + 8 * r4);
#pragma unroll
            for (int e = 0; e < 4; ++e) km_v[4 * r4 + e] = kv[e];
          }
        }
        float xm = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[r];
          if constexpr (C::MOD == MOD_ALIBI) {
            const float dist = (float)(lane_pos[qb] - jb - acc_row(r));
            x = x * a.scale_log2 - alibi_l2 * __builtin_fabsf(dist);
          } else if constexpr (C::MOD == MOD_SOFTCAP) {
            x = softcap_log2(a, x);
          } else {
            x = x * a.scale_log2;
          }
          if constexpr (C::BIAS) x += bias_v[r];
          if constexpr (C::KMASK) x += km_v[r];
          sc[r] = x;
        }
        if constexpr (MASKED) mask(sc, kb, qb);
#pragma unroll
        for (int r = 0; r < 16; ++r) xm = fmaxf(xm, sc[r]);
        // xm covers this lane's half of the row's keys; the other half sits
        // in the lane 32 apart.  Both lanes of a row must use the same
        // reference, so the halves are combined only when some lane of the
        // wave would move it (wave-uniform, rarely taken).
        const float m_old = m_run[s][qb];
        interleave_hint();
        if (__builtin_amdgcn_ballot_w64(xm > m_old + thr)) {
          const float xf = fmaxf(xm, xor32(xm));
          const bool move = xf > m_old + thr;
          const float m_new = move ? xf : m_old;
          const float alpha = !move ? 1.0f : (m_old == kNegInf ? 0.0f : fast_exp2(m_old - m_new));
          l_run[s][qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DV / 32; ++db) oacc[s][qb][db] *= alpha;
          m_run[s][qb] = m_new;
        }
        const float shift = m_run[s][qb] == kNegInf ? 0.0f : m_run[s][qb];
        l_run[s][qb] += exp_pack(sc, pk, shift);
      }

      // O^T += V^T P^T over this unit's 32 keys; the V^T operands of a key
      // half are taken at its first unit and the second half's reads are
      // issued after the first half's last product.
      pkp[0] = pk[0];
      pkp[1] = pk[1];
      if constexpr (C::SCAPB) unit_hint_scapb();
      else if constexpr (FAST && C::FOLD && !C::ALIBI_FOLD && NS == 1) unit_hint_fast();
    }
    if ((U - 1) % (NSU * QB) == 0) take_v();
    pv(((U - 1) / QB) % NSU, (U - 1) % QB, pkp);
  };

  // ---- main loop ---------------------------------------------------------------
  // The it-th tile visited is consumed from stage it % STAGES while the
  // next AHEAD - 1 have landed or are in flight; the tile AHEAD places on
  // goes into the stage freed at the end of the previous iteration.  The
  // barrier at the end of an iteration both publishes the next tile (every
  // wave waited for its own loads) and frees the current stage.
  static_assert((AHEAD - 1) * LOADS < 64, "vmcnt range");
  // Publish a landed tile: wait for this wave's loads of it (leaving the
  // `newer` tiles issued after it in flight) and its LDS stores, then the
  // work-group barrier.  Written out because __syncthreads() also waits for
  // the tiles still in flight.  The memory clobber keeps the compiler from
  // moving memory accesses across it.
  auto sync_tile = [&](int newer) {
    if constexpr (AHEAD >= 5) {
      if (newer >= 4) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(4 * LOADS) : "memory");
        return;
      }
    }
    if constexpr (AHEAD >= 4) {
      if (newer >= 3) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * LOADS) : "memory");
        return;
      }
    }
    if constexpr (AHEAD >= 3) {
      if (newer >= 2) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS) : "memory");
        return;
      }
    }
    if (newer >= 1) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS) : "memory");
      return;
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // normalise, combine, gate and store the rows of batch entry b
  // the full row sum of this lane's row (both lane halves)
  bool fast_ok = false;  // the first pass stands (its sums are in lacc)
  auto row_sum = [&](int s, int qb) {
    if (C::SCAPB || (C::FASTP && fast_ok)) {
      const float l0 = read16(lacc[s][qb][0]);
      const float l1 = read16(lacc[s][qb][1]);
      return c < 16 ? l0 : l1;
    } else {
      return l_run[s][qb] + xor32(l_run[s][qb]);
    }
  };
  auto finish_row = [&](bool gate_wait) {
    if constexpr (C::GATE_LDS) {
      if (gate_wait) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      (void)gate_wait;
    }
    // the lane's row and half and the wave's first row, formed again here:
    // kept from the prologue, the values derived from them stay live (or
    // spilled) across the loop (walking launches finish rows inside their
    // loop and use the prologue's)
    const int lane_f = C::PERSIST ? lane : lane_here();
    const int cf = C::PERSIST ? c : lane_f & 31, gf = C::PERSIST ? g : lane_f >> 5;
    const int wq0f = C::PERSIST ? wq0 : wq0_s;
    float inv[NSU][QB];
  #pragma unroll
    for (int s = 0; s < NSU; ++s)
  #pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float l = row_sum(s, qb);
        inv[s][qb] = l > 0.0f ? 1.0f / l : 0.0f;
        const int qi = wq0f + 32 * qb + cf;
        float* lse_out = a.lse[stream_of(s)];
        if (lse_out && gf == 0 && qi < a.sq) {
          const float m = m_run[s][qb] * fold_m;  // base-2 units
          const float lse = l > 0.0f ? (m + __builtin_log2f(l)) * kLn2 : kNegInf;
          lse_out[b * a.lse_sb + h * a.lse_sh + qi] = lse;
        }
      }

    // Split streams: the stream-1 waves hand their normalised rows through
    // LDS (row-major, rows padded by 4 floats) to the stream-0 wave of the
    // same rows, which stores O1/l1 - lambda O2/l2.  Both barriers are met by
    // every wave; the first frees the K/V stages.
    constexpr int XS = DV + 4;
    float* xo = (float*)lds;
    if constexpr (C::SPLIT) {
      static_assert(C::BM * XS * 4 <= C::STAGES * C::STAGE * 2, "combine buffer");
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (ws == 1) {
  #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float* xr = xo + (wr * 32 * QB + 32 * qb + cf) * XS;
  #pragma unroll
          for (int db = 0; db < DV / 32; ++db)
  #pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 v = {oacc[0][qb][db][4 * r4] * inv[0][qb], oacc[0][qb][db][4 * r4 + 1] * inv[0][qb],
                               oacc[0][qb][db][4 * r4 + 2] * inv[0][qb], oacc[0][qb][db][4 * r4 + 3] * inv[0][qb]};
              *(f32x4*)(xr + 32 * db + 8 * r4 + 4 * gf) = v;
            }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (ws == 1) return;
    }

  #pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = wq0f + 32 * qb + cf;
      if (qi >= a.sq) continue;
      bf16* op = (bf16*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si;
      const bf16* gp = !C::GATE ? nullptr
                       : C::GATE_LDS
                           ? gbuf + ((b - b_first) & 1) * C::G_ELEMS + (wq0f - q0 + 32 * qb + cf) * DV
                           : (const bf16*)a.gate + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si;
      const float* xr = xo + (wr * 32 * QB + 32 * qb + cf) * XS;
  // A lane holds dims 8 r4 + 4g + 0..3 of its row; pairs (r4 = 2r, 2r + 1)
  // trade halves with the lane 32 apart (the same row) so that each lane
  // moves 16 contiguous bytes (dims 16r + 8g .. +7) per global access.
  #pragma unroll
      for (int db = 0; db < DV / 32; ++db)
  #pragma unroll
        for (int r = 0; r < 2; ++r) {
          bf16x4 gvv[2];
          if constexpr (C::GATE && !C::GATE_LDS) {
            const u32x4 raw = *(const u32x4*)(gp + 32 * db + 16 * r + 8 * gf);
            const auto s0 = __builtin_amdgcn_permlane32_swap(raw[0], raw[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(raw[1], raw[3], false, false);
            gvv[0] = __builtin_bit_cast(bf16x4, u32x2{s0[0], s1[0]});
            gvv[1] = __builtin_bit_cast(bf16x4, u32x2{s0[1], s1[1]});
          }
          u32x2 packed[2];
  #pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r4 = 2 * r + hh;
            const int d = 32 * db + 8 * r4 + 4 * gf;
            float ov[4];
  #pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = oacc[0][qb][db][4 * r4 + e] * inv[0][qb];
            if constexpr (C::SPLIT) {
              const f32x4 o2 = *(const f32x4*)(xr + d);
  #pragma unroll
              for (int e = 0; e < 4; ++e) ov[e] -= a.lambda * o2[e];
            }
            if constexpr (C::GATE) {
              const bf16x4 gv = C::GATE_LDS ? *(const bf16x4*)(gp + d) : gvv[hh];
  #pragma unroll
              for (int e = 0; e < 4; ++e) ov[e] *= sigmoid((float)gv[e]);
            }
            const bf16x4 out = {(bf16)ov[0], (bf16)ov[1], (bf16)ov[2], (bf16)ov[3]};
            packed[hh] = __builtin_bit_cast(u32x2, out);
          }
          const auto t0 = __builtin_amdgcn_permlane32_swap(packed[0][0], packed[1][0], false, false);
          const auto t1 = __builtin_amdgcn_permlane32_swap(packed[0][1], packed[1][1], false, false);
          *(u32x4*)(op + 32 * db + 16 * r + 8 * gf) = u32x4{t0[0], t1[0], t0[1], t1[1]};
        }
    }
  };
  if constexpr (C::FASTP) if (fast_try) {
    using F = std::integral_constant<bool, false>;
    using T = std::integral_constant<bool, true>;
    using FD = std::integral_constant<bool, C::ALIBI_FOLD>;  // the penalty rides on the fold
    if (n_total > 0) {
      if (!pre_issued) {
        issue(0, 0);
#pragma unroll
        for (int t = 1; t < AHEAD; ++t)
          if (t < n_total) issue(t, t);
      }
      sync_tile(min(AHEAD, n_total) - 1);
    }
    for (int it = 0; it < n_total; ++it) {
      const int kt = tile_of(it);
      const int stage = it % C::STAGES;
      const int j0 = kt * BN, j1 = j0 + BN - 1;
      const bool empty = wave_idle || j0 > w_hi_max || j1 < w_lo_min;
      const bool full = j0 >= w_lo_max && j1 <= w_hi_min;
      if (it + AHEAD < n_total) issue(it + AHEAD, stage == 0 ? C::STAGES - 1 : stage - 1);
      if (!empty) {
        if (full)
          compute_tile(stage, kt, F{}, FD{}, T{});
        else
          compute_tile(stage, kt, T{}, FD{}, T{});
      }
      if (it + 1 < n_total) sync_tile(min(AHEAD - 1, n_total - 2 - it));
    }
    // Every row with allowed keys must end with a sum in [lo, 2^100]: then no
    // term overflowed, and the largest is at least lo / S_k, so the terms
    // below fp32's normal range (2^-126) that may have been lost hold at most
    // S_k 2^-126 / lo of the mass: under 2^-22 for S_k <= 2^24 with the
    // softcap's lo = 2^-80 (terms relative to 2^c), far less with 2^-64.
    constexpr float lo = C::SCAPB ? 0x1p-80f : 0x1p-64f;
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l0 = read16(lacc[0][qb][0]);
      const float l1 = read16(lacc[0][qb][1]);
      const float l = c < 16 ? l0 : l1;
      // rows past S_q (zero queries, under ALiBi possibly far below range)
      // produce no output and are left out
      const bool real = wq0 + 32 * qb + c < a.sq;
      const bool has = row_w[qb] > 0;
      bad |= real & ((has & !(l >= lo)) | !(l <= 0x1p100f));
    }
    __shared__ int pass_bad;
    // (every lane of the writing waves stores the same value, so no lane
    // index stays live across the tile loop for a single-lane store)
    if (w == 0) pass_bad = 0;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (__builtin_amdgcn_ballot_w64(bad)) pass_bad = 1;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    fast_ok = pass_bad == 0;
    if (!fast_ok) reset_state();
    if constexpr (C::SCAPB) {
      // the softcap pass ran against the reference c
      if (fast_ok)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m_run[0][qb] = a.softcap_log2;
    }
  }
  if (C::FASTP && fast_ok) {
    // the first pass stands
  } else if (n_total > 0) {
    // the key-mask column of a tile goes to LDS one step after its load
    // was issued; the prologue stores all but the newest
    issue(0, 0);
#pragma unroll
    for (int t = 1; t < AHEAD; ++t)
      if (t < n_total) {
        store_kmask(t - 1);
        issue(t, t);
      }
    // with fewer tiles than the pipeline holds, no iteration stores the last
    if (n_total < AHEAD) store_kmask(n_total - 1);
    sync_tile(min(AHEAD, n_total) - 1);
  }
  const int n_careful = C::FASTP && fast_ok ? 0 : n_total;  // tiles of the checked pass
  for (int it = 0; it < n_careful; ++it) {
    const int kt = C::PERSIST ? tile_of(it % n_kt) : tile_of(it);
    const int stage = it % C::STAGES;
    const bool next = it + 1 < n_total, next2 = it + AHEAD < n_total;
    const int j0 = kt * BN, j1 = j0 + BN - 1;
    const bool empty = wave_idle || j0 > w_hi_max || j1 < w_lo_min;
    const bool full = j0 >= w_lo_max && j1 <= w_hi_min;
    // the newest tile issued so far is it + AHEAD - 1 (if it exists)
    if (it + AHEAD - 1 < n_total) store_kmask((it + AHEAD - 1) % C::STAGES);
    if (next2) issue(it + AHEAD, stage == 0 ? C::STAGES - 1 : stage - 1);
    if (!empty) {
      using F = std::integral_constant<bool, false>;
      using T = std::integral_constant<bool, true>;
      if (!C::FOLD || C::ALIBI_FOLD || C::KMASK || need_fold) {
        if (full)
          compute_tile(stage, kt, F{}, T{}, F{});
        else
          compute_tile(stage, kt, T{}, T{}, F{});
      } else if constexpr (C::FOLD && !C::ALIBI_FOLD && !C::KMASK) {
        if (full)
          compute_tile(stage, kt, F{}, F{}, F{});
        else
          compute_tile(stage, kt, T{}, F{}, F{});
      }
    }
    bool boundary = false;
    if constexpr (C::PERSIST) {
      if (it % n_kt == n_kt - 1 && next) {
        // the entry's last tile: its rows are done; the next entry's first
        // tiles are already in flight.  Its Q and gate loads go out after
        // them, and the tile wait below leaves them outstanding too (loads
        // return in issue order).
        finish_row(n_kt < 2);
        ++b;
        reset_state();
        load_q(b);
        issue_gate(b, (b - b_first) & 1);
        boundary = true;
      }
    }
    if (next) {
      if constexpr (C::PERSIST) {
        static_assert(AHEAD == 2, "entry hand-over waits");
        constexpr int EXTRA = NSU * QB * (DQK / 16) + C::GCH;  // Q and gate loads of an entry
        static_assert(LOADS + EXTRA < 64, "vmcnt range");
        const int newer = min(AHEAD - 1, n_total - 2 - it);
        if (boundary) {
          if (newer >= 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS + EXTRA) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(EXTRA) : "memory");
        } else {
          sync_tile(newer);
        }
      } else {
        sync_tile(min(AHEAD - 1, n_total - 2 - it));
      }
    }
  }
  if constexpr (C::PERSIST) {
    // entries left without a tile (no key at all) still write their rows
    if (n_kt == 0) {
      for (int r = 1; r < n_rep; ++r) {
        finish_row(true);
        ++b;
        issue_gate(b, (b - b_first) & 1);
      }
    }
  }

  // ---- epilogue: normalise, combine, gate, store --------------------------------
  if constexpr (C::DEC) {
    if (a.n_split > 1) {
      // one key range of a split decode: normalised float32 output and
      // natural-log LSE of this range (0 and -inf when it held no key)
      const float l = row_sum(0, 0);
      const float iv = l > 0.0f ? 1.0f / l : 0.0f;
      const int qi = wq0 + c;
      if (qi < a.sq) {
        const int64_t prow = ((int64_t)(split * a.nb + b) * a.nh + h) * a.sq + qi;
        if (g == 0)
          a.lse_part[prow] = l > 0.0f ? (m_run[0][0] * fold_m + __builtin_log2f(l)) * kLn2 : kNegInf;
        float* op = a.o_part + prow * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * db + 8 * r4 + 4 * g;
            const f32x4 ov = {oacc[0][0][db][4 * r4] * iv, oacc[0][0][db][4 * r4 + 1] * iv,
                              oacc[0][0][db][4 * r4 + 2] * iv, oacc[0][0][db][4 * r4 + 3] * iv};
            *(f32x4*)(op + d) = ov;
          }
      }
      return;
    }
  }
  finish_row(!C::PERSIST || n_kt < 2);
}

}  // namespace fl
