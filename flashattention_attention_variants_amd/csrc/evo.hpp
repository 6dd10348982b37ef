// evo.hpp -- Evoformer gated attention over rows of at most 256 positions
// (bf16, C = 32) on gfx950 matrix cores.
//
// AlphaFold2's MSA attention (gist.science explainer of Flashlight,
// "Technical Summary: Problem Statement"; papers.lqhl.me wiki, "设计取舍":
// a bias broadcast over an extra dimension) takes a softmax over the 256
// residues of one MSA row (row form; the pair bias [H, N_res, N_res] is the
// same for every MSA row) or over the 128 sequences of one residue column
// (column form, no bias).  Rows this short fit a work-group whole: NKU waves
// hold the 32*NKU query rows of one (entry, head), and the work-group walks a
// run of entries (MSA rows or residue columns) of one head.  With the row
// form's bias, the bias stays in registers for the whole walk (two waves
// per SIMD); without a bias (the column form) the gate rows are read from
// memory in the epilogue instead of LDS, and the kernel runs three waves
// per SIMD (129 registers; at 128 positions three work-groups of four
// waves share a compute unit).  (Loading K and V two entries ahead through three
// LDS stages, the gate one entry ahead, did not help: a timestamp trace
// puts an entry at about 3.4 us of units and 3 us of load issue and
// barrier wait however the loads are placed.)
//
// Per entry, K, V, Q and (with a bias) the gate rows land in LDS by DMA
// while the entry before computes (two LDS stages, by entry parity); the
// keys' mask terms follow through registers.  A wave then computes, per 32-key unit,
//
//   S^T  = K (f Q)^T + c I Bias^T + ext     MFMA 32x32x16 bf16
//   p    = 2^(m S^T)                         one multiply, one exponential
//   O^T += V^T P^T                           P rounded to bf16
//
// with scale*log2(e) = m f, f a signed power of two (f Q is exact in bf16)
// and m in [0.5, 1): S^T is the base-2 score over m.  The pair bias goes
// through the matrix cores: the wave's 32 query rows x 32*NKU keys of its
// head's bias stay in registers for the whole launch as B operands of a
// product with c I, c = log2(e) / m in two bf16 parts (every product is
// exact, so the bias term keeps float32 accuracy).  ext is one more k-step:
// the key's mask term (0, or -inf for an excluded key or one past the row's
// end) against a query-side 1 and, in the checked pass, the running
// reference against a key-side 1.
//
// First pass: reference 0 and no running max, which rows of ordinary logits
// never need.  A wave with a row whose sum ends outside [2^-60, 2^100] (or
// is zero: no allowed key, or every term underflowed) recomputes its rows
// with a lazy running reference, moved only when a score passes it by more
// than 8 (so p <= 256), as the online softmax of the general kernel.
#pragma once

#include "attn_mfma.hpp"

namespace fl {

template <int NKU_, bool BIAS_>
struct EvoCfg {
  static constexpr int NKU = NKU_;  // 32-key units per row, and waves per work-group
  static constexpr bool BIAS = BIAS_;
  static constexpr int NW = NKU_;
  static constexpr int LP = 32 * NKU_;  // positions per entry, padded
  static constexpr int MAT = LP * 64;   // bytes of one [LP, 32] bf16 matrix
  // one LDS stage: K, V, Q, gate, then the keys' mask terms (bf16)
  // without a bias: the gate is read from memory in the epilogue, and three
  // waves per SIMD
  static constexpr bool GLDS = BIAS_;
  static constexpr int WPE = BIAS_ ? 2 : 3;
  static constexpr int K_OFF = 0, V_OFF = MAT, Q_OFF = 2 * MAT, G_OFF = 3 * MAT,
                       T_OFF = (GLDS ? 4 : 3) * MAT;
  static constexpr int STAGE = (GLDS ? 4 : 3) * MAT + 2 * LP;
  static_assert(NKU == 2 || NKU == 4 || NKU == 8, "row lengths");
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
};

// Logical 16-byte chunk p of row r of a swizzled LDS matrix sits at chunk
// p ^ evo_swz(r): the 16 rows that one 16-byte read serves in a cycle (one
// logical chunk each, 64-byte rows) then fall on distinct banks.
__device__ __forceinline__ constexpr int evo_swz(int r) { return (r >> 2) & 3; }

template <class C>
__global__ __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void evo_kernel(KernelArgs a) {
  constexpr int NKU = C::NKU, LP = C::LP;
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;
  const int L = a.sq;  // positions per entry: queries and keys
  // work-group -> (head, run of entries).  Work-group ids go to the 8 XCDs
  // in turn; units u = (run, head pair) take two consecutive slots of one
  // XCD, one per head of the pair, so that the two heads' 64-byte halves of
  // each 128-byte row of q, k, v and gate are fetched into one L2 (one head
  // per XCD fetched every line twice), and with 8 heads each XCD keeps one
  // head pair and its pair bias.  Ids past the last unit, and the missing
  // second head of an odd count, end at once.
  const int n_hp = (a.nh + 1) >> 1;
  const int slot = (int)(blockIdx.x >> 3), unit = (slot >> 1) * 8 + (int)(blockIdx.x & 7);
  const int h = 2 * (unit % n_hp) + (slot & 1);
  const int b_first = (unit / n_hp) * a.rows_per_wg;
  if (h >= a.nh || b_first >= a.nb) return;
  const int b_end = min(b_first + a.rows_per_wg, a.nb);
  const int qrow = 32 * w + c;  // this lane's query row
  const bool wave_busy = 32 * w < L;
  const bf16 zero = (bf16)0.0f, one = (bf16)1.0f;

  // scale*log2(e) = fold_m * fold_q (a zero scale gives fold_q = 0)
  float fold_m = 1.0f, fold_q = 0.0f;
  if (a.scale_log2 != 0.0f) {
    int e = 0;
    const float f = frexpf(a.scale_log2, &e);
    fold_m = __builtin_fabsf(f);
    fold_q = __builtin_copysignf(ldexpf(1.0f, e), a.scale_log2);
  }

  // c I in two bf16 parts, the A operands of the bias products of k-steps
  // t = 0, 1 (keys 16t + 0..15 of a unit): lane (c, g) holds row c over
  // k-slots 8g..8g+7, nonzero where 16t + 8g + slot = c.  B operands: the
  // bias rows of the lane's query, keys 32u + 16t + 8g .. +7 (16 bytes).
  bf16x8 idh[2], idl[2];
  bf16x8 bop[C::BIAS ? NKU : 1][2];
  if constexpr (C::BIAS) {
    const float cb = kLog2e / fold_m;
    const bf16 ch = (bf16)cb, cl = (bf16)(cb - (float)ch);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool on = c == 16 * t + 8 * g + e;
        idh[t][e] = on ? ch : zero;
        idl[t][e] = on ? cl : zero;
      }
  }
  // The bias rows, loaded once the first entry's loads are out.  Rows past
  // L copy row L - 1; keys past L read whatever follows (those keys are
  // excluded by their mask term).  They are taken at once, before the walk:
  // a first use inside the units would make the compiler wait there for
  // them, and with them (loads retire in order) for the next entry's loads
  // issued meanwhile.
  auto take_bias = [&]() {
    if constexpr (C::BIAS) {
      const bf16* bh = (const bf16*)a.bias + (int64_t)h * a.bias_sh;
      const __amdgpu_buffer_rsrc_t brs = make_rsrc(bh, ((int64_t)(L - 1) * a.bias_si + L) * 2);
      const int br = min(qrow, L - 1) * (int)a.bias_si;
#pragma unroll
      for (int u = 0; u < NKU; ++u)
#pragma unroll
        for (int t = 0; t < 2; ++t) bop[u][t] = load16(brs, (br + 32 * u + 16 * t + 8 * g) * 2);
#pragma unroll
      for (int u = 0; u < NKU; ++u)
#pragma unroll
        for (int t = 0; t < 2; ++t) asm volatile("" ::"v"(bop[u][t]));
    }
  };

  // ---- loads of one entry --------------------------------------------------
  // K, V, Q and gate rows of entry bb into LDS stage st, 16 bytes per lane
  // and instruction, lane-linear in LDS (the swizzle picks which global
  // chunk a lane fetches); rows past L read as zeros.  Then this thread's
  // key (tid < LP): kept unless past the row or excluded by the key mask.
  int mbyte = 1;  // the key-mask byte of this thread's key in the next entry
  auto issue = [&](int bb, int st) {
    char* sbase = lds + st * C::STAGE;
    auto dma = [&](const void* p, int64_t sb, int64_t sh, int64_t si, int off, bool swz) {
      const char* base = (const char*)p + 2 * ((int64_t)bb * sb + (int64_t)h * sh);
      const int row_b = (int)(2 * si);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (int64_t)(L - 1) * row_b + 64);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int blk = i * C::NW + w;  // 64 slots of 16 bytes
        const int sl = blk * 64 + lane;
        const int r = sl >> 2, p4 = sl & 3;
        lds_load16(rs, sbase + off + blk * 1024, r * row_b + 16 * (swz ? p4 ^ evo_swz(r) : p4));
      }
    };
    dma(a.k[0], a.k_sb, a.k_sh, a.k_si, C::K_OFF, true);
    dma(a.v, a.v_sb, a.v_sh, a.v_si, C::V_OFF, false);
    dma(a.q[0], a.q_sb, a.q_sh, a.q_si, C::Q_OFF, true);
    if constexpr (C::GLDS) dma(a.gate, a.o_sb, a.o_sh, a.o_si, C::G_OFF, true);
    // read raw and tested at the hand-over: a test here would wait for this
    // load, and so for the DMA loads above
    if (a.kmask) mbyte = a.kmask[(int64_t)bb * a.km_sb + (int64_t)min(tid, L - 1) * a.km_sj];
  };

  // ---- per-lane LDS offsets ----------------------------------------------------
  // K operand of k-step t for key row 32u + c (the swizzle of rows 32u + c
  // does not depend on u)
  int k_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) k_off[t] = C::K_OFF + c * 64 + 16 * ((2 * t + g) ^ evo_swz(c));
  // V^T operands by transposed reads: the 16-lane block (g, c / 16) reads
  // keys k0 + 0..3 (k0 = 32u + 16st + 8hf + 4g) x dims 16(c / 16) + 0..15;
  // lane i of the block points at key k0 + i / 4, dims + 4(i % 4) .. +3
  // and receives dim c of the four keys.  Rows are 64 bytes, so the 32
  // lanes served per cycle read four whole rows: no bank conflict.
  const int li = c & 15;
  const int v_off = C::V_OFF + (4 * g + (li >> 2)) * 64 + 2 * (16 * (c >> 4) + 4 * (li & 3));

  // ---- one entry -------------------------------------------------------------
  u32x4 pend[2];       // this lane's output (dims 16r + 8g .. +7), stored later
  char* pend_ptr = nullptr;

  auto compute = [&](int bb, const char* sb) {
    // Q operands (B of S^T): row qrow, dims 16t + 8g .. +7, times fold_q
    bf16x8 qop[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 raw = *(const bf16x8*)(sb + C::Q_OFF + qrow * 64 + 16 * ((2 * t + g) ^ evo_swz(qrow)));
      const f32x8 f = __builtin_convertvector(raw, f32x8);
      qop[t] = __builtin_convertvector(f * fold_q, bf16x8);
    }
    const bf16* kterm = (const bf16*)(sb + C::T_OFF);
    const uint32_t vbase = lds_addr(sb);

    // S^T of unit u against the query-side ext operand qx
    auto s_unit = [&](int u, const bf16x8& qx) {
      const bf16 km = kterm[32 * u + c];
      const bf16 k0 = g == 0 ? one : zero, k1 = g == 0 ? km : zero;
      const bf16x8 kx = {k0, k1, zero, zero, zero, zero, zero, zero};
      f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qx, f32x16{}, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 kop = *(const bf16x8*)(sb + k_off[t] + 2048 * u);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[t], acc, 0, 0, 0);
      }
      if constexpr (C::BIAS) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(idh[t], bop[u][t], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(idl[t], bop[u][t], acc, 0, 0, 0);
        }
      }
      return acc;
    };
    // p = 2^(fold_m x) rounded to bf16 in the B-operand order of the P.V
    // steps (register 8st + e holds key 16st + 8(e/4) + 4g + e%4), and the
    // sums of the rounded values
    auto p_unit = [&](const f32x16& x, bf16x8 (&pk)[2], float& l0, float& l1) {
      const bf16x2 ones = {one, one};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(x[8 * st + e] * fold_m);
        pk[st] = __builtin_convertvector(p, bf16x8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pk[st][e], pk[st][e + 1]};
          if (e & 2)
            l1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l1, false);
          else
            l0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l0, false);
        }
      }
    };
    f32x16 oacc = {};
    auto pv = [&](int u, const bf16x8 (&pk)[2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint32_t ad = vbase + v_off + (32 * u + 16 * st) * 64;
        const u32x2 lo = ds_read_tr(ad), hi = ds_read_tr(ad + 8 * 64);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
        oacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pk[st], oacc, 0, 0, 0);
      }
    };
    // (a lane-half swap with one value in both operands came out of the
    // compiler with both results equal, so the other half is read across)
    auto both_halves_sum = [](float x) { return x + lane_xor32(x); };

    // first pass: reference 0, the next unit's S^T beside this unit's
    // exponentials
    const bf16x8 qx0 = g == 0 ? bf16x8{zero, one, zero, zero, zero, zero, zero, zero} : bf16x8{};
    float l0 = 0.0f, l1 = 0.0f;
    {
      f32x16 x = s_unit(0, qx0);
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        // one unit per scheduling region: left free, the scheduler hoists
        // later units' operand reads and runs out of registers
        __builtin_amdgcn_sched_barrier(0);
        f32x16 xn;
        if (u + 1 < NKU) xn = s_unit(u + 1, qx0);
        bf16x8 pk[2];
        p_unit(x, pk, l0, l1);
        // the sums in their unit (left free, they sink to the end of the
        // pass and keep every unit's P in registers)
        asm volatile("" : "+v"(l0), "+v"(l1));
        pv(u, pk);
        if (u + 1 < NKU) x = xn;
      }
    }
    float lt = both_halves_sum(l0 + l1);
    const bool bad = qrow < L && !(lt >= 0x1p-60f && lt <= 0x1p100f);
    if (__builtin_amdgcn_ballot_w64(bad)) {
      // checked pass over the wave's rows: reference mref (bf16-exact, in
      // S^T units) moved to a unit's max when the max passes it by more
      // than 8 / fold_m, or at the row's first allowed keys
      oacc = f32x16{};
      float ls = 0.0f, mref = 0.0f;
      bool mset = false;
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        const bf16x8 qx = g == 0 ? bf16x8{(bf16)(-mref), one, zero, zero, zero, zero, zero, zero} : bf16x8{};
        f32x16 x = s_unit(u, qx);
        float mx = x[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
        mx = fmaxf(mx, lane_xor32(mx));
        const bool grow = mx > kNegInf && (!mset || mx * fold_m > 8.0f);
        if (__builtin_amdgcn_ballot_w64(grow)) {
          if (grow) {
            const float nref = (float)(bf16)(mref + mx);
            const float d = nref - mref;
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] -= d;
            const float al = mset ? fast_exp2(-d * fold_m) : 0.0f;
            oacc *= al;
            ls *= al;
            mref = nref;
            mset = true;
          }
        }
        bf16x8 pk[2];
        float a0 = 0.0f, a1 = 0.0f;
        p_unit(x, pk, a0, a1);
        ls += a0 + a1;
        pv(u, pk);
      }
      lt = both_halves_sum(ls);
    }

    // epilogue: O / l (0 for a row with no allowed key), gated; the lane
    // holds dims 8 r4 + 4g + 0..3 of its row, and pairs (r4 = 2r, 2r + 1)
    // trade halves with the lane 32 apart so that each lane then holds the
    // 16 contiguous bytes of dims 16r + 8g .. +7
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const char* grow_p = sb + C::G_OFF + qrow * 64;
    const bf16* gmem = (const bf16*)a.gate + (int64_t)bb * a.o_sb + (int64_t)h * a.o_sh +
                       (int64_t)min(qrow, L - 1) * a.o_si;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      u32x2 packed[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r4 = 2 * r + hh;
        const bf16x4 gv = C::GLDS ? *(const bf16x4*)(grow_p + 16 * (r4 ^ evo_swz(qrow)) + 8 * g)
                                  : *(const bf16x4*)(gmem + 8 * r4 + 4 * g);
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = oacc[4 * r4 + e] * inv * sigmoid((float)gv[e]);
        const bf16x4 out = {(bf16)ov[0], (bf16)ov[1], (bf16)ov[2], (bf16)ov[3]};
        packed[hh] = __builtin_bit_cast(u32x2, out);
      }
      const auto t0 = __builtin_amdgcn_permlane32_swap(packed[0][0], packed[1][0], false, false);
      const auto t1 = __builtin_amdgcn_permlane32_swap(packed[0][1], packed[1][1], false, false);
      pend[r] = u32x4{t0[0], t1[0], t0[1], t1[1]};
    }
    pend_ptr = qrow < L ? (char*)a.o + 2 * ((int64_t)bb * a.o_sb + (int64_t)h * a.o_sh +
                                            (int64_t)qrow * a.o_si + 8 * g)
                        : nullptr;
  };
  auto flush = [&]() {
    if (pend_ptr) {
      *(u32x4*)pend_ptr = pend[0];
      *(u32x4*)(pend_ptr + 32) = pend[1];
    }
    pend_ptr = nullptr;
  };

  // ---- the walk over entries --------------------------------------------------
  // Entry bb's loads were issued one entry earlier.  At the hand-over each
  // wave waits for its own loads (the previous entry's output stores went
  // out after the last hand-over and are long done), publishes the keys'
  // mask terms, and the barrier makes the stage visible and frees the other
  // stage; then the next entry's loads go out, the previous entry's output
  // is stored, and the entry computes.
  issue(b_first, 0);
  take_bias();
  for (int bb = b_first; bb < b_end; ++bb) {
    const int st = (bb - b_first) & 1;
    char* sb = lds + st * C::STAGE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < LP) ((bf16*)(sb + C::T_OFF))[tid] = tid < L && mbyte != 0 ? zero : (bf16)kNegInf;
    __syncthreads();
    if (bb + 1 < b_end) issue(bb + 1, st ^ 1);
    flush();
    if (wave_busy) compute(bb, sb);
  }
  flush();
}

}  // namespace fl
