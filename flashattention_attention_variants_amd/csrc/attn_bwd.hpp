// attn_bwd.hpp -- backward of the bf16 fused attention (gfx950 matrix cores).
//
// With S = scale Q K^T, s = mod(S) masked, P = softmax(s) and the saved
// LSE, the gradients of a loss with output gradient dO are
//
//   D_i = sum_j P_ij dP_ij                     (= sum_d dO_id O_id)
//   dP  = dO V^T,   dS = P * (dP - D) * mod'(S)
//   dQ  = scale dS K,   dK = scale dS^T Q,   dV = P^T dO
//
// D is never taken from the stored output, and P is renormalised: dO . O
// with O rounded to bf16 carries an error of about 2^-9 |dO| |O|, and the P
// recomputed from the forward's LSE sums to 1 only within the rounding of
// the forward's row sum (up to 0.4% off at logits of standard deviation
// 25); under a sharp softmax dP - D is a small difference of large values,
// so either error dominates the gradients (1.1% mean relative error of dQ
// at those logits).  The dQ launch runs its sweep with D~ = dO . O and, in
// float32 beside it, Z = sum_j P and X = sum_j P (dP - D~) (D~ enters the
// dP product as one more k-step, so X carries no cancellation); with P/Z
// exact, D = sum_j P dP / Z = D~ + X / Z, and dQ linear in D, one more
// product corrects it at the end: dQ = scale / Z (dS~ K + (D~ - D) E),
// E = sum_j P mod' K.  It writes D
// and the LSE in log2 units for the dK, dV launch, whose P keeps the
// factor Z (a relative error of the order of the forward's rounding, not
// amplified).
//
// with mod' = 1 for plain scores and ALiBi (an additive term) and
// 1 - tanh^2(S / cap) for softcap; P is recomputed from the scores and the
// LSE, never stored (the single-pass forward keeps no score matrix; the
// pages leave training to future work: gist.science explainer,
// "Significance and Claims").
//
// Two launches share one kernel template.  Each wave owns 32 "rows" for
// the whole kernel, held in registers in matrix-core operand order, and the
// work-group streams 64-entry tiles of two tensors T1, T2 through LDS:
//
//   role   rows         T1, T2        products per 32x32 unit
//   DQ     queries      K, V          X = S^T, Y = dP^T; dQ^T += K^T dS^T,
//                                                        E^T  += K^T (P mod')^T
//   DKDV   keys         Q, dO         X = S,   Y = dP;   dK^T += Q^T dS,
//                                                        dV^T += dO^T P
//
// X = T1 R1^T and Y = T2 R2^T put the row entity in the lane (one column
// per lane) and the streamed entity in the accumulator registers, exactly
// as the forward's S^T = K Q^T; the accumulations read T1 or T2 transposed
// with ds_read_b64_tr_b16, and the packed bf16 dS (or P) registers are
// directly their B operands, because the key order inside each 16-entry
// step is the forward's permutation (16st + 4g + 0..3, 16st + 8 + 4g + 0..3).
// DQ runs first and also writes D and LSE log2(e) for the DKDV launch,
// which visits, for each key tile, the tiles of every query head of the
// group that may see it, loading those two per streamed query into LDS
// beside the tile.
#pragma once

#include "attn_mfma.hpp"

namespace fl {

enum BwdRole { BWD_DQ = 0, BWD_DKDV = 1 };

// The float32 value v as three bf16 parts: each takes the next 8
// significant bits, so hi + mid + lo == v exactly.  Returned as the bit
// patterns {hi, mid, lo} in the low halves of three words.
__device__ __forceinline__ void split3_bits(float v, uint32_t (&p)[3]) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v), h = u & 0xffff0000u;
  const float r1 = v - __builtin_bit_cast(float, h);
  const uint32_t m = __builtin_bit_cast(uint32_t, r1) & 0xffff0000u;
  const float r2 = r1 - __builtin_bit_cast(float, m);
  p[0] = h >> 16;
  p[1] = m >> 16;
  p[2] = __builtin_bit_cast(uint32_t, r2) >> 16;
}
// v's three parts in k-slots 0..2 of a lane-half-0 matrix operand (zero for
// lane half 1, `half0` false); k-slots 3..5 hold `s345` (bf16 bits, 0: none)
__device__ __forceinline__ bf16x8 split3_operand(float v, bool half0, uint32_t s345 = 0) {
  uint32_t p[3];
  split3_bits(half0 ? v : 0.0f, p);
  const uint32_t k = half0 ? s345 : 0u;
  const u32x4 w = {p[0] | (p[1] << 16), p[2] | (k << 16), k | (k << 16), 0u};
  return __builtin_bit_cast(bf16x8, w);
}


template <int ROLE_, int MOD_>
struct BwdCfg {
  static constexpr int ROLE = ROLE_;
  static constexpr int MOD = MOD_;
  static constexpr int D = 64;
  static constexpr int NW = 4;
  static constexpr int BM = NW * 32;  // rows per work-group
  static constexpr int BN = 64;       // streamed entries per tile
  static constexpr int T_ELEMS = BN * D;
  static constexpr int STAGE = 2 * T_ELEMS;
  // LDS stages: the next tile loads while one computes (a third stage, two
  // tiles in flight, measured 0.5-2% slower in either launch)
  static constexpr int NSTAGE = 2;
  static constexpr int CH = BN * D / 8 / (NW * 64);  // 16-byte chunks per thread per tensor
  // The 16-byte chunks of a row are XOR-swizzled in LDS by a function of
  // the row pair j = (row >> 1) & 7, chosen for the two read shapes (64
  // banks of 4 bytes; a 16-byte read serves 16 lanes per cycle, an 8-byte
  // read 32): a row read takes one chunk of 16 consecutive rows, so the
  // eight rows of each parity (one bank half each) need eight distinct
  // swizzles; a transposed read takes four chunks (one half of the row) of
  // rows r..r+3, so rows r and r + 2 (r = 0, 1 mod 4) need swizzles in
  // opposite halves (bit 2).  j ^ 4 (j & 1) meets both; row & 7 met
  // neither and cost every read of both kinds a two-way conflict.  Rows
  // 8 apart differ by 4 in j, so their swizzles differ by 4.
  __device__ static constexpr int swz(int row) {
    const int j = (row >> 1) & 7;
    return j ^ ((j & 1) << 2);
  }
  static_assert(MOD == MOD_NONE || MOD == MOD_ALIBI || MOD == MOD_SOFTCAP, "score modification");
};

template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_kernel(KernelArgs a, BwdArgs g2) {
  constexpr int D = C::D, BN = C::BN;
  constexpr bool DQ = C::ROLE == BWD_DQ;
  __shared__ __attribute__((aligned(16))) bf16 lds[C::NSTAGE * C::STAGE];
  // DKDV: the streamed queries' LSE and D, [stage][lse, delta][entry]
  __shared__ __attribute__((aligned(16))) float stat[C::NSTAGE][2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  // ---- work-group -> (b, head, row tile) ------------------------------------------
  const int n_rows = DQ ? a.sq : a.sk;             // row entities
  const int n_rt = (n_rows + C::BM - 1) / C::BM;
  const int nh_rows = DQ ? a.nh : a.nh / a.group;  // heads the rows belong to
  // the forward's XCD-aware order over (head, row tile): the work-groups of
  // one K/V head share an XCD's L2; dense rows go out head by head, and
  // under causal-class masks the heaviest tiles go first (the last query
  // tiles for dQ, the first key tiles for dK, dV)
  int bh, rt;
  {
    KernelArgs t = a;
    t.nh = nh_rows;
    t.group = DQ ? a.group : 1;
    t.n_qt = n_rt;
    t.head_major = a.iv_kind == IV_FULL;
    t.heavy_first = DQ ? a.heavy_first : 0;
    decode_tile(t, blockIdx.x, bh, rt);
  }
  const int b = bh / nh_rows, hr = bh % nh_rows;   // query head (DQ) or K/V head (DKDV)
  const int hk = DQ ? hr / a.group : hr;
  const int r0 = rt * C::BM;
  const int wr0 = r0 + 32 * w;
  const int row = min(wr0 + c, n_rows - 1);        // this lane's row (clamped)
  const bool wave_idle = wr0 >= n_rows;

  // Document mask: the batch entry's offsets go to LDS once, where the
  // prologue's interval searches read them (a search through global memory
  // costs a round trip per step); the tiles overwrite them after the
  // barrier that closes the prologue.  A document's keys and queries are
  // the same run of positions.
  const bool doc_lds = a.iv_kind == IV_DOCUMENT && a.n_docs + 1 <= (int)(sizeof(lds) / sizeof(int));
  if (doc_lds) {
    const int32_t* off = a.doc_offsets + (int64_t)b * (a.n_docs + 1);
    for (int t = tid; t <= a.n_docs; t += C::NW * 64) ((int*)lds)[t] = off[t];
    __syncthreads();
  }
  auto doc_ivl = [&](int x, int& lo, int& hi) {
    doc_run((const int*)lds, a.n_docs, x, lo, hi);
    lo = max(lo, 0);
    hi = min(hi, (DQ ? a.sk : a.sq) - 1);
  };

  const int64_t q_row_b = a.q_si * 2, k_row_b = a.k_si * 2;

  // ---- the wave's rows in registers: B operands, lane (c, g) holds
  // R[row c][16t + 8g .. +7] -------------------------------------------------------
  bf16x8 r1[D / 16], r2[D / 16];
  {
    const bf16* p1 = DQ ? (const bf16*)a.q[0] + b * a.q_sb + hr * a.q_sh
                        : (const bf16*)a.k[0] + b * a.k_sb + hk * a.k_sh;
    const bf16* p2 = DQ ? (const bf16*)g2.dout + b * a.q_sb + hr * a.q_sh
                        : (const bf16*)a.v + b * a.v_sb + hk * a.v_sh;
    const int64_t rb = DQ ? q_row_b : k_row_b;
    const int64_t off = (int64_t)row * rb;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      r1[t] = *(const bf16x8*)((const char*)p1 + off + 32 * t + 16 * g);
      r2[t] = *(const bf16x8*)((const char*)p2 + off + 32 * t + 16 * g);
    }
  }

  // ---- per-row statistics and intervals ------------------------------------------
  float lse2_row = 0.0f, delta_row = 0.0f;  // DQ: this lane's query
  // DQ: the keys of the query; DKDV: the queries of the key.  lane_w is the
  // number of them (0: none), except under ALiBi, where it stays the last
  // one: its instance sits at 256 registers and the compare of the count
  // takes it past them
  int lane_lo, lane_w;
  if constexpr (DQ) {
    // D = dO . O over the row; the lane holds half of the head dimension
    const bf16* po = (const bf16*)g2.o + b * a.q_sb + hr * a.q_sh + (int64_t)row * a.q_si;
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const bf16x8 ov = *(const bf16x8*)(po + 16 * t + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)r2[t][e], (float)ov[e], part);
    }
    delta_row = part + __shfl_xor(part, 32);
    const int64_t li = b * a.lse_sb + hr * a.lse_sh + row;
    const float l = a.lse[0][li];
    lse2_row = l == kNegInf ? __builtin_inff() : l * kLog2e;  // no key: every p is 0
  }
  if (doc_lds) doc_ivl(row, lane_lo, lane_w);
  else if constexpr (DQ) key_interval(a, b, row, lane_lo, lane_w);
  else query_interval(a, b, row, lane_lo, lane_w);
  if constexpr (C::MOD != MOD_ALIBI) lane_w = max(lane_w - lane_lo + 1, 0);

  // streamed range of the work-group and of this wave (union over rows)
  int lo_first, hi_first, lo_last, hi_last, w_lo_min, w_hi_min, w_lo_max, w_hi_max;
  auto ivl = [&](int x, int& lo, int& hi) {
    if (doc_lds) doc_ivl(x, lo, hi);
    else if constexpr (DQ) key_interval(a, b, x, lo, hi);
    else query_interval(a, b, x, lo, hi);
  };
  ivl(r0, lo_first, hi_first);
  ivl(min(r0 + C::BM, n_rows) - 1, lo_last, hi_last);
  ivl(min(wr0, n_rows - 1), w_lo_min, w_hi_min);
  ivl(max(min(wr0 + 31, n_rows - 1), min(wr0, n_rows - 1)), w_lo_max, w_hi_max);
  if (doc_lds) __syncthreads();  // the last read of the LDS offsets
  const int t_lo = lo_first / BN;
  const int t_hi = hi_last >= lo_first ? (hi_last + BN) / BN : t_lo;
  const int n_t = t_hi - t_lo;
  // DKDV visits the query tiles of every query head of the group
  const int n_heads = DQ ? 1 : a.group;
  const int n_it = n_t * n_heads;

  float alibi_l2 = 0.0f;
  if constexpr (C::MOD == MOD_ALIBI) {
    if constexpr (DQ) alibi_l2 = alibi_slope_log2(a, hr);
  }
  // DKDV: key-side operand of the statistics' k-step (-1 in k-slots 0..2 of
  // lane half 0) and the factor that takes the LSE to score units
  bf16x8 fold_b = {};
  if constexpr (!DQ) {
    const bf16 m1 = (bf16)-1.0f, z = (bf16)0.0f;
    if (g == 0) fold_b = bf16x8{m1, m1, m1, z, z, z, z, z};
  }
  // DQ: Y = dP^T - D~ starts from -D~ (the lane's query is the column of
  // every accumulator register)
  f32x16 y_init;
#pragma unroll
  for (int r = 0; r < 16; ++r) y_init[r] = -delta_row;
  const float inv_sc = 1.0f / a.scale_log2;
  // DQ under ALiBi: the query side of the distance k-step (sigma in k-slots
  // 0..2 of lane half 0) and the LSE with the query term for either sigma
  bf16x8 sig_pos = {}, sig_neg = {};
  float lse2_pos = lse2_row, lse2_neg = lse2_row;
  if constexpr (DQ && C::MOD == MOD_ALIBI) {
    const bf16 one = (bf16)1.0f, mone = (bf16)-1.0f, z = (bf16)0.0f;
    if (g == 0) {
      sig_pos = bf16x8{one, one, one, z, z, z, z, z};
      sig_neg = bf16x8{mone, mone, mone, z, z, z, z, z};
    }
    const float qt = alibi_l2 * (float)(row - wr0);
    lse2_pos = lse2_row + qt;
    lse2_neg = lse2_row - qt;
  }

  // ---- tile loads: global -> LDS ----------------------------------------------------
  int t_off[C::CH];
  const int64_t s_row_b = DQ ? k_row_b : q_row_b;  // streamed tensors' row stride
#pragma unroll
  for (int i = 0; i < C::CH; ++i) {
    const int q = (i * C::NW + w) * 64 + lane;
    const int rr = q / 8, phys = q % 8;
    t_off[i] = rr * (int)s_row_b + 16 * (phys ^ C::swz(rr));
  }
  const int n_s = DQ ? a.sk : a.sq;  // streamed entities
  const int64_t s_span = n_s > 0 ? (int64_t)(n_s - 1) * s_row_b + D * 2 : 0;
  auto tile_coords = [&](int it, int& head, int& tile) {
    if (DQ || a.group == 1) {
      // one head: no division (a scalar division costs tens of instructions)
      head = DQ ? hr : hk;
      tile = t_lo + it;
    } else {
      head = hk * a.group + it / max(n_t, 1);
      tile = t_lo + it % max(n_t, 1);
    }
  };
  auto load_tile = [&](int it, int stage) {
    int head, tile;
    tile_coords(it, head, tile);
    const int64_t e0 = (int64_t)tile * BN;
    const char* b1;
    const char* b2;
    if constexpr (DQ) {
      b1 = (const char*)((const bf16*)a.k[0] + b * a.k_sb + hk * a.k_sh);
      b2 = (const char*)((const bf16*)a.v + b * a.v_sb + hk * a.v_sh);
    } else {
      b1 = (const char*)((const bf16*)a.q[0] + b * a.q_sb + head * a.q_sh);
      b2 = (const char*)((const bf16*)g2.dout + b * a.q_sb + head * a.q_sh);
    }
    bf16* ts = lds + stage * C::STAGE;
    // one resource over the whole block; the tile's offset rides in the
    // per-lane offset (below 2^31 up to 63 rows past the block's end)
    const __amdgpu_buffer_rsrc_t rs1 = make_rsrc(b1, s_span);
    const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(b2, s_span);
    const int e_off = (int)e0 * (int)s_row_b;
#pragma unroll
    for (int i = 0; i < C::CH; ++i) lds_load16(rs1, ts + (i * C::NW + w) * 512, t_off[i] + e_off);
#pragma unroll
    for (int i = 0; i < C::CH; ++i)
      lds_load16(rs2, ts + C::T_ELEMS + (i * C::NW + w) * 512, t_off[i] + e_off);
    if constexpr (!DQ) {
      // the tile's 64 queries' LSE (log2 units, from the dQ launch) and D,
      // straight into LDS as well (every wave loads both, so that each wave
      // issues the same number of loads; the copies write equal values);
      // queries past the end read 0 and are masked
      const int64_t so = b * a.lse_sb + head * a.lse_sh;
      const int64_t n_b = (int64_t)a.sq * 4;
      const int eo = 4 * ((int)e0 + lane);
      lds_load4(make_rsrc(g2.lse2 + so, n_b), &stat[stage][0][0], eo);
      lds_load4(make_rsrc(g2.delta + so, n_b), &stat[stage][1][0], eo);
    }
  };
  auto sync_all = [&]() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // LDS offsets of this lane's reads.  Row reads (A operands of X and Y):
  // row 32kb + c, logical chunk 2t + g.
  int rd[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) rd[t] = c * D + 8 * ((2 * t + g) ^ C::swz(c));
  // Transposed reads (A operands of the accumulations): lane i of a 16-lane
  // block points at row i/4 of a 4-entry group and 4 columns 4*(i%4) of the
  // block's 16; rows 8m + tr_row take tr_row's swizzle for even m and that
  // swizzle ^ 4 for odd m (tr[1]).
  const int tr_row = 4 * g + ((c & 15) >> 2);
  int tr[2][D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = 32 * db + 16 * (c >> 4) + 4 * (c & 3);
    tr[0][db] = tr_row * D + 8 * ((d >> 3) ^ C::swz(tr_row)) + (d & 7);
    tr[1][db] = tr_row * D + 8 * ((d >> 3) ^ C::swz(tr_row + 8)) + (d & 7);
  }

  f32x16 acc1[D / 32], acc2[D / 32];  // DQ: dQ^T and E^T; DKDV: dK^T and dV^T
  float dex = 0.0f, zex = 0.0f;        // DQ: this lane's parts of Dx and Z
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    acc1[db] = f32x16{};
    acc2[db] = f32x16{};
  }

  // A operands of an accumulation from tensor base `tb` (LDS byte address)
  // for entry half kb: [db][h2]
  auto read_tr = [&](uint32_t tb, int kb, bf16x8 (&op)[D / 32][2]) {
    u32x2 raw[D / 32 * 4];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      // one register per base, so that the row offsets below become the
      // reads' immediate offsets (left alone, the compiler adds them to the
      // stage address first and spends an add per read)
      uint32_t b0 = tb + 2 * tr[0][db], b1 = tb + 2 * tr[1][db];
      asm("" : "+v"(b0), "+v"(b1));
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[4 * db + i] = ds_read_tr((i & 1 ? b1 : b0) + 2 * (8 * i + 32 * kb) * D);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x2 lo = raw[4 * db + 2 * h2], hi = raw[4 * db + 2 * h2 + 1];
        op[db][h2] = __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
      }
  };

  // straddle_tag: some unit of the tile straddles the diagonal (ALiBi's
  // correction is compiled only into that form)
  auto compute_tile = [&](int it, int stage, auto masked_tag, auto straddle_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool STR = decltype(straddle_tag)::value;
    int head, tile;
    tile_coords(it, head, tile);
    const int e0 = tile * BN;
    const bf16* t1 = lds + stage * C::STAGE;
    const bf16* t2 = t1 + C::T_ELEMS;
    float sl = alibi_l2;
    if constexpr (C::MOD == MOD_ALIBI && !DQ) sl = alibi_slope_log2(a, head);
    // DKDV: the tile's statistics enter the products as one more k-step
    // (the forward folds its reference the same way).  The streamed side
    // (A, a query per row) carries -(hi + mid + lo) of the query's value in
    // k-slots 0..2 of lane half 0 against ones on the key side (B), so
    //   X = Q K^T - L,   L = LSE log2(e) / (scale log2(e)) = LSE / scale,
    //   Y = dO V^T - D,
    // and s = X scale log2(e) = S log2(e) - LSE log2(e), p = 2^s, dS =
    // p Y: no statistic is read per score.  The three bf16 parts hold the
    // float32 value exactly (each takes the next 8 significant bits), and
    // each product with 1 is exact.  Softcap keeps L out of X (its scores
    // pass through tanh first) and reads the LSE per score.
    constexpr bool FOLD_L = !DQ && C::MOD != MOD_SOFTCAP;
    // ALiBi: the distance penalty rides on the same k-step (as in the
    // forward).  With sigma = +1 on a unit whose queries all lie at or after
    // its keys and -1 on one whose queries all lie at or before them,
    //   -slope |q - k| = -sigma slope (q - w0) + sigma slope (k - w0),
    // w0 the wave's first row.  DKDV adds the query term to L (A side) and
    // takes the key term as three parts of slope (k - w0) / scale in k-slots
    // 3..5 of the key side (B, sign sigma) against ones; DQ takes the key
    // term as three parts on the key side (A) against sigma in the query
    // side (B) and subtracts the query term with the LSE.  A unit that
    // straddles the diagonal takes sigma = +1 and a vector correction for
    // its pairs with k > q.  Every value carried is below the distance
    // scale itself, so the float32 parts lose nothing against the plain
    // penalty.
    constexpr bool AF = C::MOD == MOD_ALIBI;
    const float a_f = sl * inv_sc;  // the slope in units of X
    bool neg[2] = {false, false}, straddle[2] = {false, false};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int u_lo = e0 + 32 * kb;  // the unit's streamed entities
      const int q_lo = DQ ? wr0 : u_lo, q_hi = q_lo + 31;
      const int k_lo = DQ ? u_lo : wr0, k_hi = k_lo + 31;
      neg[kb] = q_hi <= k_lo;
      straddle[kb] = !neg[kb] && q_lo < k_hi;
    }
    bf16x8 kb_pos = fold_b, kb_neg = fold_b;  // DKDV key side under ALiBi
    if constexpr (AF && !DQ) {
      uint32_t kp[3];
      split3_bits(a_f * (float)(row - wr0), kp);
      const uint32_t m1 = 0xbf80u;  // bf16 -1
      u32x4 wv = {m1 | (m1 << 16), m1 | (kp[0] << 16), kp[1] | (kp[2] << 16), 0u};
      if (g != 0) wv = u32x4{0u, 0u, 0u, 0u};
      kb_pos = __builtin_bit_cast(bf16x8, wv);
      if (g == 0) wv ^= u32x4{0u, 0x80000000u, 0x80008000u, 0u};
      kb_neg = __builtin_bit_cast(bf16x8, wv);
    }
    bf16x8 fold_a[2][2];  // [kb][L, D]
    if constexpr (!DQ) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // +inf (a query with no key) becomes a huge finite L: its p is 0
        float l = FOLD_L ? fminf(stat[stage][0][32 * kb + c] * inv_sc, 1e30f) : 0.0f;
        if constexpr (AF) l += (neg[kb] ? -a_f : a_f) * (float)(e0 + 32 * kb + c - wr0);
        fold_a[kb][0] = split3_operand(l, g == 0, AF ? 0x3f80u : 0u);  // ones in k-slots 3..5
        fold_a[kb][1] = split3_operand(stat[stage][1][32 * kb + c], g == 0);
      }
    }
    // X = T1 R1^T and Y = T2 R2^T of entry half kb
    auto products = [&](int kb, f32x16& x, f32x16& y) {
      x = f32x16{};
      y = f32x16{};
      if constexpr (FOLD_L)
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fold_a[kb][0], AF ? (neg[kb] ? kb_neg : kb_pos) : fold_b, x,
                                                    0, 0, 0);
      if constexpr (AF && DQ) {
        const bf16x8 ka = split3_operand(a_f * (float)(e0 + 32 * kb + c - wr0), g == 0);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, neg[kb] ? sig_neg : sig_pos, x, 0, 0, 0);
      }
      if constexpr (!DQ) y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fold_a[kb][1], fold_b, y, 0, 0, 0);
      else y = y_init;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 a1 = *(const bf16x8*)(t1 + rd[t] + 32 * kb * D);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, r1[t], x, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 a2 = *(const bf16x8*)(t2 + rd[t] + 32 * kb * D);
        y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, r2[t], y, 0, 0, 0);
      }
    };
    // (issuing the second half's products before the first half's vector
    // work measured no faster)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 x, y;
      products(kb, x, y);
      // streamed entity of register 0 in this lane; register r adds acc_row(r)
      const int eb = e0 + 32 * kb + 4 * g;
      const int ebl = eb - lane_lo;  // entry of register 0 relative to the row's first
      if constexpr (AF && STR) {
        if (straddle[kb]) {
          // sigma = +1 gave the pairs with k > q +slope (k - q): subtract twice that
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ent = eb + acc_row(r);
            const int dk = DQ ? ent - row : row - ent;  // k - q
            x[r] = dk > 0 ? x[r] - 2.0f * a_f * (float)dk : x[r];
          }
        }
      }
      float lse4[16];
      if constexpr (!DQ && !FOLD_L) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 lv = *(const f32x4*)&stat[stage][0][32 * kb + 4 * g + 8 * m];
#pragma unroll
          for (int e = 0; e < 4; ++e) lse4[4 * m + e] = lv[e];
        }
      }
      f32x16 ds, pp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ent = eb + acc_row(r);
        float s = x[r] * a.scale_log2;
        float dmod = 1.0f;
        if constexpr (C::MOD == MOD_SOFTCAP) {
          s = softcap_log2(a, x[r]);
          const float th = s * (1.0f / a.softcap_log2);
          dmod = 1.0f - th * th;
        }
        float p;
        if constexpr (DQ) p = fast_exp2(s - (AF ? (neg[kb] ? lse2_neg : lse2_pos) : lse2_row));
        else if constexpr (FOLD_L) p = fast_exp2(s);
        else p = fast_exp2(s - lse4[r]);
        // one unsigned compare: lane_lo >= 0 and the last entry is in
        // range, so ent - lane_lo cannot overflow
        if constexpr (MASKED) {
          if constexpr (C::MOD == MOD_ALIBI) p = (ent >= lane_lo && ent <= lane_w) ? p : 0.0f;
          else p = (unsigned)(ebl + acc_row(r)) < (unsigned)lane_w ? p : 0.0f;
        }
        if constexpr (DQ) {
          dex = fmaf(p, y[r], dex);
          zex += p;
          pp[r] = p * dmod;
        } else {
          pp[r] = p;
        }
        ds[r] = p * y[r] * dmod;
      }
      // B operands: 16-entry steps 2kb and 2kb + 1 in the permuted order
      bf16x8 pds[2], ppk[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x8 v1, v2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v1[e] = ds[8 * h2 + e];
          v2[e] = pp[8 * h2 + e];
        }
        pds[h2] = __builtin_convertvector(v1, bf16x8);
        ppk[h2] = __builtin_convertvector(v2, bf16x8);
      }
      bf16x8 op1[D / 32][2];
      read_tr(lds_addr(t1), kb, op1);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          acc1[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op1[db][h2], pds[h2], acc1[db], 0, 0, 0);
          if constexpr (DQ)
            acc2[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op1[db][h2], ppk[h2], acc2[db], 0, 0, 0);
        }
      if constexpr (!DQ) {
        bf16x8 op2[D / 32][2];
        read_tr(lds_addr(t2), kb, op2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            acc2[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op2[db][h2], ppk[h2], acc2[db], 0, 0, 0);
      }
    }
  };

  // ---- main loop: NSTAGE LDS stages, tiles it + 1 .. it + NSTAGE - 1 load
  // while tile it computes
  constexpr int NS = C::NSTAGE;
  constexpr int LOADS = 2 * C::CH + (DQ ? 0 : 2);  // DMA loads per tile and wave
  static_assert(NS == 2 || NS == 3, "stages");
  static_assert(LOADS < 64, "vmcnt range");
  for (int i = 0; i < NS - 1 && i < n_it; ++i) load_tile(i, i);
  int stage = 0;
  for (int it = 0; it < n_it; ++it) {
    // tile it has landed once no more than the next tile's loads are in
    // flight; the barrier publishes it and closes every wave's reads of the
    // stage that the load below refills (tile it - 1's)
    if (NS == 3 && it + 1 < n_it)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS) : "memory");
    else
      sync_all();
    if (it + NS - 1 < n_it) load_tile(it + NS - 1, stage == 0 ? NS - 1 : stage - 1);
    int head, tile;
    tile_coords(it, head, tile);
    const int e0 = tile * BN, e1 = e0 + BN - 1;
    const bool empty = wave_idle || e0 > w_hi_max || e1 < w_lo_min;
    const bool full = e0 >= w_lo_max && e1 <= w_hi_min;
    if (!empty) {
      using T = std::true_type;
      using F = std::false_type;
      // ALiBi: does some unit of the tile straddle the wave's diagonal?
      bool str = false;
      if constexpr (C::MOD == MOD_ALIBI) {
        const int q_lo = DQ ? wr0 : e0, q_hi = DQ ? wr0 + 31 : e1;
        const int k_lo = DQ ? e0 : wr0, k_hi = DQ ? e1 : wr0 + 31;
        str = q_hi > k_lo && q_lo < k_hi;
      }
      if (str) {
        if (full) compute_tile(it, stage, F{}, T{});
        else compute_tile(it, stage, T{}, T{});
      } else {
        if (full) compute_tile(it, stage, F{}, F{});
        else compute_tile(it, stage, T{}, F{});
      }
    }
    stage = stage == NS - 1 ? 0 : stage + 1;
  }

  // ---- epilogue: lane = row, registers = head dimension --------------------------
  // DQ: the exact D (both lane halves), the correction of dQ, D for dK, dV
  float dfix = 0.0f, zinv = 1.0f;
  if constexpr (DQ) {
    const float z = zex + __shfl_xor(zex, 32);
    zinv = z > 0.0f ? 1.0f / z : 0.0f;  // no key: every product is zero
    // dex sums p (dP - D~): D = D~ + dex / Z
    dfix = -(dex + __shfl_xor(dex, 32)) * zinv;
    const float dn = delta_row - dfix;
    if (g == 0 && wr0 + c < a.sq) {
      const int64_t li = b * a.lse_sb + hr * a.lse_sh + row;
      g2.delta[li] = dn;
      g2.lse2[li] = lse2_row;
    }
  }
  if (wr0 + c >= n_rows) return;
  const float sc = a.scale_log2 * kLn2;  // scale
  if constexpr (DQ) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc1[db][r] = fmaf(dfix, acc2[db][r], acc1[db][r]) * zinv;
  }
  bf16* o1;
  bf16* o2 = nullptr;
  if constexpr (DQ) {
    o1 = (bf16*)g2.dq + b * a.q_sb + hr * a.q_sh + (int64_t)row * a.q_si;
  } else {
    o1 = (bf16*)g2.dk + b * a.k_sb + hk * a.k_sh + (int64_t)row * a.k_si;
    o2 = (bf16*)g2.dv + b * a.v_sb + hk * a.v_sh + (int64_t)row * a.v_si;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * g;
      const bf16x4 v1 = {(bf16)(acc1[db][4 * r4] * sc), (bf16)(acc1[db][4 * r4 + 1] * sc),
                         (bf16)(acc1[db][4 * r4 + 2] * sc), (bf16)(acc1[db][4 * r4 + 3] * sc)};
      *(bf16x4*)(o1 + d) = v1;
      if constexpr (!DQ) {
        const bf16x4 v2 = {(bf16)acc2[db][4 * r4], (bf16)acc2[db][4 * r4 + 1],
                           (bf16)acc2[db][4 * r4 + 2], (bf16)acc2[db][4 * r4 + 3]};
        *(bf16x4*)(o2 + d) = v2;
      }
    }
}

}  // namespace fl
