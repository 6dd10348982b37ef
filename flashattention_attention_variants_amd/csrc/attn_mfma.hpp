// attn_mfma.hpp -- the bf16 fused attention forward on gfx950 matrix cores.
//
// One work-group = 4 waves = a tile of BM = 4*32*QB query rows of one (b, h).
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

template <int DQK_, int DV_, int NS_, int QB_, int MOD_, bool BIAS_, bool KMASK_, bool GATE_>
struct MfmaCfg {
  static constexpr int DQK = DQK_;   // q/k head dim (multiple of 16)
  static constexpr int DV = DV_;     // v head dim (multiple of 32)
  static constexpr int NS = NS_;     // softmax streams: 1, or 2 for DiffAttn
  static constexpr int QB = QB_;     // 32-query blocks per wave
  static constexpr int MOD = MOD_;
  static constexpr bool BIAS = BIAS_;
  static constexpr bool KMASK = KMASK_;
  static constexpr bool GATE = GATE_;
  static constexpr int NW = 4;               // waves per work-group
  static constexpr int BM = NW * 32 * QB;    // query rows per work-group
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KP = DQK + 8;         // LDS row pitch of K (bf16): conflict-free b128 reads
  static constexpr int VP = DV + 16;         // LDS row pitch of V (bf16): conflict-free tr reads
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int V_ELEMS = BN * VP;
  static constexpr int STAGE = NS * K_ELEMS + V_ELEMS;
  static constexpr int KCH = BN * DQK / 8 / (NW * 64);  // 16-byte K chunks per thread
  static constexpr int VCH = BN * DV / 8 / (NW * 64);   // 16-byte V chunks per thread
  // plain scores: no modification, bias or key mask; the scale then folds
  // into the exponent (one fma per score)
  static constexpr bool PLAIN = (MOD == MOD_NONE) && !BIAS && !KMASK;
  // one stream fits 2 waves per SIMD; two streams need the whole register file
  static constexpr int WAVES_PER_EU = NS == 1 ? 2 : 1;
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

// Buffer resource over [base, base + bytes); 0x00020000 is the raw 32-bit
// data-format word of gfx9 buffer descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <class C>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(C::WAVES_PER_EU)))
void attn_mfma_kernel(KernelArgs a) {
  constexpr int BN = C::BN, DQK = C::DQK, DV = C::DV, NS = C::NS, QB = C::QB;
  constexpr int KP = C::KP, VP = C::VP;
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) float kmadd[C::KMASK ? 2 * BN : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, g = lane >> 5;

  int bh, qt;
  decode_tile(a, blockIdx.x, bh, qt);
  const int b = bh / a.nh, h = bh % a.nh, hk = h / a.group;
  const int q0 = qt * C::BM;
  const int qlast = min(q0 + C::BM, a.sq) - 1;

  // ---- key-tile range of the work-group (union over its rows) -------------
  int lo_first, hi_first, lo_last, hi_last;
  key_interval(a, b, q0, lo_first, hi_first);
  key_interval(a, b, qlast, lo_last, hi_last);
  const int kt_lo = lo_first / BN;
  const int kt_hi = hi_last >= lo_first ? (hi_last + BN) / BN : kt_lo;

  // ---- this wave's rows and their key intervals ----------------------------
  const int wq0 = q0 + w * 32 * QB;
  const int wq1 = min(wq0 + 32 * QB, a.sq) - 1;  // last valid row of the wave
  int w_lo_min, w_hi_min, w_lo_max, w_hi_max;
  key_interval(a, b, min(wq0, a.sq - 1), w_lo_min, w_hi_min);
  key_interval(a, b, max(wq1, 0), w_lo_max, w_hi_max);
  const bool wave_idle = wq0 >= a.sq;

  int row_lo[QB], row_hi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(wq0 + 32 * qb + c, a.sq - 1);  // rows past S_q copy the last row
    key_interval(a, b, qi, row_lo[qb], row_hi[qb]);
  }

  // ---- Q operands in registers ---------------------------------------------
  // B operand of S^T = K Q^T: lane (c, g) holds Q[row c][16t + 8g .. +7].
  bf16x8 qreg[NS][QB][DQK / 16];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = wq0 + 32 * qb + c;
      const bf16* qp = (const bf16*)a.q[s] + b * a.q_sb + h * a.q_sh + (int64_t)qi * a.q_si;
#pragma unroll
      for (int t = 0; t < DQK / 16; ++t) {
        bf16x8 z = {};
        qreg[s][qb][t] = qi < a.sq ? *(const bf16x8*)(qp + 16 * t + 8 * g) : z;
      }
    }

  // ---- per-row softmax state -------------------------------------------------
  f32x16 oacc[NS][QB][DV / 32];
  float m_run[NS][QB], l_run[NS][QB];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[s][qb] = kNegInf;
      l_run[s][qb] = 0.0f;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) oacc[s][qb][db] = f32x16{};
    }

  // Scores live in base 2: plain scores keep q.k and fold scale*log2(e) into
  // the exponent; modified scores are converted to base-2 units first.
  const float cf = C::PLAIN ? a.scale_log2 : 1.0f;
  // Lazy rescale: the running max used in the exponent only moves when a
  // score exceeds it by more than 8 (base 2), so p <= 256 and most tiles
  // skip the accumulator rescale.  Exact: numerator and denominator share it.
  const float thr = 8.0f / cf;
  const float alibi_l2 = C::MOD == MOD_ALIBI ? alibi_slope_log2(a, h) : 0.0f;

  // ---- global -> register -> LDS tile movement -------------------------------
  // Each (b, K/V head) block is addressed through a bounds-checked buffer
  // resource re-based at every tile, so keys past S_k read as zeros with no
  // per-lane predicate.
  const char* kblk[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    kblk[s] = (const char*)((const bf16*)a.k[s] + b * a.k_sb + hk * a.k_sh);
  const char* vblk = (const char*)((const bf16*)a.v + b * a.v_sb + hk * a.v_sh);
  const int64_t k_row_b = a.k_si * 2, v_row_b = a.v_si * 2;
  const int64_t k_span = a.sk > 0 ? (int64_t)(a.sk - 1) * k_row_b + DQK * 2 : 0;
  const int64_t v_span = a.sk > 0 ? (int64_t)(a.sk - 1) * v_row_b + DV * 2 : 0;

  int k_off[C::KCH], k_lds[C::KCH], v_off[C::VCH], v_lds[C::VCH];
#pragma unroll
  for (int i = 0; i < C::KCH; ++i) {
    const int chunk = tid + 256 * i;
    const int key = chunk / (DQK / 8), col = chunk % (DQK / 8);
    k_off[i] = key * (int)k_row_b + 16 * col;
    k_lds[i] = key * KP + 8 * col;
  }
#pragma unroll
  for (int i = 0; i < C::VCH; ++i) {
    const int chunk = tid + 256 * i;
    const int key = chunk / (DV / 8), col = chunk % (DV / 8);
    v_off[i] = key * (int)v_row_b + 16 * col;
    v_lds[i] = key * VP + 8 * col;
  }

  bf16x8 kpre[NS][C::KCH], vpre[C::VCH];
  float kmpre = 0.0f;

  auto load_tile = [&](int kt) {
    const int64_t j0 = (int64_t)kt * BN;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(kblk[s] + j0 * k_row_b, k_span - j0 * k_row_b);
#pragma unroll
      for (int i = 0; i < C::KCH; ++i) kpre[s][i] = load16(rs, k_off[i]);
    }
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vblk + j0 * v_row_b, v_span - j0 * v_row_b);
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) vpre[i] = load16(rs, v_off[i]);
    if (C::KMASK && tid < BN) {
      const int j = (int)j0 + tid;
      kmpre = (j < a.sk && (!a.kmask || a.kmask[b * a.km_sb + (int64_t)j * a.km_sj] != 0))
                  ? 0.0f
                  : kNegInf;
    }
  };

  auto store_tile = [&](int stage) {
    bf16* ks = lds + stage * C::STAGE;
    bf16* vs = ks + NS * C::K_ELEMS;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < C::KCH; ++i) *(bf16x8*)(ks + s * C::K_ELEMS + k_lds[i]) = kpre[s][i];
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) *(bf16x8*)(vs + v_lds[i]) = vpre[i];
    if (C::KMASK && tid < BN) kmadd[stage * BN + tid] = kmpre;
  };

  // LDS element offsets of this lane's operand reads
  const int k_rd = c * KP + 8 * g;  // + 32kb*KP + 16t
  // transposed V read: lane i of each 16-lane block points at row (i/4) of a
  // 4-key group and 4 d-columns (i%4) of the block's 16 columns
  const int v_rd = (4 * g + ((c & 15) >> 2)) * VP + 16 * (c >> 4) + 4 * (c & 3);  // + 16st*VP + 32db

  // ---- one key tile: S^T, softmax update, O^T += V^T P^T ---------------------
  // Work units u = (stream s, query block qb) run as a two-stage pipeline:
  // the S^T products of unit u+1 are issued before the softmax of unit u, so
  // the matrix cores work while the vector ALUs exponentiate, and P.V of unit
  // u follows its softmax at once so P dies early.
  auto compute_tile = [&](int stage, int kt, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr int U = NS * QB;
    const bf16* ks = lds + stage * C::STAGE;
    const bf16* vs = ks + NS * C::K_ELEMS;
    const int j0 = kt * BN;

    bf16x8 kop[2][DQK / 16];  // K operands of the current stream
    auto read_k = [&](int s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t)
          kop[kb][t] = *(const bf16x8*)(ks + s * C::K_ELEMS + k_rd + 32 * kb * KP + 16 * t);
    };
    auto qk = [&](int u, f32x16 (&acc)[2]) {
      const int s = u / QB, qb = u % QB;
      if (qb == 0) read_k(s);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < DQK / 16; ++t)
          acc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb][t], qreg[s][qb][t], acc[kb], 0, 0, 0);
      }
    };

    f32x16 sacc[2][2];  // [pipeline slot][32-key block]
    qk(0, sacc[0]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = u / QB, qb = u % QB;
      if (u + 1 < U) qk(u + 1, sacc[(u + 1) & 1]);
      f32x16 (&sc)[2] = sacc[u & 1];
      const int qi = wq0 + 32 * qb + c;

      // score modification, bias, key mask, positional mask
      float xm = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int jb = j0 + 32 * kb + 4 * g;  // key of register 0 in this lane
        float bias_v[16];
        if constexpr (C::BIAS) {
          const int qi_c = min(qi, a.sq - 1);
          const bf16* bp = (const bf16*)a.bias + h * a.bias_sh + (int64_t)qi_c * a.bias_si;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int j = jb + 8 * r4;
            bf16x4 bv = {};
            if (!MASKED || j < a.sk) bv = *(const bf16x4*)(bp + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) bias_v[4 * r4 + e] = (float)bv[e] * kLog2e;
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
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[kb][r];
          if constexpr (C::MOD == MOD_ALIBI) {
            const float dist = (float)(qi - jb - acc_row(r));
            x = x * a.scale_log2 - alibi_l2 * __builtin_fabsf(dist);
          } else if constexpr (C::MOD == MOD_SOFTCAP) {
            x = softcap_log2(a, x);
          } else if constexpr (!C::PLAIN) {
            x = x * a.scale_log2;
          }
          if constexpr (C::BIAS) x += bias_v[r];
          if constexpr (C::KMASK) x += km_v[r];
          if constexpr (MASKED) {
            const int j = jb + acc_row(r);
            x = (j >= row_lo[qb] && j <= row_hi[qb]) ? x : kNegInf;
          }
          sc[kb][r] = x;
          xm = fmaxf(xm, x);
        }
      }
      // xm covers this lane's half of the row's keys; the other half sits in
      // the lane 32 apart.  Both lanes of a row must use the same running
      // max, so the halves are combined only when some lane of the wave
      // would move it (a wave-uniform, rarely taken branch).
      const float m_old = m_run[s][qb];
      if (__builtin_amdgcn_ballot_w64(xm > m_old + thr)) {
        const float xf = fmaxf(xm, __shfl_xor(xm, 32));
        const bool move = xf > m_old + thr;
        const float m_new = move ? xf : m_old;
        const float alpha = !move ? 1.0f : (m_old == kNegInf ? 0.0f : fast_exp2((m_old - m_new) * cf));
        l_run[s][qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) oacc[s][qb][db] *= alpha;
        m_run[s][qb] = m_new;
      }
      const float nm = m_run[s][qb] == kNegInf ? 0.0f : -m_run[s][qb] * cf;

      // p = 2^(x*cf - m*cf), rounded to bf16 in the B-operand order of the
      // P.V product; the row sum adds the rounded values.
      bf16x8 pk[4];
      float lsum = 0.0f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        f32x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = fast_exp2(__builtin_fmaf(sc[st >> 1][8 * (st & 1) + e], cf, nm));
        pk[st] = __builtin_convertvector(p, bf16x8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pr = {pk[st][e], pk[st][e + 1]};
          const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsum, false);
        }
      }
      l_run[s][qb] += lsum;

      // O^T += V^T P^T.  A operand of lane (c, g): V^T[d = 32db + c][keys
      // 16st + 4g + 0..3, 16st + 8 + 4g + 0..3], two transposed 8-byte reads.
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
          const bf16* vp = vs + v_rd + 16 * st * VP + 32 * db;
          const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
          const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * VP));
          const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          oacc[s][qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[st], oacc[s][qb][db], 0, 0, 0);
        }
    }
  };

  // ---- main loop ---------------------------------------------------------------
  if (kt_lo < kt_hi) {
    load_tile(kt_lo);
    store_tile(0);
    __syncthreads();
  }
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int stage = (kt - kt_lo) & 1;
    const bool more = kt + 1 < kt_hi;
    if (more) load_tile(kt + 1);
    const int j0 = kt * BN, j1 = j0 + BN - 1;
    const bool empty = wave_idle || j0 > w_hi_max || j1 < w_lo_min;
    const bool full = j0 >= w_lo_max && j1 <= w_hi_min;
    if (!empty) {
      if (full)
        compute_tile(stage, kt, std::integral_constant<bool, false>{});
      else
        compute_tile(stage, kt, std::integral_constant<bool, true>{});
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, combine, gate, store --------------------------------
  float inv[NS][QB];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = l_run[s][qb] + __shfl_xor(l_run[s][qb], 32);
      inv[s][qb] = l > 0.0f ? 1.0f / l : 0.0f;
      const int qi = wq0 + 32 * qb + c;
      if (a.lse[s] && g == 0 && qi < a.sq) {
        const float m = m_run[s][qb];
        const float lse = l > 0.0f ? (m * cf + __builtin_log2f(l)) * kLn2 : kNegInf;
        a.lse[s][b * a.lse_sb + h * a.lse_sh + qi] = lse;
      }
    }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = wq0 + 32 * qb + c;
    if (qi >= a.sq) continue;
    bf16* op = (bf16*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si;
    const bf16* gp = C::GATE ? (const bf16*)a.gate + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_si
                             : nullptr;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * g;
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = oacc[0][qb][db][4 * r4 + e] * inv[0][qb];
          if constexpr (NS == 2) ov[e] -= a.lambda * oacc[1][qb][db][4 * r4 + e] * inv[1][qb];
        }
        if constexpr (C::GATE) {
          const bf16x4 gv = *(const bf16x4*)(gp + d);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] *= sigmoid((float)gv[e]);
        }
        const bf16x4 out = {(bf16)ov[0], (bf16)ov[1], (bf16)ov[2], (bf16)ov[3]};
        *(bf16x4*)(op + d) = out;
      }
  }
}

}  // namespace fl
