// ipa.hpp -- the attention core of Invariant Point Attention on gfx950.
//
// The pages name Invariant Point Attention as a data-dependent variant a
// score_mod/block_mask template cannot express (gist.science explainer,
// "Technical Summary: Problem Statement"; papers.lqhl.me wiki, "问题与动机")
// without giving its formula; the form computed is AlphaFold2's attention
// core.  Per batch entry b, query residue i and head h, with frames
// T = (R, t) mapping local to global coordinates:
//
//   logit_ij = w_L ( q_i.k_j / sqrt(C) + bias_hij
//                    - gamma_h w_C / 2 sum_p |T_i q_ip - T_j k_jp|^2 )
//   a_ij     = softmax over the keys the key mask keeps
//   o_i      = sum_j a_ij v_j
//   o_pts_ip = T_i^-1 sum_j a_ij T_j v_jp        (in the query's frame)
//   o_pair_i = sum_j a_ij z_ij
//
// One work-group = one query residue and four heads (one wave per head;
// the work-groups of a residue share an XCD, so its pair rows z_i are
// fetched into one L2).  Keys stream in tiles of 64, one key per lane: the
// lane computes its key's global points in float32 (points keep absolute
// coordinates of tens of angstroms, so distances are taken as plain
// differences, never expanded into products), the logit, and the online
// softmax update (a per-head running maximum, wave-uniform; per-lane partial
// sums rescaled by 2^(m_old - m_new)).  The value and value-point sums stay
// per lane and are reduced across the wave once at the end.  The pair
// output is the one dense contraction, [heads x keys] . [keys x C_z] per
// residue: the tile of z_i goes from HBM straight into LDS and the matrix
// cores take it as the B operand of v_mfma_f32_16x16x32_bf16 through
// transposed LDS reads, with the tile's weights (rounded to bf16) as A.
#pragma once

#include <type_traits>

#include "fl_common.hpp"

namespace fl {

struct IpaArgs {
  const bf16 *q, *k, *v;        // [B, L, H, C]
  const float *q_pts, *k_pts;   // [B, L, H, PQ, 3]
  const float* v_pts;           // [B, L, H, PV, 3]
  const float *rot, *trans;     // [B, L, 3, 3] row-major, [B, L, 3]
  const float* gamma;           // [H]
  const bf16* bias;             // [B, H, L, L] or null
  const bf16* z;                // [B, L, L, CZ] or null (CZ = 0)
  const uint8_t* kmask;         // [B, L] or null
  bf16* o;                      // [B, L, H, C]
  float* o_pts;                 // [B, L, H, PV, 3]
  bf16* o_pair;                 // [B, L, H, CZ]
  int B, L, H;
  float w_scalar;  // w_L / sqrt(C), base-2 units
  float w_bias;    // w_L, base-2 units
  float w_point;   // w_L w_C / 2, base-2 units (times gamma_h)
};

template <int C_, int PQ_, int PV_, int CZ_>
struct IpaCfg {
  static constexpr int C = C_, PQ = PQ_, PV = PV_, CZ = CZ_;
  static constexpr int BN = 64;        // keys per tile (one per lane)
  static constexpr int HW = 4;         // heads (waves) per work-group
  static constexpr int NBZ = CZ / 16;  // 16-wide column blocks of the pair output
  static constexpr int NBW = NBZ > 0 ? (NBZ + HW - 1) / HW : 0;  // blocks per wave
  static_assert(C % 8 == 0 && CZ % 16 == 0 && (PQ * 3) % 4 == 0 && (PV * 3) % 4 == 0, "ipa sizes");
};

// Wave-wide sum / max, every lane ending with the total: within rows of 16
// lanes by DPP (swaps of neighbours and pairs, then the half-row and row
// mirrors), then the four row results read into scalar registers and
// combined in one order for every lane.  Vector-ALU and scalar reads only:
// the LDS permute behind a generic shuffle costs an LDS round trip per step.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <class Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  auto dpp = [](float v, auto ctrl) { return dpp_f32<decltype(ctrl)::value>(v); };
  x = op(x, dpp(x, std::integral_constant<int, 0xb1>{}));   // quad_perm [1,0,3,2]
  x = op(x, dpp(x, std::integral_constant<int, 0x4e>{}));   // quad_perm [2,3,0,1]
  x = op(x, dpp(x, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  x = op(x, dpp(x, std::integral_constant<int, 0x140>{}));  // row_mirror
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, [](float u, float v) { return u + v; });
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float u, float v) { return fmaxf(u, v); });
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Three waves per SIMD (at most 168 registers, no spills at C_z = 128): the
// residues x head groups of the structure-module shape (768 work-groups)
// then run in one round on 256 compute units.
template <class K>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void ipa_kernel(IpaArgs a) {
  constexpr int C = K::C, PQ = K::PQ, PV = K::PV, CZ = K::CZ, BN = K::BN, HW = K::HW;
  __shared__ __attribute__((aligned(16))) bf16 zs[CZ > 0 ? 2 * BN * CZ : 8];
  __shared__ __attribute__((aligned(16))) bf16 ps[2][16 * BN];  // weights, rows = heads
  __shared__ float als[2][16];                                  // per-head rescale factors
  __shared__ float lsum[16];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = a.L, H = a.H;
  const int n_hg = (H + HW - 1) / HW;
  // work-group -> (residue, head group); the head groups of a residue go to
  // one XCD when the residues split evenly over the 8 XCDs
  int res, hg;
  {
    const int id = blockIdx.x, n_res = a.B * L;
    if ((n_res & 7) == 0) {
      const int xcd = id & 7, slot = id >> 3;
      hg = slot % n_hg;
      res = (slot / n_hg) * 8 + xcd;
    } else {
      hg = id % n_hg;
      res = id / n_hg;
    }
  }
  const int b = res / L, i = res % L;
  const int h = hg * HW + w;
  const bool active = h < H;
  const int hh = active ? h : H - 1;  // idle waves read in bounds and write nothing

  // clear the weight rows no head writes (the matrix product reads all 16)
  for (int x = tid; x < 2 * 16 * BN; x += 256) (&ps[0][0])[x] = (bf16)0.0f;
  if (tid < 32) (&als[0][0])[tid] = 0.0f;
  __syncthreads();

  // ---- the query: scaled scalar features and global points -----------------
  const int64_t qrow = ((int64_t)res * H + hh);
  float qf[C];
  {
    const bf16x8* qp = (const bf16x8*)(a.q + qrow * C);
#pragma unroll
    for (int t = 0; t < C / 8; ++t) {
      const bf16x8 x = qp[t];
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[8 * t + e] = (float)x[e] * a.w_scalar;
    }
  }
  const float* Ri = a.rot + (int64_t)res * 9;
  const float* ti = a.trans + (int64_t)res * 3;
  float qg[PQ][3];
  {
    const float* qp = a.q_pts + qrow * PQ * 3;
#pragma unroll
    for (int p = 0; p < PQ; ++p) {
      const float x0 = qp[3 * p], x1 = qp[3 * p + 1], x2 = qp[3 * p + 2];
#pragma unroll
      for (int r = 0; r < 3; ++r) qg[p][r] = fmaf(Ri[3 * r], x0, fmaf(Ri[3 * r + 1], x1, fmaf(Ri[3 * r + 2], x2, ti[r])));
    }
  }
  const float wpt = a.w_point * a.gamma[hh];

  // ---- per-lane state ------------------------------------------------------------
  float m_run = kNegInf;  // wave-uniform running maximum (base 2)
  float l_lane = 0.0f;
  float acc_o[C], acc_g[PV][3];
#pragma unroll
  for (int c = 0; c < C; ++c) acc_o[c] = 0.0f;
#pragma unroll
  for (int p = 0; p < PV; ++p) acc_g[p][0] = acc_g[p][1] = acc_g[p][2] = 0.0f;
  f32x4 acc_z[K::NBW > 0 ? K::NBW : 1];
#pragma unroll
  for (int r = 0; r < (K::NBW > 0 ? K::NBW : 1); ++r) acc_z[r] = f32x4{};

  // z_i tile -> LDS, straight from global memory (bytes past the last key
  // read as zeros through the bounds-checked resource).  Issued from
  // assembly (lds_load16), so that the compiler does not make the pair
  // product's LDS reads wait for the next tile's z in flight; the tile
  // barrier waits for it.
  const bf16* zrow = CZ > 0 ? a.z + (int64_t)res * L * CZ : nullptr;
  auto issue_z = [&](int kt, int buf) {
    if constexpr (CZ > 0) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(zrow, (int64_t)L * CZ * 2);
      constexpr int CHUNKS = BN * CZ / 8;  // 16-byte chunks of a tile
#pragma unroll
      for (int c0 = 0; c0 < CHUNKS; c0 += 256) {
        const int chunk = c0 + w * 64 + lane;  // wave-uniform LDS base, lanes in order
        lds_load16(rs, zs + buf * BN * CZ + (c0 + w * 64) * 8, kt * BN * CZ * 2 + chunk * 16);
      }
    }
  };

  const int n_kt = (L + BN - 1) / BN;
  if (n_kt > 0) issue_z(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    // Every lane loads its key's data unconditionally (keys past L and idle
    // waves read a valid key's bytes), so that all loads of a tile go out
    // together instead of behind the key-mask load; the mask and the bounds
    // enter as a select on the logit.
    const int j = kt * BN + lane;
    const int jj = min(j, L - 1);
    bool valid = active && j < L;
    if (a.kmask) valid = valid && a.kmask[(int64_t)b * L + jj] != 0;
    float s;
    float vv[C], vg[PV][3];
    {
      const int64_t kres = (int64_t)b * L + jj;
      const int64_t krow = kres * H + hh;
      const float* Rj = a.rot + kres * 9;
      const float* tj = a.trans + kres * 3;
      float R[9], tt[3];
#pragma unroll
      for (int e = 0; e < 9; ++e) R[e] = Rj[e];
#pragma unroll
      for (int e = 0; e < 3; ++e) tt[e] = tj[e];
      // scalar part
      float dot = 0.0f;
      {
        const bf16x8* kp = (const bf16x8*)(a.k + krow * C);
        const bf16x8* vp = (const bf16x8*)(a.v + krow * C);
#pragma unroll
        for (int t = 0; t < C / 8; ++t) {
          const bf16x8 kx = kp[t], vx = vp[t];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            dot = fmaf(qf[8 * t + e], (float)kx[e], dot);
            vv[8 * t + e] = (float)vx[e];
          }
        }
      }
      // point distances: plain differences of global coordinates
      float d2 = 0.0f;
      {
        const f32x4* kp4 = (const f32x4*)(a.k_pts + krow * PQ * 3);
        float kl[PQ * 3];
#pragma unroll
        for (int t = 0; t < PQ * 3 / 4; ++t) {
          const f32x4 x = kp4[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) kl[4 * t + e] = x[e];
        }
#pragma unroll
        for (int p = 0; p < PQ; ++p)
#pragma unroll
          for (int r = 0; r < 3; ++r) {
            const float g = fmaf(R[3 * r], kl[3 * p], fmaf(R[3 * r + 1], kl[3 * p + 1], fmaf(R[3 * r + 2], kl[3 * p + 2], tt[r])));
            const float d = qg[p][r] - g;
            d2 = fmaf(d, d, d2);
          }
      }
      s = dot - wpt * d2;
      if (a.bias) s = fmaf(a.w_bias, (float)a.bias[(((int64_t)b * H + hh) * L + i) * L + jj], s);
      // value points in the global frame
      {
        const f32x4* vp4 = (const f32x4*)(a.v_pts + krow * PV * 3);
        float vl[PV * 3];
#pragma unroll
        for (int t = 0; t < PV * 3 / 4; ++t) {
          const f32x4 x = vp4[t];
#pragma unroll
          for (int e = 0; e < 4; ++e) vl[4 * t + e] = x[e];
        }
#pragma unroll
        for (int p = 0; p < PV; ++p)
#pragma unroll
          for (int r = 0; r < 3; ++r)
            vg[p][r] = fmaf(R[3 * r], vl[3 * p], fmaf(R[3 * r + 1], vl[3 * p + 1], fmaf(R[3 * r + 2], vl[3 * p + 2], tt[r])));
      }
    }
    // a key outside the mask may hold anything: nothing of it reaches a sum
    s = valid ? s : kNegInf;
#pragma unroll
    for (int c = 0; c < C; ++c) vv[c] = valid ? vv[c] : 0.0f;
#pragma unroll
    for (int p = 0; p < PV; ++p)
#pragma unroll
      for (int r = 0; r < 3; ++r) vg[p][r] = valid ? vg[p][r] : 0.0f;
    // online softmax: the head's maximum moves, partial sums rescale
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = m_new == kNegInf ? 1.0f : fast_exp2(m_run - m_new);
    const float p = valid ? fast_exp2(s - m_new) : 0.0f;
    m_run = m_new;
    l_lane = fmaf(l_lane, alpha, p);
#pragma unroll
    for (int c = 0; c < C; ++c) acc_o[c] = fmaf(acc_o[c], alpha, p * vv[c]);
#pragma unroll
    for (int q = 0; q < PV; ++q)
#pragma unroll
      for (int r = 0; r < 3; ++r) acc_g[q][r] = fmaf(acc_g[q][r], alpha, p * vg[q][r]);
    if constexpr (CZ > 0) {
      if (active) {
        ps[buf][w * BN + lane] = (bf16)p;
        if (lane == 0) als[buf][w] = alpha;
      }
      // this tile's z landed (own loads), weights written: publish
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + 1 < n_kt) issue_z(kt + 1, buf ^ 1);
      // pair output: D[h][n] += sum_j P[h][j] z[j][n] on the matrix cores;
      // lane l holds rows 4(l/16)..+3 of column l%16 of its 16-column block
      const int g = lane >> 4, i16 = lane & 15;
      const f32x4 al = *(const f32x4*)&als[buf][4 * g];
#pragma unroll
      for (int r = 0; r < K::NBW; ++r) {
        const int nb = w + r * HW;
        if (nb < K::NBZ) {
          acc_z[r] *= al;
#pragma unroll
          for (int ks = 0; ks < BN / 32; ++ks) {
            const bf16x8 pa = *(const bf16x8*)&ps[buf][i16 * BN + 32 * ks + 8 * g];
            const bf16* zb = zs + buf * BN * CZ + (32 * ks + 8 * g + (i16 >> 2)) * CZ + 16 * nb + 4 * (i16 & 3);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(zb));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(zb + 4 * CZ));
            const bf16x8 zb8 = __builtin_bit_cast(
                bf16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            acc_z[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, zb8, acc_z[r], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: reduce over the wave, normalise, store ---------------------
  // The per-lane partial sums (C values, PV x 3 point coordinates, l) go
  // through LDS: each quad of lanes adds its four (two DPP steps), one lane
  // of each quad writes the quad sums into this wave's block (row = value,
  // column = quad), and lane r adds row r's 16 quad sums (the lanes of the
  // points take the three rows of theirs).  The z tiles (or a buffer of its
  // own without z) hold the blocks once every wave is past the last tile.
  constexpr int NR = C + 3 * PV + 1;  // rows: values, point coordinates, l
  constexpr int RS = 20;              // row stride in floats (16 quads, 16-byte rows)
  constexpr int RED = HW * NR * RS;
  __shared__ __attribute__((aligned(16))) float red_own[CZ > 0 ? 4 : RED];
  static_assert(CZ == 0 || 2 * BN * CZ * 2 >= RED * 4, "reduction blocks in the z tiles");
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float* red = (CZ > 0 ? (float*)zs : red_own) + w * NR * RS;
  auto put = [&](int row, float x) {
    x += dpp_f32<0xb1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f32<0x4e>(x);  // quad_perm [2,3,0,1]
    if ((lane & 3) == 0) red[row * RS + (lane >> 2)] = x;
  };
#pragma unroll
  for (int c = 0; c < C; ++c) put(c, acc_o[c]);
#pragma unroll
  for (int q = 0; q < PV; ++q)
#pragma unroll
    for (int r = 0; r < 3; ++r) put(C + 3 * q + r, acc_g[q][r]);
  put(NR - 1, l_lane);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  auto row_total = [&](int row) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = *(const f32x4*)(red + row * RS + 4 * k);
      t += (v[0] + v[1]) + (v[2] + v[3]);
    }
    return t;
  };
  const float t0 = row_total(min(lane, NR - 1));
  const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t0), NR - 1));
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (active && lane < C) a.o[qrow * C + lane] = (bf16)(t0 * inv);
  if (active && lane >= C && lane < C + PV) {
    // back to the query residue's frame: R_i^T (y - t_i); no key: 0
    const int q = lane - C;
    const float g0 = row_total(C + 3 * q) * inv, g1 = row_total(C + 3 * q + 1) * inv,
                g2 = row_total(C + 3 * q + 2) * inv;
    const float d0 = g0 - ti[0], d1 = g1 - ti[1], d2 = g2 - ti[2];
    float* pp = a.o_pts + (qrow * PV + q) * 3;
#pragma unroll
    for (int r = 0; r < 3; ++r)
      pp[r] = l > 0.0f ? fmaf(Ri[r], d0, fmaf(Ri[3 + r], d1, Ri[6 + r] * d2)) : 0.0f;
  }
  if constexpr (CZ > 0) {
    if (lane == 0) lsum[w] = l;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int g = lane >> 4, i16 = lane & 15;
    if (g == 0) {
#pragma unroll
      for (int r = 0; r < K::NBW; ++r) {
        const int nb = w + r * HW;
        if (nb < K::NBZ) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int he = hg * HW + e;  // rows 0..3 of the block are this group's heads
            if (he < H) {
              const float le = lsum[e];
              a.o_pair[((int64_t)res * H + he) * CZ + 16 * nb + i16] =
                  (bf16)(le > 0.0f ? acc_z[r][e] / le : 0.0f);
            }
          }
        }
      }
    }
  }
}

}  // namespace fl
