// Backward kernels: recompute P from the saved log-sum-exp, no float atomics.
//
// "Flash Attention 2 -- backward pass notes", section "The math (FA2 backward
// with recompute)": per query row i and visible key j,
//   P = exp(S - L_i), dP = <dO_i, v_j>, dS = P (dP - D_i),
//   dQ_i += scale dS k_j, dK_j += scale dS q_i, dV_j += P dO_i,
// with D_i = <dO_i, O_i>.  Section "Why the WGSL kernel isn't shipped this
// turn", options 1 and 3, give the structure used here: a pre-pass writes D to
// a [B, H, T] buffer; one kernel owns query tiles and produces dQ; another
// owns key tiles and produces dK and dV.  Every output element has exactly one
// owning workgroup, so nothing accumulates across workgroups.
//
// Both main kernels keep the tile they own in registers and stream the other
// side through LDS in double-buffered blocks, like the forward kernel.
//  * dQ kernel: lanes own query rows.  S^T = K Q^T and dP^T = V dO^T give each
//    lane one query row; dS^T feeds dQ^T += K^T dS^T directly from registers.
//  * dK/dV kernel: lanes own key rows.  S = Q K^T and dP = dO V^T give each
//    lane one key column; P and dS feed dV^T += dO^T P and dK^T += Q^T dS.
#pragma once
#include <type_traits>
#include "fa_common.hpp"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const float* lse;
  const void* dO;
  float* dq;
  float* dk;
  float* dv;
  float* delta;
  int B, H, T;
  float scale;
  float c2;  // scale * log2(e)
};

// D[b, h, i] = <dO[b, i, h, :], O[b, i, h, :]>.  HD/4 lanes per row.
template <typename TIn, int HD>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a) {
  constexpr int LPR = HD / 4;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  const long row = (long)blockIdx.x * RPB + tid / LPR;  // row over (b, i, h)
  const long nrows = (long)a.B * a.T * a.H;
  float acc = 0.f;
  if (row < nrows) {
    const float4 o = *reinterpret_cast<const float4*>(a.o + row * HD + 4 * sub);
    float d0, d1, d2, d3;
    if (sizeof(TIn) == 4) {
      const float4 g = *reinterpret_cast<const float4*>(static_cast<const float*>(a.dO) + row * HD + 4 * sub);
      d0 = g.x, d1 = g.y, d2 = g.z, d3 = g.w;
    } else if (std::is_same<TIn, f16_t>::value) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 g = *reinterpret_cast<const h4*>(static_cast<const uint16_t*>(a.dO) + row * HD + 4 * sub);
      d0 = (float)g[0], d1 = (float)g[1], d2 = (float)g[2], d3 = (float)g[3];
    } else {
      const uint2 g = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.dO) + row * HD + 4 * sub);
      d0 = __uint_as_float(g.x << 16);
      d1 = __uint_as_float(g.x & 0xffff0000u);
      d2 = __uint_as_float(g.y << 16);
      d3 = __uint_as_float(g.y & 0xffff0000u);
    }
    acc = o.x * d0 + o.y * d1 + o.z * d2 + o.w * d3;
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && sub == 0) {
    const long h = row % a.H;
    const long bi = row / a.H;  // b * T + i
    const long b = bi / a.T, i = bi % a.T;
    a.delta[(b * a.H + h) * a.T + i] = acc;
  }
}

// dQ kernel: one workgroup per (query tile, batch*head).  Up to hd 64 the
// compiler is held to three resident waves per SIMD (at most 168 VGPRs; two
// values spill at float32 hd 64): 7% faster at float32, B64 H16 T1024 hd64.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int MR, int BC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(HD <= 64 ? 3 : 1))) void dq_kernel(
    BwdArgs a) {
  using M = Mma<TIn>;
  using frag = typename M::frag;
  constexpr int NT = NW * 64;
  constexpr int RW = 16 * MR;
  constexpr int BR = NW * RW;
  constexpr int LD = lds_ld<TIn, HD>();
  constexpr int NDT = (HD + 15) / 16;
  constexpr int NKS = HD / M::KS;
  constexpr int NCH = BC / M::CH;
  constexpr int TPC = M::CH / 16;
  static_assert(HD % M::KS == 0 && BC % M::CH == 0, "tile shape");
  static_assert(2 * 2 * BC * LD * sizeof(TIn) <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) TIn sK[2][BC * LD];
  __shared__ __attribute__((aligned(16))) TIn sV[2][BC * LD];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const int nqt = (T + BR - 1) / BR;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / nqt;
  const int qt = nqt - 1 - (w % nqt);
  const int b = bh / H, h = bh % H;
  const size_t rs = (size_t)H * HD;
  const size_t base = ((size_t)b * T * H + h) * HD;
  const TIn* Q = static_cast<const TIn*>(a.q) + base;
  const TIn* K = static_cast<const TIn*>(a.k) + base;
  const TIn* V = static_cast<const TIn*>(a.v) + base;
  const TIn* dO = static_cast<const TIn*>(a.dO) + base;
  const int i0 = qt * BR;
  const int r0 = i0 + wave * RW;
  const float c2 = a.c2;

  if (sizeof(TIn) == 4 && HD < 16) {
    for (int x = tid; x < 2 * BC * LD; x += NT) {
      (&sK[0][0])[x] = TIn{};
      (&sV[0][0])[x] = TIn{};
    }
    __syncthreads();
  }

  frag qf[MR][NKS], gf[MR][NKS];
  float l2[MR], dd[MR];
  f32x4 acc[NDT][MR];
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    const int i = r0 + 16 * mr + li;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[mr][ks] = M::ld_row_global(Q, rs, i, T, ks * M::KS, lg);
      gf[mr][ks] = M::ld_row_global(dO, rs, i, T, ks * M::KS, lg);
    }
    l2[mr] = (i < T) ? a.lse[(size_t)bh * T + i] * kLog2e : INFINITY;
    dd[mr] = (i < T) ? a.delta[(size_t)bh * T + i] : 0.f;
    // A row whose log-sum-exp is -inf saw no key; its gradient is zero.
    if (l2[mr] == -INFINITY) l2[mr] = INFINITY;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt][mr] = zero4();
  }

  const int last_row = min(i0 + BR, T) - 1;
  const int nkb = CAUSAL ? (last_row / BC + 1) : (T + BC - 1) / BC;

  TileCopy<TIn, HD, BC, NT> ck, cv;
  ck.load(K, rs, 0, T, tid);
  cv.load(V, rs, 0, T, tid);
  ck.store(sK[0], LD, tid);
  cv.store(sV[0], LD, tid);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int j0 = kb * BC;
    const int buf = kb & 1;
    if (kb + 1 < nkb) {
      ck.load(K, rs, j0 + BC, T, tid);
      cv.load(V, rs, j0 + BC, T, tid);
    }
    const TIn* cK = sK[buf];
    const TIn* cV = sV[buf];
    const bool active = !CAUSAL || (j0 <= r0 + RW - 1);
    const bool need_mask = (CAUSAL && (j0 + BC - 1 > r0)) || (j0 + BC > T);
    if (active) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        f32x4 s[MR][TPC], dp[MR][TPC];
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) s[mr][t] = dp[mr][t] = zero4();
          const int jr = ch * M::CH + 16 * t;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const frag ka = M::ld_row(cK, LD, jr, ks * M::KS, li, lg);
            const frag va = M::ld_row(cV, LD, jr, ks * M::KS, li, lg);
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              s[mr][t] = M::mma(ka, qf[mr][ks], s[mr][t]);
              dp[mr][t] = M::mma(va, gf[mr][ks], dp[mr][t]);
            }
          }
        }
        // s <- dS = P (dP - D)
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          const int i = r0 + 16 * mr + li;
#pragma unroll
          for (int t = 0; t < TPC; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float p = fast_exp2(fmaf(s[mr][t][r], c2, -l2[mr]));
              if (need_mask) {
                const int j = j0 + ch * M::CH + 16 * t + 4 * lg + r;
                if ((CAUSAL && j > i) || j >= T) p = 0.f;
              }
              s[mr][t][r] = p * (dp[mr][t][r] - dd[mr]);
            }
        }
#pragma unroll
        for (int st = 0; st < M::NSTEP; ++st) {
          frag bf[MR], bl[MR];
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            bf[mr] = M::pack(s[mr], st);
            if (PREC == 1) bl[mr] = M::pack_lo(s[mr], st);
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const frag af = M::ld_trans(cK, LD, ch * M::CH, 16 * dt, st, li, lg);
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              acc[dt][mr] = M::mma(af, bf[mr], acc[dt][mr]);
              if (PREC == 1) acc[dt][mr] = M::mma(af, bl[mr], acc[dt][mr]);
            }
          }
        }
      }
    }
    if (kb + 1 < nkb) {
      ck.store(sK[buf ^ 1], LD, tid);
      cv.store(sV[buf ^ 1], LD, tid);
    }
    __syncthreads();
  }

  float* dQ = a.dq + base;
  const float scale = a.scale;
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    const int i = r0 + 16 * mr + li;
    if (i < T) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + 4 * lg;
        if (d < HD) *reinterpret_cast<f32x4*>(dQ + (size_t)i * rs + d) = acc[dt][mr] * scale;
      }
    }
  }
}

// dK/dV kernel: one workgroup per (key tile, batch*head).  The compiler is
// held to two resident waves per SIMD (at most 256 VGPRs; left alone it takes
// 288 and one wave at float32 hd 64): 20% faster at float32, B64 H16 T1024
// hd64.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int MR, int BQ>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void dkv_kernel(
    BwdArgs a) {
  using M = Mma<TIn>;
  using frag = typename M::frag;
  constexpr int NT = NW * 64;
  constexpr int RW = 16 * MR;  // key rows per wave
  constexpr int BK = NW * RW;  // key rows per workgroup
  constexpr int LD = lds_ld<TIn, HD>();
  constexpr int NDT = (HD + 15) / 16;
  constexpr int NKS = HD / M::KS;
  constexpr int NCH = BQ / M::CH;
  constexpr int TPC = M::CH / 16;
  static_assert(HD % M::KS == 0 && BQ % M::CH == 0, "tile shape");
  static_assert(2 * 2 * BQ * LD * sizeof(TIn) + 2 * 2 * BQ * 4 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) TIn sQ[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) TIn sG[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  const int nkt = (T + BK - 1) / BK;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / nkt;
  const int kt = w % nkt;  // early key tiles see the most queries: first
  const int b = bh / H, h = bh % H;
  const size_t rs = (size_t)H * HD;
  const size_t base = ((size_t)b * T * H + h) * HD;
  const TIn* Q = static_cast<const TIn*>(a.q) + base;
  const TIn* K = static_cast<const TIn*>(a.k) + base;
  const TIn* V = static_cast<const TIn*>(a.v) + base;
  const TIn* dO = static_cast<const TIn*>(a.dO) + base;
  const float* Lg = a.lse + (size_t)bh * T;
  const float* Dg = a.delta + (size_t)bh * T;
  const int j0w = kt * BK;
  const int c0 = j0w + wave * RW;  // first key row of this wave
  const float c2 = a.c2;

  if (sizeof(TIn) == 4 && HD < 16) {
    for (int x = tid; x < 2 * BQ * LD; x += NT) {
      (&sQ[0][0])[x] = TIn{};
      (&sG[0][0])[x] = TIn{};
    }
    __syncthreads();
  }

  frag kf[MR][NKS], vf[MR][NKS];
  f32x4 dk[NDT][MR], dv[NDT][MR];
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    const int j = c0 + 16 * mr + li;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[mr][ks] = M::ld_row_global(K, rs, j, T, ks * M::KS, lg);
      vf[mr][ks] = neg_frag(M::ld_row_global(V, rs, j, T, ks * M::KS, lg));  // held negated: see dp below
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dk[dt][mr] = dv[dt][mr] = zero4();
  }

  // Query blocks that can see at least one key of this tile.
  const int qb0 = CAUSAL ? (j0w / BQ) : 0;
  const int nqb = (T + BQ - 1) / BQ;

  auto load_ld = [&](int blk, int sb) {
    for (int x = tid; x < BQ; x += NT) {
      const int i = blk * BQ + x;
      float l2 = INFINITY, d = 0.f;
      if (i < T) {
        l2 = Lg[i] * kLog2e;
        if (l2 == -INFINITY) l2 = INFINITY;
        d = Dg[i];
      }
      sL[sb][x] = l2;
      sD[sb][x] = d;
    }
  };

  TileCopy<TIn, HD, BQ, NT> cq, cg;
  cq.load(Q, rs, qb0 * BQ, T, tid);
  cg.load(dO, rs, qb0 * BQ, T, tid);
  cq.store(sQ[0], LD, tid);
  cg.store(sG[0], LD, tid);
  load_ld(qb0, 0);
  __syncthreads();

  for (int qb = qb0; qb < nqb; ++qb) {
    const int q0 = qb * BQ;
    const int buf = (qb - qb0) & 1;
    if (qb + 1 < nqb) {
      cq.load(Q, rs, q0 + BQ, T, tid);
      cg.load(dO, rs, q0 + BQ, T, tid);
    }
    const TIn* cQ = sQ[buf];
    const TIn* cG = sG[buf];
    const bool active = !CAUSAL || (q0 + BQ - 1 >= c0);
    const bool need_mask = CAUSAL && (q0 < c0 + RW - 1);
    if (active) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        f32x4 s[MR][TPC], dp[MR][TPC];
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
          const int ir = ch * M::CH + 16 * t;
          // dp starts from D of its rows and accumulates dO (-V)^T, giving
          // D - dP, so dS = P (dP - D) below takes one multiply
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[buf][ir + 4 * lg]);
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            s[mr][t] = zero4();
            dp[mr][t] = d4;
          }
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const frag qa = M::ld_row(cQ, LD, ir, ks * M::KS, li, lg);
            const frag ga = M::ld_row(cG, LD, ir, ks * M::KS, li, lg);
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              s[mr][t] = M::mma(qa, kf[mr][ks], s[mr][t]);
              dp[mr][t] = M::mma(ga, vf[mr][ks], dp[mr][t]);
            }
          }
        }
        // s <- P, dp <- dS.  Lane (li, lg) holds rows i = ir + 4*lg + r of key column li.
#pragma unroll
        for (int t = 0; t < TPC; ++t) {
          const int ir = ch * M::CH + 16 * t + 4 * lg;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(&sL[buf][ir]);
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            const int j = c0 + 16 * mr + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float p = fast_exp2(fmaf(s[mr][t][r], c2, -lv[r]));
              if (need_mask && (q0 + ir + r < j)) p = 0.f;
              s[mr][t][r] = p;
              dp[mr][t][r] = -(p * dp[mr][t][r]);  // dp held D - dP
            }
          }
        }
#pragma unroll
        for (int st = 0; st < M::NSTEP; ++st) {
          frag bp[MR], bs[MR], bpl[MR], bsl[MR];
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            bp[mr] = M::pack(s[mr], st);
            bs[mr] = M::pack(dp[mr], st);
            if (PREC == 1) {
              bpl[mr] = M::pack_lo(s[mr], st);
              bsl[mr] = M::pack_lo(dp[mr], st);
            }
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const frag ga = M::ld_trans(cG, LD, ch * M::CH, 16 * dt, st, li, lg);
            const frag qa = M::ld_trans(cQ, LD, ch * M::CH, 16 * dt, st, li, lg);
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              dv[dt][mr] = M::mma(ga, bp[mr], dv[dt][mr]);
              dk[dt][mr] = M::mma(qa, bs[mr], dk[dt][mr]);
              if (PREC == 1) {
                dv[dt][mr] = M::mma(ga, bpl[mr], dv[dt][mr]);
                dk[dt][mr] = M::mma(qa, bsl[mr], dk[dt][mr]);
              }
            }
          }
        }
      }
    }
    if (qb + 1 < nqb) {
      cq.store(sQ[buf ^ 1], LD, tid);
      cg.store(sG[buf ^ 1], LD, tid);
      load_ld(qb + 1, buf ^ 1);
    }
    __syncthreads();
  }

  float* dK = a.dk + base;
  float* dV = a.dv + base;
  const float scale = a.scale;
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    const int j = c0 + 16 * mr + li;
    if (j < T) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + 4 * lg;
        if (d < HD) {
          *reinterpret_cast<f32x4*>(dK + (size_t)j * rs + d) = dk[dt][mr] * scale;
          *reinterpret_cast<f32x4*>(dV + (size_t)j * rs + d) = dv[dt][mr];
        }
      }
    }
  }
}

}  // namespace fa
