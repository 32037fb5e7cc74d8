// bfloat16 backward kernels on 32x32 MFMA tiles.
//
// Same mathematics and ownership as dq_kernel / dkv_kernel ("Flash Attention
// 2 -- backward pass notes", sections "The math (FA2 backward with
// recompute)" and option 3 of "Why the WGSL kernel isn't shipped this
// turn"): the dQ kernel owns query tiles, the dK/dV kernel owns key tiles,
// P = exp(S - L) is recomputed in both, and dS = P (dP - D).
//  * dQ kernel: each wave owns 32 query rows (Q and dO fragments in
//    registers).  Per key block: S^T = K Q^T and dP^T = V dO^T with K, V
//    from the LDS block; dQ^T += K^T dS^T with K^T by LDS transpose reads.
//  * dK/dV kernel: each wave owns 32 key rows (K and V fragments in
//    registers).  Per query block: S = Q K^T and dP = dO V^T with Q, dO from
//    the LDS block; dV^T += dO^T P and dK^T += Q^T dS with the transposed
//    operands by LDS transpose reads.
//  * Blocks clear of the causal diagonal and of the sequence end take a path
//    with no masks and no per-tile branches; the others mask element-wise and
//    skip 32-row tiles wholly on the masked side of the diagonal.
#pragma once
#include <type_traits>

#include "fa_bwd.hpp"
#include "fa_mfma32.hpp"

namespace fa {

// FUSE_D: compute D_i = <dO_i, O_i> for the tile's rows from O (float32) and
// the dO fragments already in registers, and write it to a.delta, instead of
// reading a.delta (the pre-pass folded into this kernel).
template <int HD, bool CAUSAL, int PREC, int NW, int BC, bool FUSE_D>
__global__ __launch_bounds__(NW * 64, HD <= 64 ? 2 : 1) void dq32_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int LD = HD + 8;
  constexpr int NDT = HD / 32;
  constexpr int NKS = HD / 16;
  constexpr int NKT = BC / 32;
  static_assert(HD % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(2 * 2 * BC * LD * 2 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) bf16_t sK[2][BC * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][BC * LD];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  const int nqt = (T + BR - 1) / BR;
  const int total = nqt * a.B * H;
  for (int round = 0;; ++round) {
    const int w = persistent_item(round, total);
    if (w < 0) break;
  const int bh = w / nqt;
  const int qt = nqt - 1 - (w % nqt);
  const int b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * HD;
  const size_t base = ((size_t)b * T * H + hh) * HD;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + base;
  const bf16_t* K = static_cast<const bf16_t*>(a.k) + base;
  const bf16_t* V = static_cast<const bf16_t*>(a.v) + base;
  const bf16_t* dO = static_cast<const bf16_t*>(a.dO) + base;
  const int i0 = qt * BR;
  const int r0 = i0 + wave * 32;
  const int row = r0 + n;
  const float c2 = a.c2;
  const int vis = (CAUSAL ? min(row, T - 1) : T - 1) - 4 * h;

  bf16x8 qf[NKS], gf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = ld_row_global32(Q, rs, row, T, 16 * ks, h);
    gf[ks] = ld_row_global32(dO, rs, row, T, 16 * ks, h);
  }
  float l2 = INFINITY, dd = 0.f;
  if (FUSE_D) {
    // lane (n, h) holds dO[row][16 ks + 8h .. +7]; its partner (n, 1-h) the rest
    float part = 0.f;
    if (row < T) {
      const float* orow = a.o + base + (size_t)row * rs;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(orow + 16 * ks + 8 * h);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(orow + 16 * ks + 8 * h + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) part += o0[e] * (float)gf[ks][e] + o1[e] * (float)gf[ks][4 + e];
      }
    }
    dd = part + __shfl_xor(part, 32);
    if (row < T && h == 0) a.delta[(size_t)bh * T + row] = dd;
  }
  if (row < T) {
    l2 = a.lse[(size_t)bh * T + row] * kLog2e;
    if (l2 == -INFINITY) l2 = INFINITY;  // a row that saw no key has zero gradient
    if (!FUSE_D) dd = a.delta[(size_t)bh * T + row];
  }
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();

  const int last_row = min(i0 + BR, T) - 1;
  const int nkb = CAUSAL ? (last_row / BC + 1) : (T + BC - 1) / BC;

  TileCopy<bf16_t, HD, BC, NT> ck, cv;
  ck.load(K, rs, 0, T, tid);
  cv.load(V, rs, 0, T, tid);
  ck.store(sK[0], LD, tid);
  cv.store(sV[0], LD, tid);
  __syncthreads();

  auto block = [&](const bf16_t* cK, const bf16_t* cV, const int j0, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    auto live = [&](int kt) { return !(MASK && CAUSAL) || (j0 + 32 * kt <= r0 + 31); };
    f32x16 s[NKT], dp[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = dp[kt] = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        if (live(kt)) {
          s[kt] = mma32(ld_row32(cK, LD, 32 * kt, 16 * ks, n, h), qf[ks], s[kt]);
          dp[kt] = mma32(ld_row32(cV, LD, 32 * kt, 16 * ks, n, h), gf[ks], dp[kt]);
        }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      if (!live(kt)) continue;
      const int lim = vis - (j0 + 32 * kt);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = fast_exp2(fmaf(s[kt][e], c2, -l2));
        if (MASK && 8 * (e >> 2) + (e & 3) > lim) p = 0.f;
        s[kt][e] = p * (dp[kt][e] - dd);
      }
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
      if (live(kt)) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 bf = pack32(s[kt], st);
          bf16x8 bl;
          if (PREC == 1) bl = pack32_lo(s[kt], st);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8 af = ld_tr32(cK, LD, 32 * kt + 16 * st, 32 * dt, lane);
            acc[dt] = mma32(af, bf, acc[dt]);
            if (PREC == 1) acc[dt] = mma32(af, bl, acc[dt]);
          }
        }
      }
  };

  for (int kb = 0; kb < nkb; ++kb) {
    const int j0 = kb * BC;
    const int buf = kb & 1;
    if (kb + 1 < nkb) {
      ck.load(K, rs, j0 + BC, T, tid);
      cv.load(V, rs, j0 + BC, T, tid);
    }
    if (!CAUSAL || j0 <= r0 + 31) {
      const bool need_mask = (CAUSAL && (j0 + BC - 1 > r0)) || (j0 + BC > T);
      if (need_mask)
        block(sK[buf], sV[buf], j0, std::true_type{});
      else
        block(sK[buf], sV[buf], j0, std::false_type{});
    }
    if (kb + 1 < nkb) {
      ck.store(sK[buf ^ 1], LD, tid);
      cv.store(sV[buf ^ 1], LD, tid);
    }
    __syncthreads();
  }

  if (row < T) {
    float* out = a.dq + base + (size_t)row * rs;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        f32x4 v4 = {acc[dt][4 * bb] * sc, acc[dt][4 * bb + 1] * sc, acc[dt][4 * bb + 2] * sc, acc[dt][4 * bb + 3] * sc};
        *reinterpret_cast<f32x4*>(out + 32 * dt + 8 * bb + 4 * h) = v4;
      }
  }
  }
}

template <int HD, bool CAUSAL, int PREC, int NW, int BQ>
__global__ __launch_bounds__(NW * 64, HD <= 64 ? 2 : 1) void dkv32_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;
  constexpr int LD = HD + 8;
  constexpr int NDT = HD / 32;
  constexpr int NKS = HD / 16;
  constexpr int NIT = BQ / 32;
  static_assert(HD % 32 == 0 && BQ % 32 == 0, "tile shape");
  static_assert(2 * 2 * BQ * LD * 2 + 2 * 2 * BQ * 4 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sG[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  const int nkt = (T + BK - 1) / BK;
  const int total = nkt * a.B * H;
  for (int round = 0;; ++round) {
    const int w = persistent_item(round, total);
    if (w < 0) break;
  const int bh = w / nkt;
  const int kt = w % nkt;
  const int b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * HD;
  const size_t base = ((size_t)b * T * H + hh) * HD;
  const bf16_t* Q = static_cast<const bf16_t*>(a.q) + base;
  const bf16_t* K = static_cast<const bf16_t*>(a.k) + base;
  const bf16_t* V = static_cast<const bf16_t*>(a.v) + base;
  const bf16_t* dO = static_cast<const bf16_t*>(a.dO) + base;
  const float* Lg = a.lse + (size_t)bh * T;
  const float* Dg = a.delta + (size_t)bh * T;
  const int j0w = kt * BK;
  const int c0 = j0w + wave * 32;  // first key of this wave
  const int col = c0 + n;          // this lane's key
  const float c2 = a.c2;
  // Element e of a query tile starting at row ir is masked (causal) iff
  // ir + 8*(e/4) + 4h + e%4 < col, i.e. 8*(e/4) + e%4 < lo - ir.
  const int lo = col - 4 * h;

  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = ld_row_global32(K, rs, col, T, 16 * ks, h);
    vf[ks] = ld_row_global32(V, rs, col, T, 16 * ks, h);
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = zero16();

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

  TileCopy<bf16_t, HD, BQ, NT> cq, cg;
  cq.load(Q, rs, qb0 * BQ, T, tid);
  cg.load(dO, rs, qb0 * BQ, T, tid);
  cq.store(sQ[0], LD, tid);
  cg.store(sG[0], LD, tid);
  load_ld(qb0, 0);
  __syncthreads();

  // One query block as a three-stage software pipeline over its 32-row
  // tiles: A(t) = the S and dP products, B(t) = P and dS in registers (VALU and
  // exp), C(t) = the dV and dK products.  The order A(t+1), B(t), C(t) keeps
  // independent matrix and vector work next to each other in one basic block.
  auto block = [&](const bf16_t* cQ, const bf16_t* cG, const float* cL, const float* cD, const int q0,
                   auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    f32x16 s[2], dp[2];
    auto stage_a = [&](int it, f32x16& sa, f32x16& da) {
      sa = zero16();
      da = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sa = mma32(ld_row32(cQ, LD, 32 * it, 16 * ks, n, h), kf[ks], sa);
        da = mma32(ld_row32(cG, LD, 32 * it, 16 * ks, n, h), vf[ks], da);
      }
    };
    stage_a(0, s[0], dp[0]);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      f32x16& sc = s[it & 1];
      f32x16& dc = dp[it & 1];
      if (it + 1 < NIT) stage_a(it + 1, s[(it + 1) & 1], dp[(it + 1) & 1]);
      // stage B: P = exp2(S c - L), dS = P (dP - D), packed for the products
      const int lim = lo - (q0 + 32 * it);
      bf16x8 bp[2], bs[2], bpl[2], bsl[2];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int rr = 32 * it + 8 * bb + 4 * h;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&cL[rr]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&cD[rr]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * bb + r;
          float p = fast_exp2(fmaf(sc[e], c2, -lv[r]));
          if (MASK && CAUSAL && 8 * bb + r < lim) p = 0.f;
          sc[e] = p;
          dc[e] = p * (dc[e] - d4[r]);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bp[st] = pack32(sc, st);
        bs[st] = pack32(dc, st);
        if (PREC == 1) {
          bpl[st] = pack32_lo(sc, st);
          bsl[st] = pack32_lo(dc, st);
        }
      }
      // stage C
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 ga = ld_tr32(cG, LD, 32 * it + 16 * st, 32 * dt, lane);
          const bf16x8 qa = ld_tr32(cQ, LD, 32 * it + 16 * st, 32 * dt, lane);
          dv[dt] = mma32(ga, bp[st], dv[dt]);
          dk[dt] = mma32(qa, bs[st], dk[dt]);
          if (PREC == 1) {
            dv[dt] = mma32(ga, bpl[st], dv[dt]);
            dk[dt] = mma32(qa, bsl[st], dk[dt]);
          }
        }
    }
  };

  for (int qb = qb0; qb < nqb; ++qb) {
    const int q0 = qb * BQ;
    const int buf = (qb - qb0) & 1;
    if (qb + 1 < nqb) {
      cq.load(Q, rs, q0 + BQ, T, tid);
      cg.load(dO, rs, q0 + BQ, T, tid);
    }
    if (!CAUSAL || q0 + BQ - 1 >= c0) {
      const bool need_mask = CAUSAL && (q0 < c0 + 31);
      if (need_mask)
        block(sQ[buf], sG[buf], sL[buf], sD[buf], q0, std::true_type{});
      else
        block(sQ[buf], sG[buf], sL[buf], sD[buf], q0, std::false_type{});
    }
    if (qb + 1 < nqb) {
      cq.store(sQ[buf ^ 1], LD, tid);
      cg.store(sG[buf ^ 1], LD, tid);
      load_ld(qb + 1, buf ^ 1);
    }
    __syncthreads();
  }

  if (col < T) {
    float* outk = a.dk + base + (size_t)col * rs;
    float* outv = a.dv + base + (size_t)col * rs;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        f32x4 k4 = {dk[dt][4 * bb] * sc, dk[dt][4 * bb + 1] * sc, dk[dt][4 * bb + 2] * sc, dk[dt][4 * bb + 3] * sc};
        f32x4 v4 = {dv[dt][4 * bb], dv[dt][4 * bb + 1], dv[dt][4 * bb + 2], dv[dt][4 * bb + 3]};
        *reinterpret_cast<f32x4*>(outk + 32 * dt + 8 * bb + 4 * h) = k4;
        *reinterpret_cast<f32x4*>(outv + 32 * dt + 8 * bb + 4 * h) = v4;
      }
  }
  }
}

}  // namespace fa
