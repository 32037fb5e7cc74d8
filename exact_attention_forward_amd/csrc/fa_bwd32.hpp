// 16-bit (bfloat16 or IEEE half) dQ kernel on 32x32 MFMA tiles.
//
// Same mathematics and ownership as dq_kernel ("Flash Attention 2 -- backward
// pass notes", sections "The math (FA2 backward with recompute)" and option 3
// of "Why the WGSL kernel isn't shipped this turn"): the kernel owns query
// tiles and recomputes P = exp(S - L); dS = P (dP - D).  Each wave owns 32
// query rows (Q and dO fragments in registers).  Per key block: S^T = K Q^T
// and dP^T = V dO^T with K, V from the LDS block; dQ^T += K^T dS^T with K^T
// by LDS transpose reads.  Blocks clear of the causal diagonal and of the
// sequence end take a path with no masks and no per-tile branches; the others
// mask element-wise and skip 32-key tiles wholly on the masked side of the
// diagonal.  (The dK/dV kernels: dkv64_kernel for hd 64, the 16x16 dkv_kernel
// otherwise.)
#pragma once
#include <type_traits>

#include "fa_bwd.hpp"
#include "fa_mfma32.hpp"

#ifndef FA_DQ_OCC128
#define FA_DQ_OCC128 2  // two waves per SIMD at hd 128 (D from the pre-pass; hd 128 reaches this
                        // kernel only under the causal mask)
#endif

namespace fa {

// FUSE_D: compute D_i = <dO_i, O_i> for the tile's rows from O (float32) and
// the dO fragments already in registers, and write it to a.delta, instead of
// reading a.delta (the pre-pass folded into this kernel).
//
// Like the dK/dV kernel, each workgroup walks one continuous stream of (query
// tile, key block) pairs: the last key block of a tile fetches the first key
// block of the workgroup's next tile, and requests the next tile's Q, dO (and
// O) rows as soon as its own S and dP products no longer need the current
// ones (under the causal mask; without it, right after that block, where
// fewer values are live), so a new tile starts with its first block in LDS.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int BC, bool FUSE_D>
__global__ __launch_bounds__(NW * 64, HD <= 64 ? 2 : FA_DQ_OCC128) void dq32_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int LD = HD <= 64 ? HD + 8 : HD + 24;  // LDS row pitch (elements); see lds_ld
  constexpr int NDT = HD / 32;
  constexpr int NKS = HD / 16;
  constexpr int NKT = BC / 32;
  using V8 = typename Frag32<TIn>::V;
  static_assert(HD % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(2 * 2 * BC * LD * 2 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) bf16_t sK[2][BC * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][BC * LD];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const size_t rs = (size_t)H * HD;
  const float c2 = a.c2;
  const int nqt = (T + BR - 1) / BR;
  const int total = nqt * a.B * H;
  const bf16_t* Qg = static_cast<const bf16_t*>(a.q);
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* Vg = static_cast<const bf16_t*>(a.v);
  const bf16_t* Gg = static_cast<const bf16_t*>(a.dO);

  // work item w = (batch-head w / nqt, query tile nqt - 1 - w % nqt): long tiles first
  auto item_base = [&](int w) {
    const int bh = w / nqt;
    return ((size_t)(bh / H) * T * H + bh % H) * HD;
  };
  auto item_i0 = [&](int w) { return (nqt - 1 - w % nqt) * BR; };
  auto item_nkb = [&](int w) {
    const int last_row = min(item_i0(w) + BR, T) - 1;
    return CAUSAL ? (last_row / BC + 1) : (T + BC - 1) / BC;
  };

  TileCopy<bf16_t, HD, BC, NT> ck, cv;
  auto fetch = [&](int w, int kb) {
    const size_t bs = item_base(w);
    ck.load(Kg + bs, rs, kb * BC, T, tid);
    cv.load(Vg + bs, rs, kb * BC, T, tid);
  };
  auto commit = [&](int sb) {
    ck.store(sK[sb], LD, tid);
    cv.store(sV[sb], LD, tid);
  };

  // Rows of this lane: Q and dO fragments, O for D, raw L (and D).  Rows past T
  // read row T-1; their results are never stored.
  V8 qf[NKS], gf[NKS];
  f32x4 of[FUSE_D ? 2 * NKS : 1];
  float lraw = 0.f, draw = 0.f;
  auto load_rows = [&](int w) {
    const size_t bs = item_base(w);
    const int rc = min(item_i0(w) + wave * 32 + n, T - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = *reinterpret_cast<const V8*>(Qg + bs + (size_t)rc * rs + 16 * ks + 8 * h);
      gf[ks] = *reinterpret_cast<const V8*>(Gg + bs + (size_t)rc * rs + 16 * ks + 8 * h);
      if (FUSE_D) {
        // lane (n, h) holds dO[row][16 ks + 8h .. +7]; its partner (n, 1-h) the rest
        of[2 * ks] = *reinterpret_cast<const f32x4*>(a.o + bs + (size_t)rc * rs + 16 * ks + 8 * h);
        of[2 * ks + 1] = *reinterpret_cast<const f32x4*>(a.o + bs + (size_t)rc * rs + 16 * ks + 8 * h + 4);
      }
    }
    const size_t r = (size_t)(w / nqt) * T + rc;
    lraw = a.lse[r];
    if (!FUSE_D) draw = a.delta[r];
  };

  int w = persistent_item(0, total);
  if (w < 0) return;
  fetch(w, 0);
  load_rows(w);
  commit(0);
  __syncthreads();
  int buf = 0;

  for (int round = 0;; ++round) {
    const size_t base = item_base(w);
    const int i0 = item_i0(w);
    const int r0 = i0 + wave * 32;
    const int row = r0 + n;
    const int nkb = item_nkb(w);
    const int vis = (CAUSAL ? min(row, T - 1) : T - 1) - 4 * h;
    float dd = draw;
    if (FUSE_D) {
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          part += of[2 * ks][e] * (float)gf[ks][e] + of[2 * ks + 1][e] * (float)gf[ks][4 + e];
      dd = part + __shfl_xor(part, 32);
      if (row < T && h == 0) a.delta[(size_t)(w / nqt) * T + row] = dd;
    }
    float l2 = row < T ? lraw * kLog2e : INFINITY;
    if (l2 == -INFINITY) l2 = INFINITY;  // a row that saw no key has zero gradient
    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();

    // next_rows >= 0: after the S and dP products, request the rows of item next_rows
    auto block = [&](const bf16_t* cK, const bf16_t* cV, const int j0, const int next_rows, auto masked) {
      constexpr bool MASK = decltype(masked)::value;
      // keeps the two variants' LDS reads apart (hoisted above the branch,
      // they stay live across it and spill)
      asm volatile("" ::: "memory");
      auto live = [&](int kt) { return !(MASK && CAUSAL) || (j0 + 32 * kt <= r0 + 31); };
      f32x16 s[NKT], dp[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = dp[kt] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
          if (live(kt)) {
            s[kt] = mma32(ld_row32<V8>(cK, LD, 32 * kt, 16 * ks, n, h), qf[ks], s[kt]);
            dp[kt] = mma32(ld_row32<V8>(cV, LD, 32 * kt, 16 * ks, n, h), gf[ks], dp[kt]);
          }
      if (next_rows >= 0) load_rows(next_rows);
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
            const V8 bf = pack32<V8>(s[kt], st);
            V8 bl;
            if (PREC == 1) bl = pack32_lo<V8>(s[kt], st);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const V8 af = ld_tr32<V8>(cK, LD, 32 * kt + 16 * st, 32 * dt, lane);
              acc[dt] = mma32(af, bf, acc[dt]);
              if (PREC == 1) acc[dt] = mma32(af, bl, acc[dt]);
            }
          }
        }
    };

    auto step = [&](const int kb, const int next_rows) {
      const int j0 = kb * BC;
      if (!CAUSAL || j0 <= r0 + 31) {
        const bool need_mask = (CAUSAL && (j0 + BC - 1 > r0)) || (j0 + BC > T);
        if (need_mask)
          block(sK[buf], sV[buf], j0, next_rows, std::true_type{});
        else
          block(sK[buf], sV[buf], j0, next_rows, std::false_type{});
      } else if (next_rows >= 0) {
        load_rows(next_rows);  // this wave skips the block
      }
    };
    for (int kb = 0; kb + 1 < nkb; ++kb) {
      fetch(w, kb + 1);
      step(kb, -1);
      commit(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    // The last block is peeled so that the next rows, loaded inside it, are
    // not live across the loop.
    const int wn = persistent_item(round + 1, total);
    if (wn >= 0) fetch(wn, 0);
    // (without the mask the compiler keeps more of the block live and the
    // early row loads spill; there they follow the block)
    step(nkb - 1, CAUSAL ? wn : -1);
    if (!CAUSAL && wn >= 0) load_rows(wn);
    if (wn >= 0) commit(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    if (wn >= 0) {
      // Wait for the next rows here, before the stores below: once loads and
      // stores are in flight together, a wait for a load also waits for every
      // store.
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(gf[ks]));
      if (FUSE_D)
#pragma unroll
        for (int x = 0; x < 2 * NKS; ++x) asm volatile("" ::"v"(of[x]));
      asm volatile("" ::"v"(lraw), "v"(draw));
    }

    if (row < T) {
      float* out = a.dq + base + (size_t)row * rs;
      const float sc = a.scale;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          f32x4 v4 = {acc[dt][4 * bb] * sc, acc[dt][4 * bb + 1] * sc, acc[dt][4 * bb + 2] * sc,
                      acc[dt][4 * bb + 3] * sc};
          *reinterpret_cast<f32x4*>(out + 32 * dt + 8 * bb + 4 * h) = v4;
        }
    }
    if (wn < 0) break;
    w = wn;
  }
}

}  // namespace fa
