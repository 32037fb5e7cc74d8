// 16-bit (bfloat16 or IEEE half) backward kernels on 32x32 MFMA tiles.
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

// The dK/dV kernel walks one continuous stream of (key tile, query block)
// pairs per workgroup: while a block is computed, the next one is fetched
// into registers (the next query block of the tile, or the first one of the
// workgroup's next tile), so a new tile starts with its first block already in
// LDS.  The next tile's K and V fragments are requested before the finished
// tile's dK and dV are stored, so waiting for them never waits for the stores.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int BQ>
__global__ __launch_bounds__(NW * 64, HD <= 64 ? 2 : 1) void dkv32_kernel(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;
  constexpr int LD = HD <= 64 ? HD + 8 : HD + 24;  // LDS row pitch (elements); see lds_ld
  constexpr int NDT = HD / 32;
  constexpr int NKS = HD / 16;
  constexpr int NIT = BQ / 32;
  using V8 = typename Frag32<TIn>::V;
  static_assert(HD % 32 == 0 && BQ % 32 == 0, "tile shape");
  static_assert(BQ <= NT, "one thread per query row fetches that row's L and D");
  static_assert(2 * 2 * BQ * LD * 2 + 2 * 2 * BQ * 4 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(16))) bf16_t sQ[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sG[2][BQ * LD];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const size_t rs = (size_t)H * HD;
  const float c2 = a.c2;
  const int nkt = (T + BK - 1) / BK;
  const int nqb = (T + BQ - 1) / BQ;
  const int total = nkt * a.B * H;
  const bf16_t* Qg = static_cast<const bf16_t*>(a.q);
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* Vg = static_cast<const bf16_t*>(a.v);
  const bf16_t* Gg = static_cast<const bf16_t*>(a.dO);

  // work item w = (batch-head w / nkt, key tile w % nkt)
  auto item_base = [&](int w) {
    const int bh = w / nkt;
    return ((size_t)(bh / H) * T * H + bh % H) * HD;
  };
  auto item_qb0 = [&](int w) { return CAUSAL ? (w % nkt) * BK / BQ : 0; };

  TileCopy<bf16_t, HD, BQ, NT> cq, cg;
  // L and D of query row tid of the fetched block, converted only when they
  // are written to LDS so that the loads are not waited for early
  // (rows past T read row T-1 and are zeroed on the way into LDS)
  float lnext = 0.f, dnext = 0.f;
  int qnext = 0;
  auto fetch = [&](int w, int qb) {
    const size_t bs = item_base(w);
    cq.load(Qg + bs, rs, qb * BQ, T, tid);
    cg.load(Gg + bs, rs, qb * BQ, T, tid);
    qnext = qb * BQ;
    if (tid < BQ) {
      const size_t r = (size_t)(w / nkt) * T + min(qb * BQ + tid, T - 1);
      lnext = a.lse[r];
      dnext = a.delta[r];
    }
  };
  auto commit = [&](int sb) {
    cq.store(sQ[sb], LD, tid);
    cg.store(sG[sb], LD, tid);
    if (tid < BQ) {
      const bool live = qnext + tid < T;
      const float l2 = lnext * kLog2e;
      // a row that saw no key, or a row past T, has zero gradient
      sL[sb][tid] = live && l2 != -INFINITY ? l2 : INFINITY;
      sD[sb][tid] = live ? dnext : 0.f;
    }
  };
  V8 kf[NKS], vf[NKS];
  auto load_kv = [&](int w) {
    const size_t bs = item_base(w);
    const int c = (w % nkt) * BK + wave * 32 + n;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = ld_row_global32<V8>(Kg + bs, rs, c, T, 16 * ks, h);
      vf[ks] = ld_row_global32<V8>(Vg + bs, rs, c, T, 16 * ks, h);
    }
  };

  int w = persistent_item(0, total);
  if (w < 0) return;
  fetch(w, item_qb0(w));
  load_kv(w);
  commit(0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));
  __syncthreads();
  int buf = 0;

  for (int round = 0;; ++round) {
    const size_t base = item_base(w);
    const int j0w = (w % nkt) * BK;
    const int c0 = j0w + wave * 32;  // first key of this wave
    const int col = c0 + n;          // this lane's key
    // Element e of a query tile starting at row ir is masked (causal) iff
    // ir + 8*(e/4) + 4h + e%4 < col, i.e. 8*(e/4) + e%4 < lo - ir.
    const int lo = col - 4 * h;
    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = zero16();

    // One query block as a three-stage software pipeline over its 32-row
    // tiles: A(t) = the S and dP products, B(t) = P and dS in registers (VALU
    // and exp), C(t) = the dV and dK products.  The order A(t+1), B(t), C(t)
    // keeps independent matrix and vector work next to each other.
    // FIRST: the first 32-row tile to visit; under the causal mask the tiles
    // before it lie wholly above this wave's first key (every P is zero).
    auto block = [&](const bf16_t* cQ, const bf16_t* cG, const float* cL, const float* cD, const int q0,
                     auto masked, auto first) {
      constexpr bool MASK = decltype(masked)::value;
      constexpr int FIRST = decltype(first)::value;
      f32x16 s[2], dp[2];
      auto stage_a = [&](int it, f32x16& sa, f32x16& da) {
        sa = zero16();
        da = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          sa = mma32(ld_row32<V8>(cQ, LD, 32 * it, 16 * ks, n, h), kf[ks], sa);
          da = mma32(ld_row32<V8>(cG, LD, 32 * it, 16 * ks, n, h), vf[ks], da);
        }
      };
      stage_a(FIRST, s[FIRST & 1], dp[FIRST & 1]);
#pragma unroll
      for (int it = FIRST; it < NIT; ++it) {
        f32x16& sc = s[it & 1];
        f32x16& dc = dp[it & 1];
        if (it + 1 < NIT) stage_a(it + 1, s[(it + 1) & 1], dp[(it + 1) & 1]);
        // stage B: P = exp2(S c - L), dS = P (dP - D), packed for the products
        const int lim = lo - (q0 + 32 * it);
        V8 bp[2], bs[2], bpl[2], bsl[2];
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
          bp[st] = pack32<V8>(sc, st);
          bs[st] = pack32<V8>(dc, st);
          if (PREC == 1) {
            bpl[st] = pack32_lo<V8>(sc, st);
            bsl[st] = pack32_lo<V8>(dc, st);
          }
        }
        // stage C
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const V8 ga = ld_tr32<V8>(cG, LD, 32 * it + 16 * st, 32 * dt, lane);
            const V8 qa = ld_tr32<V8>(cQ, LD, 32 * it + 16 * st, 32 * dt, lane);
            dv[dt] = mma32(ga, bp[st], dv[dt]);
            dk[dt] = mma32(qa, bs[st], dk[dt]);
            if (PREC == 1) {
              dv[dt] = mma32(ga, bpl[st], dv[dt]);
              dk[dt] = mma32(qa, bsl[st], dk[dt]);
            }
          }
      }
    };

    int wn = -1;
    for (int qb = item_qb0(w); qb < nqb; ++qb) {
      const int q0 = qb * BQ;
      const bool more = qb + 1 < nqb;
      int fw = w, fqb = qb + 1;  // the block to fetch: the tile's next one, or the next tile's first
      if (!more) {
        wn = persistent_item(round + 1, total);
        fw = wn;
        fqb = wn >= 0 ? item_qb0(wn) : 0;
      }
      if (fw >= 0) fetch(fw, fqb);
      if (!CAUSAL || q0 + BQ - 1 >= c0) {
        if (CAUSAL && q0 < c0 + 31) {
          // tiles wholly above the wave's first key are skipped (c0 - q0 is a
          // multiple of 32; the block is visited only if its last tile is live)
          const int it0 = q0 >= c0 ? 0 : (c0 - q0) >> 5;
          static_assert(NIT <= 4, "first-tile dispatch covers up to four tiles");
          auto masked = [&](auto f) { block(sQ[buf], sG[buf], sL[buf], sD[buf], q0, std::true_type{}, f); };
          if (it0 == 0) masked(std::integral_constant<int, 0>{});
          if constexpr (NIT > 1) if (it0 == 1) masked(std::integral_constant<int, 1>{});
          if constexpr (NIT > 2) if (it0 == 2) masked(std::integral_constant<int, 2>{});
          if constexpr (NIT > 3) if (it0 == 3) masked(std::integral_constant<int, 3>{});
        } else {
          block(sQ[buf], sG[buf], sL[buf], sD[buf], q0, std::false_type{}, std::integral_constant<int, 0>{});
        }
      }
      if (more || wn >= 0) commit(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    if (wn >= 0) {
      load_kv(wn);
      // Wait for the fragments here, before the stores below: once loads and
      // stores are in flight together, a wait for a load also waits for every
      // store.
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));
    }

    if (col < T) {
      float* outk = a.dk + base + (size_t)col * rs;
      float* outv = a.dv + base + (size_t)col * rs;
      const float sc = a.scale;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          f32x4 k4 = {dk[dt][4 * bb] * sc, dk[dt][4 * bb + 1] * sc, dk[dt][4 * bb + 2] * sc,
                      dk[dt][4 * bb + 3] * sc};
          f32x4 v4 = {dv[dt][4 * bb], dv[dt][4 * bb + 1], dv[dt][4 * bb + 2], dv[dt][4 * bb + 3]};
          *reinterpret_cast<f32x4*>(outk + 32 * dt + 8 * bb + 4 * h) = k4;
          *reinterpret_cast<f32x4*>(outv + 32 * dt + 8 * bb + 4 * h) = v4;
        }
    }
    if (wn < 0) break;
    w = wn;
  }
}

}  // namespace fa
