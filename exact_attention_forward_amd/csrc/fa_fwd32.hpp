// bfloat16 forward kernel on 32x32 MFMA tiles.
//
// Same algorithm as fwd_kernel ("Flash Attention 2 -- forward pass notes",
// section "Loop (per (b, h, Q-tile))"): online softmax over streamed K/V
// blocks, causal block skip, O and L = m + ln l written once.  Each wave owns
// 32 query rows; lane (n, h) owns row n of the wave together with lane
// (n, 1-h), so the row max and row sum need one exchange across lane halves.
//  * S^T = K Q^T per 32-key tile: K from the LDS block, Q^T from registers.
//  * O^T += V^T P^T: P^T straight from the S^T registers (see fa_mfma32.hpp),
//    V^T by LDS transpose reads of the row-major V block.
//  * Every block runs straight-line code, so the independent MFMA chains of
//    the block interleave; blocks crossing the causal diagonal or the end of
//    the sequence add an element-wise mask before the row max.
//  * The rescale of O by alpha is skipped when no row of the wave raised its
//    running max in the block.
#pragma once
#include <type_traits>

#include "fa_fwd.hpp"
#include "fa_mfma32.hpp"

namespace fa {

template <int HD, bool CAUSAL, int PREC, int NW, int BC>
__global__ __launch_bounds__(NW * 64, HD <= 64 ? 2 : 1) void fwd32_kernel(FwdArgs a) {
  // Persistent: the grid is sized to the resident workgroups and each loops over work items.
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int LD = HD + 8;
  constexpr int NDT = HD / 32;  // 32-wide output tiles
  constexpr int NKS = HD / 16;  // product steps over the head dim
  constexpr int NKT = BC / 32;  // 32-key tiles per block
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
  const int i0 = qt * BR;
  const int r0 = i0 + wave * 32;
  const int row = r0 + n;
  const float c2 = a.c2;
  // Largest visible key of this lane's row, minus the lane-half offset of the
  // C layout: element e of a tile starting at key jt is masked iff
  // 8*(e/4) + e%4 > vis - jt.
  const int vis = (CAUSAL ? min(row, T - 1) : T - 1) - 4 * h;

  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_row_global32(Q, rs, row, T, 16 * ks, h);

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = zero16();
  float mrow = -INFINITY, lrow = 0.f;

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
    f32x16 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = mma32(ld_row32(cK, LD, 32 * kt, 16 * ks, n, h), qf[ks], s[kt]);
    if (MASK) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const int lim = vis - (j0 + 32 * kt);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (8 * (e >> 2) + (e & 3) > lim) s[kt][e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrow, mx * c2);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const bool grew = mnew > mrow;
    const float alpha = (mrow == -INFINITY) ? 0.f : fast_exp2(mrow - mnew);
    mrow = mnew;
    // P = exp2(s c2 - m); the row sum adds the unrounded float weights.
    bf16x8 pk[NKT][2];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[kt][e] = fast_exp2(fmaf(s[kt][e], c2, -muse));
        ls += s[kt][e];
      }
      if (PREC == 0) {
#pragma unroll
        for (int st = 0; st < 2; ++st) pk[kt][st] = pack32(s[kt], st);
      }
    }
    lrow = lrow * alpha + ls;
    if (__any(grew)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 bf = PREC == 0 ? pk[kt][st] : pack32(s[kt], st);
        bf16x8 bl;
        if (PREC == 1) bl = pack32_lo(s[kt], st);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 af = ld_tr32(cV, LD, 32 * kt + 16 * st, 32 * dt, lane);
          oacc[dt] = mma32(af, bf, oacc[dt]);
          if (PREC == 1) oacc[dt] = mma32(af, bl, oacc[dt]);
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

  const float l = lrow + __shfl_xor(lrow, 32);
  if (row < T) {
    float* O = a.o + base + (size_t)row * rs;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        f32x4 v4 = {oacc[dt][4 * bb] * inv, oacc[dt][4 * bb + 1] * inv, oacc[dt][4 * bb + 2] * inv,
                    oacc[dt][4 * bb + 3] * inv};
        *reinterpret_cast<f32x4*>(O + 32 * dt + 8 * bb + 4 * h) = v4;
      }
    if (h == 0) a.lse[(size_t)bh * T + row] = l > 0.f ? (mrow + log2f(l)) * kLn2 : -INFINITY;
  }
  }
}

}  // namespace fa
