// Forward kernel: exact attention with an online softmax, one workgroup per
// (query tile, batch*head).
//
// Follows the loop of "Flash Attention 2 -- forward pass notes", section
// "Loop (per (b, h, Q-tile))": the query tile stays on chip, key/value blocks
// stream through LDS, each row keeps a running max m, running sum l and
// running output, rescaled by alpha = exp(m_old - m_new) when the max grows;
// key blocks wholly above the causal diagonal are skipped; the epilogue
// divides by l and stores O and the log-sum-exp L = m + ln l (the quantity
// the backward notes, section "The math (FA2 backward with recompute)", need).
//
// gfx950 mapping:
//  * NW waves per workgroup; each wave owns 16*MR query rows whose Q
//    fragments live in registers for the whole kernel.
//  * Scores are computed transposed, S^T = K Q^T, so each lane owns one query
//    row (li) of every 16x16 tile: the row max and row sum need only the two
//    butterfly steps across lane groups, and alpha is a per-lane scalar.
//  * The output is accumulated transposed, O^T += V^T P^T, with P^T taken from
//    the S^T registers directly and V^T read from the row-major V tile (LDS
//    transpose reads for bfloat16).
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA.
//  * K/V blocks are double-buffered: the next block's global loads are issued
//    before the current block's math.
#pragma once
#include "fa_common.hpp"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, H, T;
  float c2;                    // scale * log2(e)
  unsigned one2 = 0x3F803F80u;  // bfloat16 pair (1, 1): a scalar operand for row sums by dot products
  // Key split: split s handles keys [s kchunk, (s + 1) kchunk) and writes its
  // partial O and L at o + s o_split, lse + s lse_split (fwd_kernel: split =
  // blockIdx.y; fwd32_kernel: nsplit splits per query tile among its work
  // items).  kchunk = 0: one split covering every key.
  int kchunk = 0;
  size_t o_split = 0, lse_split = 0;
  int nsplit = 1;
};

// PREC: 0 = operands rounded to bfloat16 (or exact f32), 1 = P split into a
// bfloat16 high part and a bfloat16 residual (two products).
// CONTROL (deliberately wrong variants that exist only so that checks can be
// shown to reject them):
//   kCtlNoRescale  the "broken" kernel of the fused-attention lesson (blocks
//                  "controls" and "correctness"): when a row's running max
//                  rises, l and the accumulated output are NOT multiplied by
//                  alpha; wrong whenever a later key block raises a row's max;
//   kCtlNoMax      the unsafe softmax: no max is subtracted, p = exp(s); with
//                  half-precision P operands any score >= ln 65520 overflows
//                  (lesson, block "overflow").
enum Control { kCtlNone = 0, kCtlNoRescale = 1, kCtlNoMax = 2 };
// Up to hd 64 the compiler is held to three resident waves per SIMD (at most
// 168 VGPRs, no spills): 11% faster than two at float32, B64 H16 T1024 hd64.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int MR, int BC, int CONTROL = kCtlNone>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(HD <= 64 ? 3 : 1))) void fwd_kernel(
    FwdArgs a) {
  using M = Mma<TIn>;
  using frag = typename M::frag;
  constexpr int NT = NW * 64;
  constexpr int RW = 16 * MR;
  constexpr int BR = NW * RW;
  constexpr int LD = lds_ld<TIn, HD>();
  constexpr int NDT = (HD + 15) / 16;
  constexpr int NKS = HD / M::KS;
  constexpr int NJT = BC / 16;
  constexpr int NCH = BC / M::CH;
  constexpr int TPC = M::CH / 16;  // C tiles per register chunk
  static_assert(HD % M::KS == 0, "head dim must be a multiple of the MFMA contraction");
  static_assert(BC % M::CH == 0, "key block must be a multiple of the register chunk");
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
  const int qt = nqt - 1 - (w % nqt);  // longest causal tiles first
  const int b = bh / H, h = bh % H;
  const size_t rs = (size_t)H * HD;
  const size_t base = ((size_t)b * T * H + h) * HD;
  const TIn* Q = static_cast<const TIn*>(a.q) + base;
  const TIn* K = static_cast<const TIn*>(a.k) + base;
  const TIn* V = static_cast<const TIn*>(a.v) + base;

  const int i0 = qt * BR;
  const int r0 = i0 + wave * RW;
  const float c2 = a.c2;

  if (sizeof(TIn) == 4 && HD < 16) {
    // Columns HD..15 of the f32 tiles are read as rows of unused output
    // tiles; keep them finite.
    for (int x = tid; x < 2 * BC * LD; x += NT) {
      (&sK[0][0])[x] = TIn{};
      (&sV[0][0])[x] = TIn{};
    }
    __syncthreads();
  }

  frag qf[MR][NKS];
#pragma unroll
  for (int mr = 0; mr < MR; ++mr)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[mr][ks] = M::ld_row_global(Q, rs, r0 + 16 * mr + li, T, ks * M::KS, lg);

  f32x4 oacc[NDT][MR];
  float mrow[MR], lrow[MR];
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    mrow[mr] = -INFINITY;
    lrow[mr] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt][mr] = zero4();
  }

  const int last_row = min(i0 + BR, T) - 1;
  // key blocks [kb0, nkb) of this split (all blocks when a.kchunk == 0)
  const int nkb_all = CAUSAL ? (last_row / BC + 1) : (T + BC - 1) / BC;
  const int kb0 = a.kchunk ? (int)blockIdx.y * (a.kchunk / BC) : 0;
  const int nkb = a.kchunk ? min(nkb_all, kb0 + a.kchunk / BC) : nkb_all;

  TileCopy<TIn, HD, BC, NT> ck, cv;
  ck.load(K, rs, kb0 * BC, T, tid);
  cv.load(V, rs, kb0 * BC, T, tid);
  ck.store(sK[0], LD, tid);
  cv.store(sV[0], LD, tid);
  __syncthreads();

  for (int kb = kb0; kb < nkb; ++kb) {
    const int j0 = kb * BC;
    const int buf = (kb - kb0) & 1;
    if (kb + 1 < nkb) {
      ck.load(K, rs, j0 + BC, T, tid);
      cv.load(V, rs, j0 + BC, T, tid);
    }
    const TIn* cK = sK[buf];
    const TIn* cV = sV[buf];
    const bool active = !CAUSAL || (j0 <= r0 + RW - 1);
    if (active) {
      f32x4 s[MR][NJT];
#pragma unroll
      for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) s[mr][jt] = zero4();
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const frag af = M::ld_row(cK, LD, 16 * jt, ks * M::KS, li, lg);
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) s[mr][jt] = M::mma(af, qf[mr][ks], s[mr][jt]);
        }

      const bool need_mask = (CAUSAL && (j0 + BC - 1 > r0)) || (j0 + BC > T);
      if (need_mask) {
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          const int i = r0 + 16 * mr + li;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = j0 + 16 * jt + 4 * lg + r;
              if ((CAUSAL && j > i) || j >= T) s[mr][jt][r] = -INFINITY;
            }
        }
      }

#pragma unroll
      for (int mr = 0; mr < MR; ++mr) {
        float mx = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[mr][jt][r]);
        mx = group_max(mx);
        const float mold = mrow[mr];
        const float mnew = CONTROL == kCtlNoMax ? 0.f : fmaxf(mold, mx * c2);
        const float alpha = CONTROL != kCtlNone ? 1.f : ((mold == -INFINITY) ? 0.f : fast_exp2(mold - mnew));
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        mrow[mr] = mnew;
        float ls = 0.f;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(s[mr][jt][r], c2, -muse));
            s[mr][jt][r] = p;
            ls += p;
          }
        lrow[mr] = lrow[mr] * alpha + ls;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt][mr] *= alpha;
      }

#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int st = 0; st < M::NSTEP; ++st) {
          frag bf[MR], bl[MR];
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            bf[mr] = M::pack(&s[mr][ch * TPC], st);
            if (PREC == 1) bl[mr] = M::pack_lo(&s[mr][ch * TPC], st);
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const frag af = M::ld_trans(cV, LD, ch * M::CH, 16 * dt, st, li, lg);
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              oacc[dt][mr] = M::mma(af, bf[mr], oacc[dt][mr]);
              if (PREC == 1) oacc[dt][mr] = M::mma(af, bl[mr], oacc[dt][mr]);
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

  float* O = a.o + blockIdx.y * a.o_split + base;
  float* Lout = a.lse + blockIdx.y * a.lse_split;
#pragma unroll
  for (int mr = 0; mr < MR; ++mr) {
    const float l = group_sum(lrow[mr]);
    const int i = r0 + 16 * mr + li;
    if (i < T) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + 4 * lg;
        if (d < HD) *reinterpret_cast<f32x4*>(O + (size_t)i * rs + d) = oacc[dt][mr] * inv;
      }
      if (lg == 0) Lout[(size_t)bh * T + i] = l > 0.f ? (mrow[mr] + log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace fa
