// 16-bit (bfloat16 or IEEE half) forward kernel on 32x32 MFMA tiles.
//
// Same algorithm as fwd_kernel ("Flash Attention 2 -- forward pass notes",
// section "Loop (per (b, h, Q-tile))"): online softmax over streamed K/V
// blocks, causal block skip, O and L = m + ln l written once.
//  * Each wave owns MS sub-tiles of 32 query rows.  Lane (n, h) owns row n of
//    every sub-tile together with lane (n, 1-h), so the row max and row sum
//    need one exchange across lane halves (v_permlane32_swap).
//  * S^T = K Q^T per 32-key tile: K from the LDS block, Q^T from registers.
//    O^T += V^T P^T: P^T straight from the S^T registers (see fa_mfma32.hpp),
//    V^T by LDS transpose reads of the row-major V block.  Every K or V
//    operand read from LDS feeds the products of all MS sub-tiles, and the
//    vector-ALU softmax of one sub-tile overlaps the matrix products of the
//    other.
//  * The running max is a reference value for the exponentials, not
//    necessarily the exact row max: it is raised (and O, l rescaled) only when
//    a block's max exceeds it by more than 2^8 in the exponential's units.
//    The normalised result is the same for any reference (O = sum p v / sum p
//    with the same p in both), and weights up to 2^8 stay far from overflow
//    (in half precision too, whose largest finite value is 65504).
//  * Row sums add the 16-bit weights that enter the P V product (dot
//    products with (1, 1)), so O is normalised by exactly the weights used.
//  * Blocks crossing the causal diagonal or the end of the sequence apply an
//    element-wise -inf mask to the raw scores before the row max; sub-tiles
//    wholly above the diagonal skip the block.
#pragma once
#include <type_traits>

#include "fa_fwd.hpp"
#include "fa_mfma32.hpp"

namespace fa {

// Max over lanes l and l ^ 32 (the two halves of one row).
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Adds the eight 16-bit values of an operand fragment to two partial sums
// (one2 holds the pair (1, 1) in the fragment's format).
// The pairs are taken with shufflevector: reinterpreting the fragment as four
// 32-bit words before the dot products was mis-lowered by the compiler (the
// same register fed every product).
__device__ __forceinline__ void sum8(bf16x8 v, unsigned one2, float& acc0, float& acc1) {
  const bf16x2 o = __builtin_bit_cast(bf16x2, one2);
  acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), o, acc0, false);
  acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), o, acc1, false);
  acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), o, acc0, false);
  acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), o, acc1, false);
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void sum8(f16x8 v, unsigned one2, float& acc0, float& acc1) {
  const f16x2 o = __builtin_bit_cast(f16x2, one2);
  acc0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), o, acc0, false);
  acc1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), o, acc1, false);
  acc0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), o, acc0, false);
  acc1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), o, acc1, false);
}

// Exponent headroom (base 2) before the reference max is raised.
constexpr float kRescaleSlack = 8.f;
constexpr float kSlackWeight = 256.f;  // 2^kRescaleSlack: the largest P the reference rule allows

// Max of the 16 elements of a C tile, as a shallow tree.
__device__ __forceinline__ float tile_max(const f32x16& x) {
  float m[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) m[g] = fmaxf(fmaxf(x[4 * g], x[4 * g + 1]), fmaxf(x[4 * g + 2], x[4 * g + 3]));
  return fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
}

// Sub-tile u of wave w covers rows 32 w (u = 0) and 32 (2 NW - 1 - w) (u = 1)
// of the workgroup's tile, so under the causal mask every wave has the same
// number of (row, key) pairs to visit.
template <int NW, int MS>
__device__ __forceinline__ int subtile_row(int wave, int u) {
  return MS == 1 ? 32 * wave : (u == 0 ? 32 * wave : 32 * (2 * NW - 1 - wave));
}

#ifndef FA_FWD_WPE64
#define FA_FWD_WPE64 2
#endif
#ifndef FA_FWD_WPE128
#define FA_FWD_WPE128 2
#endif
// SPLIT: the work items are (query tile, head, key split) and each writes a
// partial O and L for the merge; false compiles the plain kernel with the
// split bookkeeping folded away.
template <typename TIn, int HD, bool CAUSAL, int PREC, int NW, int BC, int MS, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(HD <= 64 ? FA_FWD_WPE64 : FA_FWD_WPE128, HD <= 64 ? FA_FWD_WPE64 : FA_FWD_WPE128)))
void fwd32_kernel(FwdArgs a) {
  // Persistent: the grid is sized to the resident workgroups and each loops over work items.
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32 * MS;
  constexpr int LD = HD <= 64 ? HD + 8 : HD + 24;  // LDS row pitch (elements); see lds_ld
  constexpr int NDT = HD / 32;  // 32-wide output tiles
  constexpr int NKS = HD / 16;  // product steps over the head dim
  constexpr int NKT = BC / 32;  // 32-key tiles per block
  static_assert(HD % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(2 * 2 * BC * LD * 2 <= 160 * 1024, "LDS budget");
  static_assert(MS == 1 || MS == 2, "one or two sub-tiles per wave");
  using Copy = TileStream<HD, BC, NT>;
  using V8 = typename Frag32<TIn>::V;

  __shared__ __attribute__((aligned(16))) bf16_t sK[2][BC * LD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][BC * LD];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const unsigned one2 = a.one2;
  const float c2 = a.c2;
  const size_t rs = (size_t)H * HD;
  unsigned goff[Copy::PER];  // byte offsets of this thread's copy vectors within a block
#pragma unroll
  for (int p = 0; p < Copy::PER; ++p) goff[p] = (unsigned)((Copy::vrow(tid, p) * rs + Copy::vcol(tid, p)) * 2);

  const int nqt = (T + BR - 1) / BR;
  const int nsp = SPLIT ? a.nsplit : 1;  // key splits per query tile
  const int total = nqt * a.B * H * nsp;
  for (int round = 0;; ++round) {
    const int w = persistent_item(round, total);
    if (w < 0) break;
    const int sp = SPLIT ? w % nsp : 0;
    const int wq = SPLIT ? w / nsp : w;
    const int bh = wq / nqt;
    const int qt = nqt - 1 - (wq % nqt);
    const int b = bh / H, hh = bh % H;
    const size_t base = ((size_t)b * T * H + hh) * HD;
    const bf16_t* Q = static_cast<const bf16_t*>(a.q) + base;
    const bf16_t* K = static_cast<const bf16_t*>(a.k) + base;
    const bf16_t* V = static_cast<const bf16_t*>(a.v) + base;
    const int i0 = qt * BR;
    const int nkb = CAUSAL ? ((min(i0 + BR, T) - 1) / BC + 1) : (T + BC - 1) / BC;
    // this split's key blocks (none when its range starts past the visible keys:
    // then O = 0 and L = -inf, which the merge skips)
    const int kb_lo = SPLIT ? sp * (a.kchunk / BC) : 0;
    const int kb_end = SPLIT ? min(nkb, kb_lo + a.kchunk / BC) : nkb;
    float* const Og = SPLIT ? a.o + (size_t)sp * a.o_split : a.o;
    float* const Lg = SPLIT ? a.lse + (size_t)sp * a.lse_split : a.lse;

    V8 qf[MS][NKS];
    f32x16 oacc[MS][NDT];
    float mref[MS], ls0[MS], ls1[MS];
    int r0[MS], vis[MS], lastb[MS];
#pragma unroll
    for (int u = 0; u < MS; ++u) {
      r0[u] = i0 + subtile_row<NW, MS>(wave, u);
      const int row = r0[u] + n;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[u][ks] = ld_row_global32<V8>(Q, rs, row, T, 16 * ks, h);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[u][dt] = zero16();
      mref[u] = -INFINITY;
      ls0[u] = ls1[u] = 0.f;
      // Largest visible key of this lane's row, minus the lane-half offset of
      // the C layout: element e of a tile starting at key jt is masked iff
      // 8*(e/4) + e%4 > vis - jt.
      vis[u] = (CAUSAL ? min(row, T - 1) : T - 1) - 4 * h;
      lastb[u] = r0[u] >= T ? -1 : (CAUSAL ? min(r0[u] + 31, T - 1) / BC : nkb - 1);
    }

    Copy ck, cv;
    auto fetch = [&](int j) {  // block of keys starting at j into the copy registers
      if (j + BC <= T) {
        ck.load(K + (size_t)j * rs, goff);
        cv.load(V + (size_t)j * rs, goff);
      } else {
        ck.load_clamped(K, rs, j, T, tid);
        cv.load_clamped(V, rs, j, T, tid);
      }
    };
    if (!SPLIT || kb_lo < kb_end) {  // uniform over the workgroup
      fetch(kb_lo * BC);
      ck.store(sK[0], LD, tid);
      cv.store(sV[0], LD, tid);
      __syncthreads();
    }

    // Mask and reference-max update (with rescale) for one sub-tile's raw
    // scores s of the block at key j0.
    auto softmax_max = [&](int u, f32x16* s, int j0, auto masked) {
      if (decltype(masked)::value) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int lim = vis[u] - (j0 + 32 * kt);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (8 * (e >> 2) + (e & 3) > lim) s[kt][e] = -INFINITY;
        }
      }
      float mx = tile_max(s[0]);
#pragma unroll
      for (int kt = 1; kt < NKT; ++kt) mx = fmaxf(mx, tile_max(s[kt]));
      const float mb = half_swap_max(mx) * c2;
      const bool raise = mb > mref[u] + kRescaleSlack;
      if (__any(raise)) {
        const float mnew = raise ? mb : mref[u];
        const float alpha = mref[u] == -INFINITY ? 0.f : fast_exp2(mref[u] - mnew);
        mref[u] = mnew;
        ls0[u] *= alpha;
        ls1[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[u][dt] *= alpha;
      }
    };
    // P = exp2(s c2 - m) packed to bfloat16 (pk; the residual in pl for the
    // split precision), row sums updated.
    auto softmax_exp = [&](int u, f32x16* s, V8 (*pk)[2], V8 (*pl)[2]) {
      const float muse = mref[u] == -INFINITY ? 0.f : mref[u];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kt][e] = fast_exp2(fmaf(s[kt][e], c2, -muse));
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          pk[kt][st] = pack32<V8>(s[kt], st);
          if (PREC == 0) sum8(pk[kt][st], one2, ls0[u], ls1[u]);
          if (PREC == 1) pl[kt][st] = pack32_lo<V8>(s[kt], st);
        }
        if (PREC == 1) {
#pragma unroll
          for (int e = 0; e < 16; ++e) ((e & 1) ? ls1[u] : ls0[u]) += s[kt][e];
        }
      }
    };

    // One K/V block with compile-time sub-tile states: 0 = not visited,
    // 1 = every key visible, 2 = element-wise mask (causal diagonal or the end
    // of the sequence).
    auto block = [&](const bf16_t* cK, const bf16_t* cV, int j0, auto sa, auto sb) {
      constexpr int S0 = decltype(sa)::value, S1 = decltype(sb)::value;
      constexpr bool live[2] = {S0 != 0, MS > 1 && S1 != 0};
      f32x16 s[MS][NKT];
#pragma unroll
      for (int u = 0; u < MS; ++u)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) s[u][kt] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const V8 kop = ld_row32<V8>(cK, LD, 32 * kt, 16 * ks, n, h);
#pragma unroll
          for (int u = 0; u < MS; ++u)
            if (live[u]) s[u][kt] = mma32(kop, qf[u][ks], s[u][kt]);
        }
      if (live[0]) softmax_max(0, s[0], j0, std::integral_constant<bool, S0 == 2>{});
      if constexpr (MS > 1)
        if (live[1]) softmax_max(1, s[1], j0, std::integral_constant<bool, S1 == 2>{});
      V8 vop[NKT][2][NDT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vop[kt][st][dt] = ld_tr32<V8>(cV, LD, 32 * kt + 16 * st, 32 * dt, lane);
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        if (!live[u]) continue;
        V8 pk[NKT][2], pl[NKT][2];
        softmax_exp(u, s[u], pk, pl);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              oacc[u][dt] = mma32(vop[kt][st][dt], pk[kt][st], oacc[u][dt]);
              if (PREC == 1) oacc[u][dt] = mma32(vop[kt][st][dt], pl[kt][st], oacc[u][dt]);
            }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    for (int kb = kb_lo; kb < kb_end; ++kb) {
      const int j0 = kb * BC;
      const int buf = (kb - kb_lo) & 1;
      if (kb + 1 < kb_end) fetch(j0 + BC);
      int code = 0;
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        const int st = kb > lastb[u] ? 0 : (((CAUSAL && j0 + BC - 1 > r0[u]) || j0 + BC > T) ? 2 : 1);
        code = 3 * code + st;
      }
      const bf16_t* cK = sK[buf];
      const bf16_t* cV = sV[buf];
      if constexpr (MS == 2) {
        switch (code) {
          case 4: block(cK, cV, j0, I1{}, I1{}); break;
          case 7: block(cK, cV, j0, I2{}, I1{}); break;
          case 1: block(cK, cV, j0, I0{}, I1{}); break;
          case 2: block(cK, cV, j0, I0{}, I2{}); break;
          case 5: block(cK, cV, j0, I1{}, I2{}); break;
          case 8: block(cK, cV, j0, I2{}, I2{}); break;
          case 3: block(cK, cV, j0, I1{}, I0{}); break;
          case 6: block(cK, cV, j0, I2{}, I0{}); break;
          default: break;
        }
      } else {
        if (code == 1) block(cK, cV, j0, I1{}, I0{});
        else if (code == 2) block(cK, cV, j0, I2{}, I0{});
      }
      if (kb + 1 < kb_end) {
        ck.store(sK[buf ^ 1], LD, tid);
        cv.store(sV[buf ^ 1], LD, tid);
      }
      __syncthreads();
    }

#pragma unroll
    for (int u = 0; u < MS; ++u) {
      const int row = r0[u] + n;
      const float l = half_swap_sum(ls0[u] + ls1[u]);
      if (row < T) {
        float* O = Og + base + (size_t)row * rs;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            f32x4 v4 = {oacc[u][dt][4 * bb] * inv, oacc[u][dt][4 * bb + 1] * inv, oacc[u][dt][4 * bb + 2] * inv,
                        oacc[u][dt][4 * bb + 3] * inv};
            *reinterpret_cast<f32x4*>(O + 32 * dt + 8 * bb + 4 * h) = v4;
          }
        if (h == 0) Lg[(size_t)bh * T + row] = l > 0.f ? (mref[u] + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

}  // namespace fa
