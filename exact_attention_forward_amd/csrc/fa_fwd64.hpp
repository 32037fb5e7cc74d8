// 16-bit (bfloat16 or IEEE half) forward kernel for hd 64.
//
// Same algorithm, tiles and schedule as fwd32_kernel<TIn, 64, ..., NW = 2,
// BC = 32, MS = 2> ("Flash Attention 2 -- forward pass notes", section "Loop
// (per (b, h, Q-tile))"): two waves per 128-row query tile, each owning two
// 32-row sub-tiles; S^T = K Q^T with Q in registers, the online softmax with
// a lazily raised reference max, O^T += V^T P^T with P from the S registers;
// O / l and L = m + ln l at the end.  The results are bitwise those of
// fwd32_kernel (up to a block whose row-sum increment lies within rounding of
// 2^slack, below); what differs is the instruction stream.
//
// At two waves per SIMD the forward is bound by vector-ALU issue, and each
// wave's own stream is a chain (scores -> max -> exp -> P V) that the other
// wave overlaps only by chance.  Three changes follow from that:
//  - K and V stream through a ring of four LDS slots filled by direct
//    global-to-LDS loads (global_load_lds_dwordx4) issued up to three blocks
//    ahead, from a wave-uniform base address plus a fixed per-lane offset:
//    no staging registers, no LDS writes and no per-lane address arithmetic
//    per block.  A block's rows are 128 contiguous bytes whose 16-byte
//    granules are XOR-swizzled by row, so the row reads of K and the
//    transposing reads of V are free of bank conflicts.
//  - Blocks visible to every row of the item run software-pipelined: the
//    scores of block j + 1 are issued in the same straight-line region as
//    the exponentials and P V products of block j, with two score buffers
//    alternating (no register copies between steps).
//  - With single-rounded P, a pipelined block takes no row max: the row-sum
//    increments show whether the reference would have been raised, and only
//    then is the block redone with the max.
//  - The diagonal and ragged blocks keep the per-block code of fwd32_kernel
//    with compile-time mask states.
#pragma once
#include <type_traits>

#include "fa_fwd32.hpp"
#include "fa_ring.hpp"

namespace fa {

template <typename TIn, bool CAUSAL, int PREC>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd64_kernel(FwdArgs a) {
  constexpr int HD = 64;
  constexpr int NW = 2, NT = NW * 64, MS = 2;
  constexpr int BR = NW * 32 * MS;  // query rows per work item
  constexpr int BC = 32;            // keys per block
  constexpr int NKS = HD / 16, NDT = HD / 32;
  constexpr int RB = 2 * HD;     // bytes per LDS row
  constexpr int BLK = BC * RB;   // bytes of one K (or V) block
  constexpr int NSLOT = 4;       // ring slots
  constexpr int LOOK = 3;        // blocks requested ahead of the one computed
  constexpr int CPB = 2 * BLK / (NT * 16);  // copies per thread per block (K and V)
  static_assert(NSLOT == LOOK + 1 && CPB == 4, "ring shape");
  using V8 = typename Frag32<TIn>::V;

  __shared__ __attribute__((aligned(1024))) unsigned char ring[NSLOT][2][BLK];

  const int T = a.T, H = a.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;
  const unsigned one2 = a.one2;
  const float c2 = a.c2;
  const size_t rs = (size_t)H * HD;
  const int nqt = (T + BR - 1) / BR;
  const int total = nqt * a.B * H;
  const bf16_t* Kg = static_cast<const bf16_t*>(a.k);
  const bf16_t* Vg = static_cast<const bf16_t*>(a.v);

  auto item_base = [&](int w) {
    const int bh = w / nqt;
    return ((size_t)(bh / H) * T * H + bh % H) * HD;
  };
  auto item_i0 = [&](int w) { return (nqt - 1 - w % nqt) * BR; };
  auto item_nkb = [&](int w) {
    return CAUSAL ? ((min(item_i0(w) + BR, T) - 1) / BC + 1) : (T + BC - 1) / BC;
  };

  // ---- the workgroup's stream of K/V blocks, copied LOOK blocks ahead ----
  // Copy c of a block (c = 0..3): tensor c / 2 (K, V), 1 KiB chunk
  // 2 wave + c % 2 of its 4 KiB = rows 8 chunk .. + 7; lane i copies row
  // 8 chunk + i / 8, LDS granule slot i % 8 (holding column granule
  // (i % 8) ^ swz128(row)).
  int crow[2], ccol[2];
  unsigned loff[2];  // byte offset of this lane's source in a block, rows not clamped
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    crow[c] = 8 * (2 * wave + c) + (lane >> 3);
    ccol[c] = 8 * ((lane & 7) ^ swz128(crow[c]));
    loff[c] = (unsigned)((crow[c] * rs + ccol[c]) * sizeof(bf16_t));
  }
  // LDS byte address of this wave's first chunk in slot 0, K
  const unsigned lds_w = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(lds_void_t*)(&ring[0][0][2 * wave * 1024]));
  int dw = persistent_item(0, total);  // item being copied
  if (dw < 0) return;
  int dkb = 0, dnkb = item_nkb(dw), dround = 0;
  size_t dbase = item_base(dw);
  int issued = 0;  // blocks requested so far (stream positions)
  auto issue = [&] {
    const unsigned dst = lds_w + (unsigned)((issued % NSLOT) * 2 * BLK);
    const size_t first = dbase + (size_t)dkb * BC * rs;
    if (dkb * BC + BC <= T) {
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const int t = c >> 1, k = c & 1;
        lds_copy16((t ? Vg : Kg) + first, loff[k], dst + t * BLK + k * 1024);
      }
    } else {
      // last, partial block: rows past T repeat row T - 1 (finite data that
      // the mask then gives zero weight)
#pragma unroll
      for (int c = 0; c < CPB; ++c) {
        const int t = c >> 1, k = c & 1;
        const int r = min(dkb * BC + crow[k], T - 1) - dkb * BC;
        lds_copy16((t ? Vg : Kg) + first, (unsigned)((r * rs + ccol[k]) * sizeof(bf16_t)), dst + t * BLK + k * 1024);
      }
    }
    ++issued;
    if (__builtin_expect(++dkb >= dnkb, 0)) {
      dw = persistent_item(++dround, total);
      dkb = 0;
      if (dw >= 0) {
        dnkb = item_nkb(dw);
        dbase = item_base(dw);
      }
    }
  };
  for (int i = 0; i < LOOK && dw >= 0; ++i) issue();

  // Operand reads from a ring slot.  K rows (A operand of S^T = K Q^T): lane
  // (n, h) reads key row n, hd elements 16 ks + 8h .. +7.
  auto ld_k = [&](int s, int ks) {
    const int g = 2 * ks + h;
    return *reinterpret_cast<const V8*>(&ring[s][0][n * RB + ((g ^ swz128(n)) << 4)]);
  };
  // V^T (A operand of O^T += V^T P^T) for product step st (keys 16 st ..)
  // and output tile dt: the transposing reads of ld_tr32 on swizzled rows.
  const int tu = lane & 15, tg = (lane >> 4) & 1;
  auto ld_vt = [&](int s, int st, int dt) {
    const int r = 16 * st + 4 * h + (tu >> 2), r2 = r + 8;
    const int c = 4 * dt + 2 * tg + ((tu & 3) >> 1);
    const int off = 8 * (tu & 1);
    const unsigned char* base = &ring[s][1][0];
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + r * RB + ((c ^ swz128(r)) << 4) + off));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + r2 * RB + ((c ^ swz128(r2)) << 4) + off));
    typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
    i16x8 rr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(V8, rr);
  };

  int pos = 0;  // stream position of the block computed next
  for (int round = 0;; ++round) {
    const int w = persistent_item(round, total);
    if (w < 0) break;
    const int bh = w / nqt;
    const size_t base = item_base(w);
    const bf16_t* Q = static_cast<const bf16_t*>(a.q) + base;
    const int i0 = item_i0(w);
    const int nkb = item_nkb(w);

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
      // element e of a tile starting at key jt is masked iff 8*(e/4) + e%4 > vis - jt
      vis[u] = (CAUSAL ? min(row, T - 1) : T - 1) - 4 * h;
      lastb[u] = r0[u] >= T ? -1 : (CAUSAL ? min(r0[u] + 31, T - 1) / BC : nkb - 1);
    }
    // Wait for the Q fragments here, once per item: a wait the compiler would
    // place for them inside the block loop would also drain the block copies
    // in flight (it cannot see them), every block.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Mask and reference-max update (with rescale) for one sub-tile's raw
    // scores s of the block at key j0.
    auto softmax_max = [&](int u, f32x16& s, int j0, auto masked) {
      if (decltype(masked)::value) {
        const int lim = vis[u] - j0;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (8 * (e >> 2) + (e & 3) > lim) s[e] = -INFINITY;
      }
      const float mb = half_swap_max(tile_max(s)) * c2;
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
    // P = exp2(s c2 - m) packed (pk; the residual in pl for split operands), row sums.
    auto softmax_exp = [&](int u, f32x16& s, V8* pk, V8* pl) {
      const float muse = mref[u] == -INFINITY ? 0.f : mref[u];
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = fast_exp2(fmaf(s[e], c2, -muse));
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        pk[st] = pack32<V8>(s, st);
        if (PREC == 0) sum8(pk[st], one2, ls0[u], ls1[u]);
        if (PREC == 1) pl[st] = pack32_lo<V8>(s, st);
      }
      if (PREC == 1) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ((e & 1) ? ls1[u] : ls0[u]) += s[e];
      }
    };
    // One K/V block in slot sl with compile-time sub-tile states: 0 = not
    // visited, 1 = every key visible, 2 = element-wise mask.
    auto block = [&](int sl, int j0, auto sa, auto sb) {
      constexpr int S0 = decltype(sa)::value, S1 = decltype(sb)::value;
      constexpr bool live[2] = {S0 != 0, S1 != 0};
      f32x16 s[MS];
#pragma unroll
      for (int u = 0; u < MS; ++u) s[u] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const V8 kop = ld_k(sl, ks);
#pragma unroll
        for (int u = 0; u < MS; ++u)
          if (live[u]) s[u] = mma32(kop, qf[u][ks], s[u]);
      }
      if (live[0]) softmax_max(0, s[0], j0, std::integral_constant<bool, S0 == 2>{});
      if (live[1]) softmax_max(1, s[1], j0, std::integral_constant<bool, S1 == 2>{});
      V8 vop[2][NDT];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vop[st][dt] = ld_vt(sl, st, dt);
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        if (!live[u]) continue;
        V8 pk[2], pl[2];
        softmax_exp(u, s[u], pk, pl);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            oacc[u][dt] = mma32(vop[st][dt], pk[st], oacc[u][dt]);
            if (PREC == 1) oacc[u][dt] = mma32(vop[st][dt], pl[st], oacc[u][dt]);
          }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    // Blocks [0, nfull) are visible to every row of the item.  They run
    // software-pipelined: the scores of block j + 1 are computed in the same
    // straight-line region as the exponentials and P V products of block j,
    // so the matrix pipe works while the wave does the vector work.
    auto scores = [&](int sl, f32x16* s) {
      V8 kop[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) kop[ks] = ld_k(sl, ks);
#pragma unroll
      for (int u = 0; u < MS; ++u) s[u] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int u = 0; u < MS; ++u) s[u] = mma32(kop[ks], qf[u][ks], s[u]);
    };
    // With single-rounded P (PREC 0) a pipelined block skips the row max:
    // its exponentials use the current reference, and the increments of the
    // row sums decide afterwards.  If every P of the block is below 2^slack
    // (each increment below it), the reference rule would not have raised the
    // reference, so the result is the one the max would have given; otherwise
    // (rare once a row's first block set the reference) the sums are restored
    // and the sub-tile is redone with the max, its scores recomputed from the
    // K block still in LDS.  The first pipelined block takes the max before
    // the loop.
    constexpr bool SKIP_MAX = PREC == 0;
    auto pipe_step = [&](f32x16* sc, f32x16* sn, auto has_next) {
      constexpr bool NX = decltype(has_next)::value;
      // block pos (V) and, with NX, block pos + 1 (K) complete and visible
      wait_vm(CPB * min(LOOK - 1, issued - 1 - (NX ? pos + 1 : pos)));
      __syncthreads();
      if (dw >= 0) issue();
      if (!SKIP_MAX) {
#pragma unroll
        for (int u = 0; u < MS; ++u) softmax_max(u, sc[u], 0, std::false_type{});
      }
      const int sl = pos % NSLOT;
      V8 vop[2][NDT];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vop[st][dt] = ld_vt(sl, st, dt);
      if constexpr (NX) scores((pos + 1) % NSLOT, sn);
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        V8 pk[2], pl[2];
        const float l0 = ls0[u], l1 = ls1[u];
        softmax_exp(u, sc[u], pk, pl);
        if (SKIP_MAX && __any((ls0[u] - l0) + (ls1[u] - l1) >= kSlackWeight)) {
          ls0[u] = l0;
          ls1[u] = l1;
          f32x16 s = zero16();
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) s = mma32(ld_k(sl, ks), qf[u][ks], s);
          softmax_max(u, s, 0, std::false_type{});
          softmax_exp(u, s, pk, pl);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            oacc[u][dt] = mma32(vop[st][dt], pk[st], oacc[u][dt]);
            if (PREC == 1) oacc[u][dt] = mma32(vop[st][dt], pl[st], oacc[u][dt]);
          }
      }
      // keep the scheduler from mixing consecutive steps (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    };
    const int nfull = min(CAUSAL ? i0 / BC : nkb, T / BC);
    if (nfull > 0) {
      wait_vm(CPB * min(LOOK - 1, issued - 1 - pos));
      __syncthreads();
      // two score buffers alternate, so no copies between steps
      f32x16 sa[MS], sb[MS];
      scores(pos % NSLOT, sa);
      if (SKIP_MAX) {
#pragma unroll
        for (int u = 0; u < MS; ++u) softmax_max(u, sa[u], 0, std::false_type{});
      }
      int kb = 0;
      for (; kb + 2 < nfull; kb += 2) {
        pipe_step(sa, sb, std::true_type{});
        ++pos;
        pipe_step(sb, sa, std::true_type{});
        ++pos;
      }
      if (kb + 2 == nfull) {
        pipe_step(sa, sb, std::true_type{});
        ++pos;
        pipe_step(sb, sa, std::false_type{});
      } else {
        pipe_step(sa, sb, std::false_type{});
      }
      ++pos;
    }

    for (int kb = nfull; kb < nkb; ++kb, ++pos) {
      // this thread's copies of block `pos` done (those of later blocks may
      // still run), then the barrier makes every thread's copies visible and
      // frees the slot of block pos - 1 for the copy issued next
      wait_vm(CPB * min(LOOK - 1, issued - 1 - pos));
      __syncthreads();
      if (dw >= 0) issue();
      const int j0 = kb * BC;
      const int sl = pos % NSLOT;
      int code = 0;
#pragma unroll
      for (int u = 0; u < MS; ++u) {
        const int st = kb > lastb[u] ? 0 : (((CAUSAL && j0 + BC - 1 > r0[u]) || j0 + BC > T) ? 2 : 1);
        code = 3 * code + st;
      }
      switch (code) {
        case 4: block(sl, j0, I1{}, I1{}); break;
        case 7: block(sl, j0, I2{}, I1{}); break;
        case 1: block(sl, j0, I0{}, I1{}); break;
        case 2: block(sl, j0, I0{}, I2{}); break;
        case 5: block(sl, j0, I1{}, I2{}); break;
        case 8: block(sl, j0, I2{}, I2{}); break;
        case 3: block(sl, j0, I1{}, I0{}); break;
        case 6: block(sl, j0, I2{}, I0{}); break;
        default: break;
      }
    }

#pragma unroll
    for (int u = 0; u < MS; ++u) {
      const int row = r0[u] + n;
      const float l = half_swap_sum(ls0[u] + ls1[u]);
      if (row < T) {
        float* O = a.o + base + (size_t)row * rs;
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            f32x4 v4 = {oacc[u][dt][4 * bb] * inv, oacc[u][dt][4 * bb + 1] * inv, oacc[u][dt][4 * bb + 2] * inv,
                        oacc[u][dt][4 * bb + 3] * inv};
            *reinterpret_cast<f32x4*>(O + 32 * dt + 8 * bb + 4 * h) = v4;
          }
        if (h == 0) a.lse[(size_t)bh * T + row] = l > 0.f ? (mref[u] + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

}  // namespace fa
