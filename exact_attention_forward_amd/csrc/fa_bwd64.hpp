// 16-bit (bfloat16 or IEEE half) dK/dV kernel for hd 64 ("Flash Attention 2
// -- backward pass notes", section "The math (FA2 backward with recompute)"
// and option 3 of "Why the WGSL kernel isn't shipped this turn": one owner per
// key tile, no atomics).  Four waves own 32 keys each of a 128-key tile, with
// K and V fragments in registers; query blocks of 64 rows stream past; per
// 32-row tile S^T and dP^T (stage A), P = exp2(S c - L log2 e) and
// dS = P (dP - D) (stage B), dV += P^T dO and dK += dS^T Q (stage C); dK is
// scaled once at the end.  Tiles wholly above a wave's first key are skipped
// and the diagonal ones masked element-wise.
//
// Data movement: each workgroup walks one stream of
// equally sized LDS "positions": per work item its K tile, its V tile, then
// its query blocks (Q and dO rows with their L and D).  Positions are filled
// by direct global-to-LDS copies from a wave-uniform base plus fixed per-lane
// offsets into a ring of four slots with XOR-swizzled 128-byte rows, up to
// three positions ahead and across work items, so that
//  - no global load is tracked by the compiler: it never drains the copies
//    in flight, and a new key tile's K and V reach the registers through LDS;
//  - no registers stage the blocks and no per-lane address arithmetic runs
//    per block;
//  - the row reads (stage A, K and V fragments) and the transposing reads
//    (stage C) of the swizzled rows are free of bank conflicts.
// L arrives raw; one wave scales it by log2 e in LDS, once per block, and
// gives rows past T (which read row T - 1) an L of +inf, so P = 0 there.
#pragma once
#include <type_traits>

#include "fa_bwd32.hpp"
#include "fa_ring.hpp"

namespace fa {

template <typename TIn, bool CAUSAL, int PREC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkv64_kernel(BwdArgs a) {
  constexpr int HD = 64, NW = 4, NT = NW * 64;
  constexpr int BK = NW * 32;       // keys per work item
  constexpr int BQ = 64;            // query rows per block
  constexpr int NIT = BQ / 32;      // 32-row tiles per block
  constexpr int NDT = HD / 32, NKS = HD / 16;
  constexpr int RB = 2 * HD;        // bytes per row
  constexpr int TILE = BQ * RB;     // Q (or dO) rows of one block
  constexpr int LOFF = 2 * TILE;    // L then D of a block, after Q and dO
  constexpr int POS = LOFF + 2 * BQ * 4;
  constexpr int NSLOT = 4;
  constexpr int OPS = 5;            // copies per wave per position
  static_assert(BK * RB == 2 * TILE, "a K or V tile fills one position");
  static_assert(2 * TILE / (NT * 16) == OPS - 1, "four 16-byte copies per thread and position");
  static_assert(2 * OPS <= 15, "steady-state wait count fits the low counter bits");
  using V8 = typename Frag32<TIn>::V;

  __shared__ __attribute__((aligned(1024))) unsigned char ring[NSLOT][POS];

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

  // ---- the copy stream ----
  // Copy c of wave w fills 1 KiB chunk 4 w + c of a position's first 16 KiB
  // (rows 8 chunk .. 8 chunk + 7 of a 128-row tile: the K or V tile, or Q rows
  // 0..63 then dO rows 0..63); lane i copies row 8 chunk + i / 8 into granule
  // slot i % 8, which holds column granule (i % 8) ^ swz128(row).  The fifth
  // copy brings L (even waves) or D (odd waves) of the block's 64 rows.
  auto crow = [&](int c) __attribute__((always_inline)) { return 8 * (4 * wave + c) + (lane >> 3); };
  unsigned loff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    loff[c] = (unsigned)((crow(c) * rs + 8 * ((lane & 7) ^ swz128(crow(c)))) * sizeof(bf16_t));
  const unsigned lds_w = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(lds_void_t*)(&ring[0][4 * wave * 1024]));
  const unsigned lds_ld = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(lds_void_t*)(&ring[0][LOFF + (wave & 1) * BQ * 4]));
  const bool q_wave = wave < 2;  // waves 0, 1 copy Q rows of a block; 2, 3 dO rows
  // this wave's block source: Q, or dO addressed from 64 rows back (the dO
  // chunks hold rows 64.. of the position); and L or D
  const bf16_t* QGw = uniform_ptr(
      q_wave ? Qg : (const bf16_t*)((uintptr_t)Gg - (uintptr_t)BQ * rs * sizeof(bf16_t)));
  const float* LDg = uniform_ptr((wave & 1) ? a.delta : a.lse);

  // Cursor: the item being copied and scalar source pointers for its next
  // position, set up once per item so that a position costs a few scalar adds.
  int dw = -1, dround = -1;  // item being copied, its round
  int dp = 0, dnp = 0;       // position within the item (0 K, 1 V, 2.. blocks), count
  int dq0 = 0;               // first row of the next block
  int dj0 = 0;               // first key of the item
  const bf16_t *pk = Kg, *pv = Vg, *pq = Qg;  // K tile, V tile, next block (this wave's Q or dO rows)
  const float* pl = LDg;                       // next block's L or D
  auto next_item = [&]() __attribute__((always_inline)) {
    dw = persistent_item(++dround, total);
    dp = 0;
    if (dw >= 0) {
      const int bh = dw / nkt, kt = dw - bh * nkt;
      const size_t bs = ((size_t)(bh / H) * T * H + bh % H) * HD;
      const int qb0 = CAUSAL ? kt * BK / BQ : 0;
      dnp = 2 + nqb - qb0;
      dq0 = qb0 * BQ;
      dj0 = kt * BK;
      pk = uniform_ptr(Kg + bs + (size_t)kt * BK * rs);
      pv = uniform_ptr(Vg + bs + (size_t)kt * BK * rs);
      pq = uniform_ptr((const bf16_t*)((uintptr_t)QGw + (bs + (size_t)dq0 * rs) * sizeof(bf16_t)));
      pl = uniform_ptr(LDg + (size_t)bh * T + dq0);
    }
  };
  next_item();
  if (dw < 0) return;
  int issued = 0;        // positions requested so far
  unsigned dslot = 0;    // LDS byte offset of the slot of position `issued`
  auto issue = [&]() __attribute__((always_inline)) {
    const unsigned dst = lds_w + dslot, dstl = lds_ld + dslot;
    if (dp < 2) {
      const bf16_t* src = dp ? pv : pk;
      const int j0 = dj0;
      if (__builtin_expect(j0 + BK <= T, 1)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) lds_copy16(src, loff[c], dst + c * 1024);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r = min(j0 + crow(c), T - 1) - j0;
          lds_copy16(src, (unsigned)((r * rs + 8 * ((lane & 7) ^ swz128(crow(c)))) * sizeof(bf16_t)), dst + c * 1024);
        }
      }
      lds_copy4(pl, 0u, dstl);  // keeps five copies per position; the area is unused
    } else {
      if (__builtin_expect(dq0 + BQ <= T, 1)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) lds_copy16(pq, loff[c], dst + c * 1024);
        lds_copy4(pl, (unsigned)(lane * 4), dstl);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int rl = crow(c) - (q_wave ? 0 : BQ);  // row within the block
          const int r = min(dq0 + rl, T - 1) - dq0 + (q_wave ? 0 : BQ);
          lds_copy16(pq, (unsigned)((r * rs + 8 * ((lane & 7) ^ swz128(crow(c)))) * sizeof(bf16_t)), dst + c * 1024);
        }
        lds_copy4(pl, (unsigned)((min(dq0 + lane, T - 1) - dq0) * 4), dstl);
      }
      pq = (const bf16_t*)((uintptr_t)pq + (uintptr_t)BQ * rs * sizeof(bf16_t));
      pl += BQ;
      dq0 += BQ;
    }
    ++issued;
    dslot = dslot == (NSLOT - 1) * POS ? 0u : dslot + POS;
    if (__builtin_expect(++dp >= dnp, 0)) next_item();
  };
  // The stream state is equal across the workgroup; saying so keeps it in
  // scalar registers (the compiler cannot always prove it).
  auto uniform_state = [&]() __attribute__((always_inline)) {
    issued = __builtin_amdgcn_readfirstlane(issued);
    dslot = __builtin_amdgcn_readfirstlane(dslot);
    dw = __builtin_amdgcn_readfirstlane(dw);
    dp = __builtin_amdgcn_readfirstlane(dp);
  };
  // every wave waits for its own copies of position x, then a barrier makes
  // all of them visible
  auto wait_pos = [&](int x) __attribute__((always_inline)) {
    const int k = issued - 1 - x;  // positions issued after x
    if (__builtin_expect(k == 2, 1)) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * OPS));  // the steady state
    else wait_vm(OPS * max(0, min(NSLOT - 1, k)));
  };
  // request positions up to low + NSLOT - 1 (slots of positions below low are free)
  auto refill = [&](int low) __attribute__((always_inline)) {
    if (issued < low + NSLOT && dw >= 0) issue();
    if (issued < low + NSLOT && dw >= 0) issue();
  };
  // One wave turns the L of position x (a block starting at row q0) into
  // L log2 e; a row past T, or one that saw no key, gets +inf, so its P and
  // dS are zero.
  auto scale_l = [&](int x, int q0) __attribute__((always_inline)) {
    if (tid < BQ) {
      float* l = reinterpret_cast<float*>(&ring[x % NSLOT][LOFF]);
      const float v = l[tid];
      l[tid] = q0 + tid < T && v != -INFINITY ? v * kLog2e : INFINITY;
    }
  };
  for (int i = 0; i < NSLOT - 1 && dw >= 0; ++i) issue();

  // Operand reads from a slot, as LDS byte addresses.  Because the swizzle
  // depends on row % 8 only, and every read starts at a row that is a multiple
  // of 8, a read's address is a per-lane base, XORed with a compile-time value
  // in granule bits 4..6, plus a compile-time row offset.
  typedef __attribute__((address_space(3))) V8 lds_v8;
  const unsigned ring0 = (unsigned)(uintptr_t)(lds_void_t*)(&ring[0][0]);
  // Row reads: lane (n, h) gets row row0 + n, columns 16 ks + 8 h .. + 7:
  // granule (2 ks + h) ^ swz128(n) = ((h ^ swz128(n)) ^ 2 ks).
  const unsigned rbase = n * RB + ((h ^ swz128(n)) << 4);
  auto ld_row = [&](unsigned sb, int t0, int row0, int ks) __attribute__((always_inline)) {
    return *(const lds_v8*)(uintptr_t)(((sb + rbase) ^ (ks << 5)) + t0 + row0 * RB);
  };
  // Transposing reads (ld_tr32 on swizzled rows): rows k0 + 4 h + u / 4 and
  // + 8, columns m0 + 16 g + 4 (u % 4) .. + 3; granule (m0 / 8 + y) ^ swz,
  // y = 2 g + (u % 4) / 2, with m0 / 8 = 4 dt.
  const int tu = lane & 15, tg = (lane >> 4) & 1;
  const int trow = 4 * h + (tu >> 2);
  const unsigned tbase = trow * RB + (((2 * tg + ((tu & 3) >> 1)) ^ swz128(trow)) << 4) + 8 * (tu & 1);
  auto ld_tr = [&](unsigned sb, int t0, int k0, int m0) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) i16x4 lds_i4;
    const unsigned p = ((sb + tbase) ^ ((m0 >> 5) << 6)) + t0 + k0 * RB;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i4*)(uintptr_t)p);
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i4*)(uintptr_t)(p + 8 * RB));
    typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
    i16x8 rr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(V8, rr);
  };
  auto slot_base = [&](int x) __attribute__((always_inline)) { return ring0 + (unsigned)((x % NSLOT) * POS); };

  V8 kf[NKS], vf[NKS];
  int pos = 0;  // next position to consume
  for (int round = 0;; ++round) {
    const int w = persistent_item(round, total);
    if (w < 0) break;
    const size_t base = item_base(w);
    const int j0w = (w % nkt) * BK;
    const int qb0 = item_qb0(w);
    const int c0 = j0w + wave * 32;  // first key of this wave
    const int col = c0 + n;          // this lane's key
    // Element e of a query tile starting at row ir is masked (causal) iff
    // ir + 8*(e/4) + 4h + e%4 < col, i.e. 8*(e/4) + e%4 < lo - ir.
    const int lo = col - 4 * h;

    // K and V of the tile (positions pos, pos + 1) into registers
    uniform_state();
    pos = __builtin_amdgcn_readfirstlane(pos);
    wait_pos(pos + 2);
    __syncthreads();
    refill(pos);
    scale_l(pos + 2, qb0 * BQ);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = ld_row(slot_base(pos), 0, 32 * wave, ks);
      vf[ks] = neg_frag(ld_row(slot_base(pos + 1), 0, 32 * wave, ks));
    }
    pos += 2;

    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = zero16();

    // Stages of one 32-row tile (tile it of the block in the slot at LDS
    // address sb, first row q0): A = the S and dP products, B = P and dS in
    // registers, C = the dV and dK products.  MASK: causal diagonal.
    auto stage_a = [&](unsigned sb, int it, f32x16& sa, f32x16& da) __attribute__((always_inline)) {
      typedef __attribute__((address_space(3))) f32x4 lds_f4;
      sa = zero16();
      // The second product starts from D of its rows and accumulates dO (-V)^T
      // (the V fragments are held negated), giving D - dP: stage B forms
      // dS = P (dP - D) = -P (D - dP) with one multiply.  For the first tile
      // of the next block (pipelined order) this read comes before that
      // block's barrier: its copies completed and became visible at the
      // barrier before, and D, unlike L, is never rewritten in LDS.
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const f32x4 d = *(const lds_f4*)(uintptr_t)(sb + LOFF + 4 * (BQ + 32 * it + 8 * bb + 4 * h));
#pragma unroll
        for (int r = 0; r < 4; ++r) da[4 * bb + r] = d[r];
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sa = mma32(ld_row(sb, 0, 32 * it, ks), kf[ks], sa);
        da = mma32(ld_row(sb, TILE, 32 * it, ks), vf[ks], da);
      }
      // keep each stage's operand reads next to its products (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    };
    auto stage_bc = [&](int sl, int q0, int it, f32x16& sc, f32x16& dc, auto masked) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(masked)::value;
      const unsigned sb = slot_base(sl);
      const float* cL = reinterpret_cast<const float*>(&ring[sl][LOFF]);
      const int lim = lo - (q0 + 32 * it);
      V8 bp[2], bs[2], bpl[2], bsl[2];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int rr = 32 * it + 8 * bb + 4 * h;
        const f32x4 lv = *reinterpret_cast<const f32x4*>(&cL[rr]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * bb + r;
          float p = fast_exp2(fmaf(sc[e], c2, -lv[r]));
          if (MASK && CAUSAL && 8 * bb + r < lim) p = 0.f;
          sc[e] = p;
          dc[e] = -(p * dc[e]);  // dc held D - dP
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
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const V8 ga = ld_tr(sb, TILE, 32 * it + 16 * st, 32 * dt);
          const V8 qa = ld_tr(sb, 0, 32 * it + 16 * st, 32 * dt);
          dv[dt] = mma32(ga, bp[st], dv[dt]);
          dk[dt] = mma32(qa, bs[st], dk[dt]);
          if (PREC == 1) {
            dv[dt] = mma32(ga, bpl[st], dv[dt]);
            dk[dt] = mma32(qa, bsl[st], dk[dt]);
          }
        }
    };
    // Block top: this block's data and the next position's are in LDS.
    auto top = [&](int q0) __attribute__((always_inline)) {
      uniform_state();
      wait_pos(pos + 1);
      __syncthreads();
      refill(pos);
      scale_l(pos + 1, q0 + BQ);  // the next block, or unused space of the next item's K
    };
    using F = std::false_type;
    using Tr = std::true_type;
    static_assert(NIT == 2, "two tiles per block");
    f32x16 sA, dA, sB, dB;

    // Under the causal mask the item's first two blocks hold the diagonal: a
    // wave skips tiles wholly above its first key (c0 - q0 is a multiple of
    // 32) and masks the rest element-wise, tile by tile in the order A(1),
    // B(0), C(0), B(1), C(1).
    const int qbf = CAUSAL ? min(qb0 + BK / BQ, nqb) : qb0;
    for (int qb = qb0; qb < qbf; ++qb, ++pos) {
      const int q0 = qb * BQ;
      top(q0);
      const int sl = pos % NSLOT;
      const unsigned sb = slot_base(sl);
      if (q0 + BQ - 1 >= c0) {
        if (q0 < c0 + 31) {
          if (q0 >= c0) {
            stage_a(sb, 0, sA, dA);
            stage_a(sb, 1, sB, dB);
            stage_bc(sl, q0, 0, sA, dA, Tr{});
          } else {
            stage_a(sb, 1, sB, dB);
          }
          stage_bc(sl, q0, 1, sB, dB, Tr{});
        } else {
          stage_a(sb, 0, sA, dA);
          stage_a(sb, 1, sB, dB);
          stage_bc(sl, q0, 0, sA, dA, F{});
          stage_bc(sl, q0, 1, sB, dB, F{});
        }
      }
    }
    // The other blocks are visible to every key of the item: one pipeline
    // over their tiles, in the order A(t+1), B(t), C(t), also across blocks.
    if (qbf < nqb) {
      top(qbf * BQ);
      stage_a(slot_base(pos), 0, sA, dA);
      int qb = qbf;
      for (; qb + 1 < nqb; ++qb) {
        const int q0 = qb * BQ;
        const int sl = pos % NSLOT;
        stage_a(slot_base(sl), 1, sB, dB);
        stage_bc(sl, q0, 0, sA, dA, F{});
        stage_a(slot_base(pos + 1), 0, sA, dA);  // the next block's first tile
        stage_bc(sl, q0, 1, sB, dB, F{});
        ++pos;
        top(q0 + BQ);
      }
      const int sl = pos % NSLOT;
      stage_a(slot_base(sl), 1, sB, dB);
      stage_bc(sl, qb * BQ, 0, sA, dA, F{});
      stage_bc(sl, qb * BQ, 1, sB, dB, F{});
      ++pos;
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
  }
}

}  // namespace fa
