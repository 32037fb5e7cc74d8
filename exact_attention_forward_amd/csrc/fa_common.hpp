// Shared device-side building blocks of the attention kernels for gfx950 (CDNA4).
//
// Matrix products use 16x16 MFMA tiles with 64-lane wavefronts.  Lane l is
// split as li = l % 16 and lg = l / 16.  For every MFMA used here the lane
// layouts are:
//   A (16 x K): lane (li, lg) holds row li, a group of K/4 contraction indices
//   B (K x 16): lane (li, lg) holds column li, the same contraction group
//   C (16 x 16, float): lane (li, lg) holds column li, rows 4*lg + r, r = 0..3
// For v_mfma_f32_16x16x4_f32 the group is the single index lg; for
// v_mfma_f32_16x16x32_bf16 it is the eight indices 8*lg .. 8*lg+7.
//
// A contraction is invariant under any permutation of its index applied to
// both operands.  The kernels use this to feed a C tile (an S or dS tile just
// produced) straight back as the B operand of the next product without moving
// data between lanes: lane (li, lg) of a C tile already holds four consecutive
// contraction indices 4*lg + r of column li.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Status codes of the launchers: the C ABI's FA_ERR_UNSUPPORTED and
// FA_ERR_LAUNCH (the ABI layer checks that the values agree).
constexpr int kErrUnsupported = -3;
constexpr int kErrLaunch = -5;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct bf16_t {
  uint16_t bits;
};
// IEEE binary16 storage (the kernels convert through _Float16).
struct f16_t {
  uint16_t bits;
};
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));

// -x of an MFMA operand fragment: a float, or eight 16-bit floats (bfloat16
// or binary16, sign bits flipped).
__device__ __forceinline__ float neg_frag(float x) { return -x; }
__device__ __forceinline__ bf16x8 neg_frag(bf16x8 x) {
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x) ^ 0x80008000u);
}
__device__ __forceinline__ f16x8 neg_frag(f16x8 x) {
  return __builtin_bit_cast(f16x8, __builtin_bit_cast(u32x4, x) ^ 0x80008000u);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Butterfly reductions across the four lane groups (lanes l, l^16, l^32, l^48)
// that share a column li of a C tile.
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Workgroups go to the 8 XCDs round-robin (id % 8).  Map the hardware id to a
// logical work index so that each XCD receives one contiguous range of
// logical work: tiles of the same head then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  const int q = total / 8, rem = total % 8;
  const int x = wg % 8, slot = wg / 8;
  return x * q + (x < rem ? x : rem) + slot;
}

// Persistent-workgroup schedule.  Logical work items [0, total) are split into
// 8 contiguous ranges, one per XCD (workgroup w runs on XCD w % 8).  Round r
// hands the XCD's workgroups consecutive items of its range, in reverse
// order on odd rounds, so long and short causal items pair up.  Returns the
// item for (round r, this workgroup), or -1 once the range is exhausted; the
// result is uniform across the workgroup.
__device__ __forceinline__ int persistent_item(int r, int total) {
  const int G = gridDim.x, w = blockIdx.x;
  const int x = w % 8, slot = w / 8;
  const int nslots = (G - x + 7) / 8;
  const int q = total / 8, rem = total % 8;
  const int start = x * q + (x < rem ? x : rem), count = q + (x < rem ? 1 : 0);
  const int local = r * nslots + ((r & 1) ? nslots - 1 - slot : slot);
  return local < count ? start + local : -1;
}

// ---------------------------------------------------------------------------
// MFMA policies.  Each supplies:
//   KS     contraction length of one instruction
//   CH     contraction length of one register chunk (C tiles fed back as B)
//   NSTEP  instructions per register chunk
//   VEC    elements per 16-byte vector
//   frag   operand register type
//   mma(a, b, c)                  c += a * b
//   ld_row(X, ld, row0, k0)       A/B operand from a row-major LDS tile:
//                                 X[row0 + li][k0 + group]
//   ld_trans(Y, ld, k0, m0, step) A operand of Y^T from a row-major LDS tile
//                                 Y[k][m]: rows m0 + li, contraction indices
//                                 matching pack(..., step)
//   pack(c, step)                 B operand from the CH/16 C tiles c[]
// ---------------------------------------------------------------------------
template <typename T>
struct Mma;

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int CH = 16;
  static constexpr int NSTEP = 4;
  static constexpr int VEC = 4;
  using frag = float;

  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag ld_row(const float* X, int ld, int row0, int k0, int li, int lg) {
    return X[(row0 + li) * ld + k0 + lg];
  }
  // Step r of the 16-long chunk starting at k0 uses index k0 + 4*lg + r.
  __device__ __forceinline__ static frag ld_trans(const float* Y, int ld, int k0, int m0, int step, int li, int lg) {
    return Y[(k0 + 4 * lg + step) * ld + m0 + li];
  }
  __device__ __forceinline__ static frag pack(const f32x4* c, int step) { return c[0][step]; }
  __device__ __forceinline__ static frag pack_lo(const f32x4* c, int step) { return 0.f; }
  // Operand from global memory (row-major, leading dimension ld), zero past nrows.
  __device__ __forceinline__ static frag ld_row_global(const float* X, size_t ld, int row, int nrows, int k0, int lg) {
    return row < nrows ? X[(size_t)row * ld + k0 + lg] : 0.f;
  }
};

__device__ __forceinline__ bf16x8 cvt8(const f32x4& a, const f32x4& b) {
  bf16x8 r;
  r[0] = (__bf16)a[0];
  r[1] = (__bf16)a[1];
  r[2] = (__bf16)a[2];
  r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0];
  r[5] = (__bf16)b[1];
  r[6] = (__bf16)b[2];
  r[7] = (__bf16)b[3];
  return r;
}

template <>
struct Mma<bf16_t> {
  static constexpr int KS = 32;
  static constexpr int CH = 32;
  static constexpr int NSTEP = 1;
  static constexpr int VEC = 8;
  using frag = bf16x8;

  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag ld_row(const bf16_t* X, int ld, int row0, int k0, int li, int lg) {
    return *reinterpret_cast<const frag*>(X + (row0 + li) * ld + k0 + 8 * lg);
  }
  // Two LDS transpose reads.  Within each 16-lane group, ds_read_b64_tr_b16
  // returns to lane s, element e, the element s % 4 of the 4-element vector
  // addressed by lane 4*e + s / 4.  Lane (s, lg) therefore addresses row
  // k0 + 4*lg + s/4, columns m0 + 4*(s%4) .. +3, and receives
  // Y[k0 + 4*lg + e][m0 + s] for e = 0..3; the second read covers rows
  // k0 + 16 + 4*lg + e.  These are the indices pack() places in elements 0..7.
  __device__ __forceinline__ static frag ld_trans(const bf16_t* Y, int ld, int k0, int m0, int step, int li, int lg) {
    const bf16_t* p = Y + (k0 + 4 * lg + (li >> 2)) * ld + m0 + 4 * (li & 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * ld));
    typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
    i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, r);
  }
  __device__ __forceinline__ static frag pack(const f32x4* c, int step) { return cvt8(c[0], c[1]); }
  // Residual after rounding to bfloat16: x - (float)bf16(x), itself rounded.
  __device__ __forceinline__ static frag pack_lo(const f32x4* c, int step) {
    f32x4 a, b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = c[0][r] - (float)(__bf16)c[0][r];
      b[r] = c[1][r] - (float)(__bf16)c[1][r];
    }
    return cvt8(a, b);
  }
  __device__ __forceinline__ static frag ld_row_global(const bf16_t* X, size_t ld, int row, int nrows, int k0, int lg) {
    if (row < nrows) return *reinterpret_cast<const frag*>(X + (size_t)row * ld + k0 + 8 * lg);
    frag z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    return z;
  }
};

// IEEE half inputs: v_mfma_f32_16x16x32_f16, the same lane layouts as the
// bfloat16 policy (16-bit elements, eight per operand).
__device__ __forceinline__ f16x8 cvt8h(const f32x4& a, const f32x4& b) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (_Float16)a[e];
    r[4 + e] = (_Float16)b[e];
  }
  return r;
}

template <>
struct Mma<f16_t> {
  static constexpr int KS = 32;
  static constexpr int CH = 32;
  static constexpr int NSTEP = 1;
  static constexpr int VEC = 8;
  using frag = f16x8;

  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag ld_row(const f16_t* X, int ld, int row0, int k0, int li, int lg) {
    return *reinterpret_cast<const frag*>(X + (row0 + li) * ld + k0 + 8 * lg);
  }
  // Transposing reads as in Mma<bf16_t>::ld_trans (16-bit elements).
  __device__ __forceinline__ static frag ld_trans(const f16_t* Y, int ld, int k0, int m0, int step, int li, int lg) {
    const f16_t* p = Y + (k0 + 4 * lg + (li >> 2)) * ld + m0 + 4 * (li & 3);
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * ld));
    typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
    i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag, r);
  }
  __device__ __forceinline__ static frag pack(const f32x4* c, int step) { return cvt8h(c[0], c[1]); }
  __device__ __forceinline__ static frag pack_lo(const f32x4* c, int step) {
    f32x4 a, b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = c[0][r] - (float)(_Float16)c[0][r];
      b[r] = c[1][r] - (float)(_Float16)c[1][r];
    }
    return cvt8h(a, b);
  }
  __device__ __forceinline__ static frag ld_row_global(const f16_t* X, size_t ld, int row, int nrows, int k0, int lg) {
    if (row < nrows) return *reinterpret_cast<const frag*>(X + (size_t)row * ld + k0 + 8 * lg);
    frag z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.f;
    return z;
  }
};

// Padded LDS row length (elements).  Rows stay 16-byte aligned; the f32 path
// keeps at least 16 columns because its output tiles are 16 columns wide.
// 16-bit rows of hd 128 take 16 elements of padding here and 24 in the 32x32
// kernels (their LD): with 8, the LDS reads of those kernels conflicted on
// 18-26% of LDS cycles, and the wider pitches made the B4 H16 T8192 hd128
// kernels 1-4% faster (bitwise equal results).
template <typename T, int HD>
constexpr int lds_ld() {
  return (sizeof(T) == 4) ? ((HD < 16 ? 16 : HD) + 4) : (HD <= 64 ? HD + 8 : HD + 16);
}

// Cooperative copy of rows [row0, row0 + ROWS) of a row-major global matrix
// (leading dimension gld, nrows valid rows, HD columns) into registers, then
// into an LDS tile.  Rows past nrows repeat row nrows - 1 (finite data, so a
// zero weight on them contributes exactly zero); every kernel masks or zeroes
// the weights of those rows.  The loads carry no branches.
template <typename T, int HD, int ROWS, int NT>
struct TileCopy {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int VPR = HD / VEC;  // vectors per row
  static constexpr int NV = ROWS * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  u32x4 r[PER];  // a native vector type, so the copies stay in registers

  __device__ __forceinline__ void load(const T* G, size_t gld, int row0, int nrows, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * NT;
      const int row = v / VPR, col = (v % VPR) * VEC;
      if (NV % NT == 0 || v < NV) {
        const int gr = min(row0 + row, nrows - 1);
        r[p] = *reinterpret_cast<const u32x4*>(G + (size_t)gr * gld + col);
      }
    }
  }
  __device__ __forceinline__ void store(T* S, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * NT;
      const int row = v / VPR, col = (v % VPR) * VEC;
      if (NV % NT == 0 || v < NV) *reinterpret_cast<u32x4*>(S + row * ld + col) = r[p];
    }
  }
};

}  // namespace fa
