// 32x32 MFMA building blocks for the 16-bit kernels (v_mfma_f32_32x32x16_bf16
// and v_mfma_f32_32x32x16_f16).  Tiles in LDS and global memory are handled
// as 16-bit bit patterns; the operand vector type V (bf16x8 or f16x8) decides
// the product, the rounding of float results to operands, and nothing else.
//
// Lane l is split as n = l % 32 and h = l / 32.  Layouts:
//   A (32 x 16): lane (n, h) holds row n, contraction indices 8h .. 8h+7
//   B (16 x 32): lane (n, h) holds column n, contraction indices 8h .. 8h+7
//   C (32 x 32, float): lane (n, h) holds column n, rows 8b + 4h + r in
//                       element 4b + r (b, r = 0..3)
// On gfx950 this instruction sustains about twice the flop rate of the
// 16x16x32 form, and a 32-row wave tile halves the LDS bytes per flop.
//
// A C tile is fed back as the B operand of the next product without moving
// data between lanes: product step s (16 contraction indices) uses C rows
// 16s + 4h + r (elements 8s + r) and 16s + 8 + 4h + r (elements 8s + 4 + r).
// The matching A operand is read from a row-major LDS tile with the LDS
// transpose read: within each 16-lane group, ds_read_b64_tr_b16 returns to
// lane u, element e, the element u % 4 of the 4-vector addressed by lane
// 4e + u / 4.
#pragma once
#include "fa_common.hpp"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Operand vector of an input storage type, and a vector's element type.
template <typename TIn>
struct Frag32;
template <>
struct Frag32<bf16_t> {
  using V = bf16x8;
};
template <>
struct Frag32<f16_t> {
  using V = f16x8;
};
template <typename V>
struct VecElem;
template <>
struct VecElem<bf16x8> {
  using E = __bf16;
};
template <>
struct VecElem<f16x8> {
  using E = _Float16;
};

// X[row0 + n][k0 + 8h .. +7] from a row-major LDS tile.
template <typename V = bf16x8>
__device__ __forceinline__ V ld_row32(const bf16_t* X, int ld, int row0, int k0, int n, int h) {
  return *reinterpret_cast<const V*>(X + (row0 + n) * ld + k0 + 8 * h);
}

// A operand Y^T for one 16-long product step starting at row k0 of a
// row-major LDS tile Y[k][m]: lane (n, h) receives Y[k][m0 + n] for
// k = k0 + 4h + e (elements 0..3) and k = k0 + 8 + 4h + e (elements 4..7).
template <typename V = bf16x8>
__device__ __forceinline__ V ld_tr32(const bf16_t* Y, int ld, int k0, int m0, int lane) {
  const int u = lane & 15, g = (lane >> 4) & 1, h = lane >> 5;
  const bf16_t* p = Y + (k0 + 4 * h + (u >> 2)) * ld + m0 + 16 * g + 4 * (u & 3);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * ld));
  typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
  i16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V, r);
}

// B operand for product step s from a C tile (elements 8s .. 8s+7), rounded
// to nearest.
template <typename V = bf16x8>
__device__ __forceinline__ V pack32(const f32x16& c, int s) {
  using E = typename VecElem<V>::E;
  V r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (E)c[8 * s + e];
  return r;
}
// Residual x - round(x) of the same elements, rounded again.
template <typename V = bf16x8>
__device__ __forceinline__ V pack32_lo(const f32x16& c, int s) {
  using E = typename VecElem<V>::E;
  V r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = c[8 * s + e];
    r[e] = (E)(x - (float)(E)x);
  }
  return r;
}

// Row of a C tile held in element e of lane half h: 8*(e/4) + 4h + e%4.
__device__ __forceinline__ int crow(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

// B operand (or A operand) straight from global memory: row `row` (zero if
// past nrows), elements k0 + 8h .. +7.
template <typename V = bf16x8>
__device__ __forceinline__ V ld_row_global32(const bf16_t* X, size_t ld, int row, int nrows, int k0, int h) {
  if (row < nrows) return *reinterpret_cast<const V*>(X + (size_t)row * ld + k0 + 8 * h);
  V z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (typename VecElem<V>::E)0.f;
  return z;
}


// Global -> register -> LDS copy of a block of ROWS rows x HD bfloat16 columns
// (row-major, leading dimension gld elements in global memory, LD in LDS).
// The per-thread byte offsets are computed once, so a block load is one
// scalar base pointer plus a 32-bit offset per vector.  load() needs all ROWS
// rows present; load_clamped() repeats the last valid row past nrows (finite
// data, so zero weights on those rows contribute exactly zero).
template <int HD, int ROWS, int NT>
struct TileStream {
  static constexpr int VPR = HD / 8;  // 16-byte vectors per row
  static constexpr int NV = ROWS * VPR;
  static constexpr int PER = (NV + NT - 1) / NT;
  static_assert(NV % NT == 0, "copy must divide evenly");
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t r[PER];

  __device__ __forceinline__ static int vrow(int tid, int p) { return (tid + p * NT) / VPR; }
  __device__ __forceinline__ static int vcol(int tid, int p) { return ((tid + p * NT) % VPR) * 8; }

  // goff[p]: byte offset of vector p from the block's first row.
  __device__ __forceinline__ void load(const bf16_t* G, const unsigned* goff) {
#pragma unroll
    for (int p = 0; p < PER; ++p) r[p] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(G) + goff[p]);
  }
  __device__ __forceinline__ void load_clamped(const bf16_t* G, size_t gld, int row0, int nrows, int tid) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int gr = min(row0 + vrow(tid, p), nrows - 1);
      r[p] = *reinterpret_cast<const u32x4_t*>(G + (size_t)gr * gld + vcol(tid, p));
    }
  }
  __device__ __forceinline__ void store(bf16_t* S, int ld, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) *reinterpret_cast<u32x4_t*>(S + vrow(tid, p) * ld + vcol(tid, p)) = r[p];
  }
};

}  // namespace fa
