// Unfused attention forward (float32): the three-kernel schedule the
// fused-attention lesson compares against ("Lesson K23, fused attention",
// block "sources", Algorithm 0 of the FlashAttention paper as the page quotes
// it): a scores kernel writes S = scale Q K^T to global memory, a softmax
// kernel reads S back and writes P over it, and a third kernel reads P and V
// and writes O = P V.  The N x N score matrix is written, read, written as P
// and read again: 4 N^2 floats of global traffic per head that the fused
// kernel does not have (block "lab", field "predicts").
//
// Each kernel is a plain tiled kernel on v_mfma_f32_16x16x4_f32 (see the
// layouts in fa_common.hpp); they exist as the comparator of the lab
// measurement, not as a fast path.
#pragma once
#include "fa_common.hpp"

namespace fa {

struct UnfusedArgs {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* s;  // [B, H, T, T] scores, overwritten with P
  int B, H, T;
  float scale;
};

// S[bh][i][j] = scale <q_i, k_j> for one 64 x 64 tile; 4 waves of 16 rows.
template <int HD>
__global__ __launch_bounds__(256) void scores_kernel(UnfusedArgs a) {
  constexpr int LD = HD + 4;
  __shared__ __attribute__((aligned(16))) float sQ[64 * LD];
  __shared__ __attribute__((aligned(16))) float sK[64 * LD];
  const int T = a.T, H = a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64, bh = blockIdx.z;
  const int b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * HD;
  const float* Q = a.q + ((size_t)b * T * H + hh) * HD;
  const float* K = a.k + ((size_t)b * T * H + hh) * HD;
  for (int x = tid; x < 64 * HD / 4; x += 256) {
    const int r = x / (HD / 4), c = (x % (HD / 4)) * 4;
    const f32x4 zq = zero4();
    const f32x4 vq = i0 + r < T ? *reinterpret_cast<const f32x4*>(Q + (size_t)(i0 + r) * rs + c) : zq;
    const f32x4 vk = j0 + r < T ? *reinterpret_cast<const f32x4*>(K + (size_t)(j0 + r) * rs + c) : zq;
    *reinterpret_cast<f32x4*>(sQ + r * LD + c) = vq;
    *reinterpret_cast<f32x4*>(sK + r * LD + c) = vk;
  }
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = zero4();
#pragma unroll
  for (int ks = 0; ks < HD / 4; ++ks) {
    const float af = sQ[(16 * wave + li) * LD + 4 * ks + lg];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const float bf = sK[(16 * jt + li) * LD + 4 * ks + lg];
      acc[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bf, acc[jt], 0, 0, 0);
    }
  }
  float* S = a.s + (size_t)bh * T * T;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int j = j0 + 16 * jt + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 16 * wave + 4 * lg + r;
      if (i < T && j < T) S[(size_t)i * T + j] = a.scale * acc[jt][r];
    }
  }
}

// Row softmax in place, one wave per row: P_ij = exp(s_ij - m_i) / l_i over
// the visible keys, 0 for masked ones.
template <bool CAUSAL>
__global__ __launch_bounds__(256) void softmax_kernel(UnfusedArgs a) {
  const int T = a.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wave, bh = blockIdx.y;
  if (i >= T) return;
  float* row = a.s + ((size_t)bh * T + i) * T;
  const int nvis = CAUSAL ? i + 1 : T;
  float m = -INFINITY;
  for (int j = lane; j < nvis; j += 64) m = fmaxf(m, row[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.f;
  for (int j = lane; j < nvis; j += 64) l += fast_exp2((row[j] - m) * kLog2e);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  const float inv = 1.f / l;
  for (int j = lane; j < T; j += 64) row[j] = j < nvis ? fast_exp2((row[j] - m) * kLog2e) * inv : 0.f;
}

// O[i][:] = sum_j P[i][j] V[j][:] for 64 query rows; 4 waves of 16 rows, key
// chunks of 64 through LDS.
template <int HD, bool CAUSAL>
__global__ __launch_bounds__(256) void pv_kernel(UnfusedArgs a) {
  constexpr int HDP = HD < 16 ? 16 : HD;  // output tiles are 16 columns wide
  constexpr int NDT = HDP / 16;
  constexpr int LDP = 64 + 4, LDV = HDP + 4;
  __shared__ __attribute__((aligned(16))) float sP[64 * LDP];
  __shared__ __attribute__((aligned(16))) float sV[64 * LDV];
  const int T = a.T, H = a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int i0 = blockIdx.x * 64, bh = blockIdx.y;
  const int b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * HD;
  const float* V = a.v + ((size_t)b * T * H + hh) * HD;
  const float* P = a.s + (size_t)bh * T * T;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero4();
  const int jend = CAUSAL ? min(T, i0 + 64) : T;
  for (int j0 = 0; j0 < jend; j0 += 64) {
    for (int x = tid; x < 64 * 16; x += 256) {
      const int r = x / 16, c = (x % 16) * 4;
      f32x4 vp = zero4();
      if (i0 + r < T) {
        const float* src = P + (size_t)(i0 + r) * T + j0 + c;
        if (j0 + c + 3 < T && (T & 3) == 0) {
          vp = *reinterpret_cast<const f32x4*>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) vp[e] = j0 + c + e < T ? src[e] : 0.f;
        }
      }
      *reinterpret_cast<f32x4*>(sP + r * LDP + c) = vp;
    }
    for (int x = tid; x < 64 * HDP / 4; x += 256) {
      const int r = x / (HDP / 4), c = (x % (HDP / 4)) * 4;
      f32x4 vv = zero4();
      if (j0 + r < T && c < HD) vv = *reinterpret_cast<const f32x4*>(V + (size_t)(j0 + r) * rs + c);
      *reinterpret_cast<f32x4*>(sV + r * LDV + c) = vv;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const float af = sP[(16 * wave + li) * LDP + 4 * ks + lg];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const float bf = sV[(4 * ks + lg) * LDV + 16 * dt + li];
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bf, acc[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  float* O = a.o + ((size_t)b * T * H + hh) * HD;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int c = 16 * dt + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 16 * wave + 4 * lg + r;
      if (i < T && c < HD) O[(size_t)i * rs + c] = acc[dt][r];
    }
  }
}

template <int HD>
int run_unfused(const UnfusedArgs& a, bool causal, hipStream_t s) {
  const unsigned nt = (unsigned)((a.T + 63) / 64), bhn = (unsigned)(a.B * a.H);
  hipLaunchKernelGGL(scores_kernel<HD>, dim3(nt, nt, bhn), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return kErrLaunch;
  if (causal)
    hipLaunchKernelGGL(softmax_kernel<true>, dim3((unsigned)((a.T + 3) / 4), bhn), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(softmax_kernel<false>, dim3((unsigned)((a.T + 3) / 4), bhn), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return kErrLaunch;
  if (causal)
    hipLaunchKernelGGL((pv_kernel<HD, true>), dim3(nt, bhn), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((pv_kernel<HD, false>), dim3(nt, bhn), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : kErrLaunch;
}

}  // namespace fa
