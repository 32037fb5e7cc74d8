// Split-key forward: the merge of per-split partial results.
//
// A split handles one range of keys and produces, for every row, the partial
// output O_s (normalised by its own row sum) and L_s = m_s + ln l_s; a split
// that sees no key of a row leaves L_s = -inf, O_s = 0.  The partial states
// combine with the associative merge of the online normaliser ("Flash
// Attention 2 -- forward pass notes", the merge after the loop; the
// fused-attention lesson, block "sources.onlineSoftmax", calls it associative
// and commutative): with M = max_s L_s,
//   L = M + ln sum_s exp(L_s - M),   O = sum_s exp(L_s - L) O_s.
// The merge here walks the splits in order with a running (M, sum, O).
#pragma once
#include "fa_common.hpp"

namespace fa {

struct MergeArgs {
  const float* opart;  // [nsplit][B, T, H, hd]
  const float* lpart;  // [nsplit][B, H, T]
  float* o;
  float* lse;
  int B, H, T, nsplit;
  size_t o_split, lse_split;
};

template <int HD>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int G = HD / 4;  // float4 groups per row
  constexpr int RPB = 256 / G;
  const int t = threadIdx.x;
  const int r = t / G, c = (t % G) * 4;
  const int bh = blockIdx.y, i = blockIdx.x * RPB + r;
  const int T = a.T, H = a.H;
  if (i >= T) return;
  const int b = bh / H, hh = bh % H;
  const size_t off = ((size_t)b * T * H + hh) * HD + (size_t)i * H * HD + c;
  const size_t loff = (size_t)bh * T + i;
  float M = -INFINITY, S = 0.f;
  f32x4 acc = zero4();
  for (int s = 0; s < a.nsplit; ++s) {
    const float Ls = a.lpart[s * a.lse_split + loff];
    if (Ls == -INFINITY) continue;
    const float Mn = fmaxf(M, Ls);
    const float keep = M == -INFINITY ? 0.f : expf(M - Mn);
    const float w = expf(Ls - Mn);
    const f32x4 os = *reinterpret_cast<const f32x4*>(a.opart + s * a.o_split + off);
    acc = acc * keep + os * w;
    S = S * keep + w;
    M = Mn;
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  *reinterpret_cast<f32x4*>(a.o + off) = acc * inv;
  if (c == 0) a.lse[loff] = S > 0.f ? M + logf(S) : -INFINITY;
}

}  // namespace fa
