// Kernel instantiation and launch helpers shared by the per-dtype translation
// units.  Tile shapes per (input type, head dim) live in TileCfg.
#pragma once
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "fa_bwd.hpp"
#include "fa_bwd32.hpp"
#include "fa_bwd64.hpp"
#include "fa_fwd.hpp"
#include "fa_fwd32.hpp"
#include "fa_fwd64.hpp"
#include "fa_split.hpp"
#include "fa_unfused.hpp"

namespace fa {

// NW waves per workgroup; MR 16-row subtiles per wave; BC/BQ rows of the
// streamed side per LDS block.
template <typename TIn, int HD>
struct TileCfg;

// 16-bit kernels use 32x32 tiles: NW waves of 32 rows each.  The block
// sizes can be overridden at compile time for tuning sweeps.
#ifndef FA_FWD_BC64
#define FA_FWD_BC64 32
#endif
#ifndef FA_FWD_NW64
#define FA_FWD_NW64 2
#endif
#ifndef FA_FWD_MS64
#define FA_FWD_MS64 2
#endif
#ifndef FA_DQ_BC64
#define FA_DQ_BC64 64
#endif
// hd 128: 32-key blocks in the forward and dQ kernels fit two waves per SIMD
// (forward 217-231 VGPRs, dQ without fused D 232-235).  A 32x32 dK/dV kernel
// cannot (236 spills at 256), so 16-bit hd 128 dK/dV, and dQ without the
// causal mask, run the 16x16 kernels (see run_dq, run_dkv); 16-bit hd 64 dK/dV
// runs dkv64_kernel.
#ifndef FA_FWD_BC128
#define FA_FWD_BC128 32
#endif
#ifndef FA_DQ_BC128
#define FA_DQ_BC128 32
#endif
#ifndef FA_NW64
#define FA_NW64 4
#endif
// FWD_MS: 32-row sub-tiles per wave in the forward (rows per workgroup = 32 NW MS).
// The 32x32 forward serves hd 128 and the split-key forward; hd 64's plain
// forward is fwd64_kernel.
template <int HD>
struct TileCfg32 {
  static constexpr int FWD_NW = HD <= 64 ? FA_FWD_NW64 : 4, FWD_BC = HD <= 64 ? FA_FWD_BC64 : FA_FWD_BC128;
  static constexpr int FWD_MS = HD <= 64 ? FA_FWD_MS64 : 1;
  static constexpr int DQ_NW = HD <= 64 ? FA_NW64 : 4, DQ_BC = HD <= 64 ? FA_DQ_BC64 : FA_DQ_BC128;
};

template <int HD>
struct TileCfg<float, HD> {
  static constexpr int FWD_NW = 4, FWD_MR = HD <= 64 ? 2 : 1, FWD_BC = 32;
  static constexpr int DQ_NW = 4, DQ_MR = HD <= 64 ? 2 : 1, DQ_BC = 32;
  static constexpr int DKV_NW = 4, DKV_MR = HD <= 64 ? 2 : 1, DKV_BQ = 32;  // hd 128: one row tile per wave fits two
                                                                            // waves per SIMD without spills
};
template <>
struct TileCfg<bf16_t, 64> {
  static constexpr int FWD_NW = 4, FWD_MR = 2, FWD_BC = 64;
  static constexpr int DQ_NW = 4, DQ_MR = 2, DQ_BC = 64;
  static constexpr int DKV_NW = 4, DKV_MR = 2, DKV_BQ = 64;
};
template <int HD>
struct TileCfg<f16_t, HD> : TileCfg<bf16_t, HD> {};
template <>
struct TileCfg<bf16_t, 128> {
  static constexpr int FWD_NW = 4, FWD_MR = 2, FWD_BC = 64;
  static constexpr int DQ_NW = 4, DQ_MR = 1, DQ_BC = 64;
  static constexpr int DKV_NW = 4, DKV_MR = 1, DKV_BQ = 64;
};

inline int launch_status() { return hipGetLastError() == hipSuccess ? 0 : kErrLaunch; }

// Compute units of the current device (cached per device id; calls from
// several host threads may fill an entry concurrently with the same value).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Resident workgroups per compute unit of one kernel on the current device.
// The cache is keyed by (device, kernel address, block size): kernels of one
// function type (every forward instantiation, say) have different register
// and LDS footprints, so each needs its own entry.
inline int resident_per_cu(const void* kernel, int threads) {
  struct Entry {
    int dev;
    const void* kernel;
    int threads;
    int per_cu;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  {
    std::lock_guard<std::mutex> g(mu);
    for (const Entry& e : cache)
      if (e.dev == dev && e.kernel == kernel && e.threads == threads) return e.per_cu;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0) n = 1;
  std::lock_guard<std::mutex> g(mu);
  cache.push_back(Entry{dev, kernel, threads, n});
  return n;
}

// Grid for a persistent kernel: every resident workgroup slot, at most one per item.
template <typename K>
inline long persistent_grid(K kernel, int threads, long items) {
  const long slots = (long)resident_per_cu(reinterpret_cast<const void*>(kernel), threads) * device_cus();
  return items < slots ? items : slots;
}

template <typename TIn>
constexpr bool is_bf16 = std::is_same<TIn, bf16_t>::value;
// 16-bit inputs run the 32x32 kernels
template <typename TIn>
constexpr bool is_16bit = std::is_same<TIn, bf16_t>::value || std::is_same<TIn, f16_t>::value;

template <typename TIn, int HD, bool CAUSAL, int PREC, int CONTROL = kCtlNone>
int run_fwd(const FwdArgs& a, hipStream_t s) {
  if constexpr (CONTROL != kCtlNone && is_bf16<TIn>) {
    return kErrUnsupported;  // the control variants are built for float32 and half inputs only
  } else if constexpr (CONTROL == kCtlNone && is_16bit<TIn> && HD == 64) {
    // hd 64: the pipelined forward with K/V streamed into an LDS ring
    auto* k = &fwd64_kernel<TIn, CAUSAL, PREC>;
    const long items = (long)((a.T + 127) / 128) * a.B * a.H;
    FwdArgs b = a;
    if constexpr (!is_bf16<TIn>) b.one2 = 0x3C003C00u;  // half pair (1, 1) for the row sums
    hipLaunchKernelGGL(k, dim3((unsigned)persistent_grid(k, 128, items)), dim3(128), 0, s, b);
    return launch_status();
  } else if constexpr (CONTROL == kCtlNone && is_16bit<TIn>) {
    using C = TileCfg32<HD>;
    auto* k = &fwd32_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_BC, C::FWD_MS>;
    constexpr int BR = C::FWD_NW * 32 * C::FWD_MS;
    const long items = (long)((a.T + BR - 1) / BR) * a.B * a.H;
    FwdArgs b = a;
    if constexpr (!is_bf16<TIn>) b.one2 = 0x3C003C00u;  // half pair (1, 1) for the row sums
    hipLaunchKernelGGL(k, dim3((unsigned)persistent_grid(k, C::FWD_NW * 64, items)), dim3(C::FWD_NW * 64), 0, s, b);
    return launch_status();
  } else {
    using C = TileCfg<TIn, HD>;
    constexpr int BR = C::FWD_NW * 16 * C::FWD_MR;
    const long nqt = (a.T + BR - 1) / BR;
    const long grid = nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_MR, C::FWD_BC, CONTROL>),
                       dim3((unsigned)grid), dim3(C::FWD_NW * 64), 0, s, a);
    return launch_status();
  }
}

template <typename TIn, int HD>
int run_delta(const BwdArgs& a, hipStream_t s) {
  constexpr int RPB = 256 / (HD / 4);
  const long nrows = (long)a.B * a.T * a.H;
  hipLaunchKernelGGL((delta_kernel<TIn, HD>), dim3((unsigned)((nrows + RPB - 1) / RPB)), dim3(256), 0, s, a);
  return launch_status();
}

template <typename TIn, int HD, bool CAUSAL, int PREC, bool FUSE_D = false>
int run_dq(const BwdArgs& a, hipStream_t s) {
  // 16-bit hd 128 without the causal mask runs the 16x16 kernel: there the
  // 32x32 one needs 356-398 VGPRs (one wave per SIMD), and the 16x16 one at
  // two waves is 13% faster at B4 H16 T8192.
  if constexpr (is_16bit<TIn> && (HD <= 64 || CAUSAL)) {
    using C = TileCfg32<HD>;
    // hd 128 takes D from the pre-pass: the O rows for fusing it would need
    // 64 more VGPRs and the kernel would drop to one wave per SIMD
    if constexpr (HD > 64 && FUSE_D) {
      const int st = run_delta<TIn, HD>(a, s);
      if (st) return st;
    }
    auto* k = &dq32_kernel<TIn, HD, CAUSAL, PREC, C::DQ_NW, C::DQ_BC, (HD > 64 ? false : FUSE_D)>;
    const long items = (long)((a.T + C::DQ_NW * 32 - 1) / (C::DQ_NW * 32)) * a.B * a.H;
    hipLaunchKernelGGL(k, dim3((unsigned)persistent_grid(k, C::DQ_NW * 64, items)), dim3(C::DQ_NW * 64), 0, s, a);
    return launch_status();
  } else {
    if constexpr (FUSE_D) {  // float32 path: the pre-pass, then the dQ kernel
      const int st = run_delta<TIn, HD>(a, s);
      if (st) return st;
    }
    using C = TileCfg<TIn, HD>;
    constexpr int BR = C::DQ_NW * 16 * C::DQ_MR;
    const long grid = (long)((a.T + BR - 1) / BR) * a.B * a.H;
    hipLaunchKernelGGL((dq_kernel<TIn, HD, CAUSAL, PREC, C::DQ_NW, C::DQ_MR, C::DQ_BC>), dim3((unsigned)grid),
                       dim3(C::DQ_NW * 64), 0, s, a);
    return launch_status();
  }
}

template <typename TIn, int HD, bool CAUSAL, int PREC>
int run_dkv(const BwdArgs& a, hipStream_t s) {
  // 16-bit hd 128 runs the 16x16 kernel: 32 keys x 128 columns of dK and dV
  // per wave hold the 32x32 kernel to one wave per SIMD (502 VGPRs), and the
  // 16x16 one at two waves per SIMD is 12-13% faster at B4 H16 T8192.
  if constexpr (is_16bit<TIn> && HD == 64) {
    // hd 64: Q/dO blocks and the K/V tiles streamed through an LDS ring
    auto* k = &dkv64_kernel<TIn, CAUSAL, PREC>;
    const long items = (long)((a.T + 127) / 128) * a.B * a.H;
    hipLaunchKernelGGL(k, dim3((unsigned)persistent_grid(k, 256, items)), dim3(256), 0, s, a);
    return launch_status();
  } else {
    using C = TileCfg<TIn, HD>;
    constexpr int BK = C::DKV_NW * 16 * C::DKV_MR;
    const long grid = (long)((a.T + BK - 1) / BK) * a.B * a.H;
    hipLaunchKernelGGL((dkv_kernel<TIn, HD, CAUSAL, PREC, C::DKV_NW, C::DKV_MR, C::DKV_BQ>), dim3((unsigned)grid),
                       dim3(C::DKV_NW * 64), 0, s, a);
    return launch_status();
  }
}

// Split-key forward: partial results of nsplit key ranges into a workspace,
// then their merge into o and lse.
struct SplitArgs {
  FwdArgs f;  // f.o, f.lse point into the workspace
  float* o;
  float* lse;
  int nsplit;
};

template <typename TIn, int HD, bool CAUSAL, int PREC>
int run_fwd_split(const SplitArgs& sa, hipStream_t s) {
  FwdArgs a = sa.f;
  const size_t n = (size_t)a.B * a.T * a.H * HD, nr = (size_t)a.B * a.H * a.T;
  const int per = (a.T + sa.nsplit - 1) / sa.nsplit;
  a.o_split = n;
  a.lse_split = nr;
  a.nsplit = sa.nsplit;
  if constexpr (is_16bit<TIn>) {  // the 32x32 forward, (query tile, head, split) work items
    using C = TileCfg32<HD>;
    a.kchunk = (per + C::FWD_BC - 1) / C::FWD_BC * C::FWD_BC;
    if constexpr (!is_bf16<TIn>) a.one2 = 0x3C003C00u;
    auto* k = &fwd32_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_BC, C::FWD_MS, true>;
    constexpr int BR = C::FWD_NW * 32 * C::FWD_MS;
    const long items = (long)((a.T + BR - 1) / BR) * a.B * a.H * sa.nsplit;
    hipLaunchKernelGGL(k, dim3((unsigned)persistent_grid(k, C::FWD_NW * 64, items)), dim3(C::FWD_NW * 64), 0, s, a);
  } else {
    using C = TileCfg<TIn, HD>;
    constexpr int BR = C::FWD_NW * 16 * C::FWD_MR;
    a.kchunk = (per + C::FWD_BC - 1) / C::FWD_BC * C::FWD_BC;
    const long nqt = (a.T + BR - 1) / BR;
    hipLaunchKernelGGL((fwd_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_MR, C::FWD_BC>),
                       dim3((unsigned)(nqt * a.B * a.H), (unsigned)sa.nsplit), dim3(C::FWD_NW * 64), 0, s, a);
  }
  if (launch_status()) return kErrLaunch;
  MergeArgs m{a.o, a.lse, sa.o, sa.lse, a.B, a.H, a.T, sa.nsplit, n, nr};
  constexpr int RPB = 256 / (HD / 4);
  hipLaunchKernelGGL(merge_kernel<HD>, dim3((unsigned)((a.T + RPB - 1) / RPB), (unsigned)(a.B * a.H)), dim3(256), 0,
                     s, m);
  return launch_status();
}

// The plain forward's work items and the workgroups of its kernel the chip
// holds at once.
template <typename TIn, int HD, bool CAUSAL, int PREC>
void fwd_fill(const FwdArgs& a, long* items, long* slots) {
  const long bh = (long)a.B * a.H;
  if constexpr (is_16bit<TIn> && HD == 64) {
    *items = (long)((a.T + 127) / 128) * bh;
    *slots = (long)resident_per_cu(reinterpret_cast<const void*>(&fwd64_kernel<TIn, CAUSAL, PREC>), 128) * device_cus();
  } else if constexpr (is_16bit<TIn>) {
    using C = TileCfg32<HD>;
    constexpr int BR = C::FWD_NW * 32 * C::FWD_MS;
    *items = (long)((a.T + BR - 1) / BR) * bh;
    *slots = (long)resident_per_cu(
                 reinterpret_cast<const void*>(&fwd32_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_BC, C::FWD_MS>),
                 C::FWD_NW * 64) * device_cus();
  } else {
    using C = TileCfg<TIn, HD>;
    constexpr int BR = C::FWD_NW * 16 * C::FWD_MR;
    *items = (long)((a.T + BR - 1) / BR) * bh;
    *slots = (long)resident_per_cu(
                 reinterpret_cast<const void*>(&fwd_kernel<TIn, HD, CAUSAL, PREC, C::FWD_NW, C::FWD_MR, C::FWD_BC>),
                 C::FWD_NW * 64) * device_cus();
  }
}

// Key splits for a forward whose work items fill at most half of the resident
// workgroups (few batch-heads, long rows): enough splits to fill them, at
// most 64 and at least 128 keys per split; 1 otherwise.
inline int auto_splits(long items, long slots, int T) {
  if (items <= 0 || 2 * items > slots) return 1;
  long n = slots / items;
  if (n > 64) n = 64;
  if (n > T / 128) n = T / 128;
  return n >= 2 ? (int)n : 1;
}

// The library's workspace for stream s: one buffer per (device, stream),
// allocated on first use, grown when a call needs more (after waiting for the
// stream, so that no queued work still uses the old buffer) and kept until the
// process ends.  Calls on one stream run in order, so they can share it.
// Returns null (the caller then does without) if the stream is being captured
// and the buffer would have to grow, or if an allocation fails.
inline float* stream_workspace(hipStream_t s, size_t bytes) {
  int dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  struct Entry {
    int dev;
    hipStream_t s;
    float* p;
    size_t bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  Entry* e = nullptr;
  for (auto& x : cache)
    if (x.dev == dev && x.s == s) e = &x;
  if (e != nullptr && e->bytes >= bytes) return e->p;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  float* p = nullptr;
  bool ok = true;
  if (e != nullptr) ok = hipStreamSynchronize(s) == hipSuccess && hipFree(e->p) == hipSuccess;
  ok = ok && hipMalloc(reinterpret_cast<void**>(&p), bytes) == hipSuccess;
  (void)hipSetDevice(cur);
  if (!ok) {
    (void)hipGetLastError();
    if (e != nullptr) {
      e->p = nullptr;
      e->bytes = 0;
    }
    return nullptr;
  }
  if (e == nullptr) cache.push_back(Entry{dev, s, p, bytes});
  else {
    e->p = p;
    e->bytes = bytes;
  }
  return p;
}

// fa_forward: the plain forward, or the split-key forward with nsplit from
// auto_splits in the stream's workspace (the plain forward without one).
template <typename TIn, int HD, bool CAUSAL, int PREC>
int run_fwd_auto(const FwdArgs& a, hipStream_t s) {
  long items = 0, slots = 0;
  fwd_fill<TIn, HD, CAUSAL, PREC>(a, &items, &slots);
  const int nsplit = auto_splits(items, slots, a.T);
  if (nsplit < 2) return run_fwd<TIn, HD, CAUSAL, PREC>(a, s);
  const size_t n = (size_t)a.B * a.T * a.H * HD, nr = (size_t)a.B * a.H * a.T;
  float* ws = stream_workspace(s, (size_t)nsplit * (n + nr) * sizeof(float));
  if (ws == nullptr) return run_fwd<TIn, HD, CAUSAL, PREC>(a, s);
  FwdArgs f = a;
  f.o = ws;
  f.lse = ws + (size_t)nsplit * n;
  return run_fwd_split<TIn, HD, CAUSAL, PREC>(SplitArgs{f, a.o, a.lse, nsplit}, s);
}

enum Stage { kFwd = 0, kDq = 1, kDkv = 2, kDqDelta = 3, kFwdNoRescale = 4, kFwdSplit = 5, kFwdNoMax = 6, kFwdAuto = 7,
            kFwdSplits = 8 };

template <typename TIn, int HD, bool CAUSAL, int PREC>
int run_stage(int stage, const void* args, hipStream_t s) {
  switch (stage) {
    case kFwd: return run_fwd<TIn, HD, CAUSAL, PREC>(*static_cast<const FwdArgs*>(args), s);
    case kFwdNoRescale: return run_fwd<TIn, HD, CAUSAL, PREC, kCtlNoRescale>(*static_cast<const FwdArgs*>(args), s);
    case kFwdNoMax: return run_fwd<TIn, HD, CAUSAL, PREC, kCtlNoMax>(*static_cast<const FwdArgs*>(args), s);
    case kFwdSplit: return run_fwd_split<TIn, HD, CAUSAL, PREC>(*static_cast<const SplitArgs*>(args), s);
    case kFwdAuto: return run_fwd_auto<TIn, HD, CAUSAL, PREC>(*static_cast<const FwdArgs*>(args), s);
    case kFwdSplits: {  // the split count run_fwd_auto would use (no launch)
      long items = 0, slots = 0;
      fwd_fill<TIn, HD, CAUSAL, PREC>(*static_cast<const FwdArgs*>(args), &items, &slots);
      return auto_splits(items, slots, static_cast<const FwdArgs*>(args)->T);
    }
    case kDq: return run_dq<TIn, HD, CAUSAL, PREC>(*static_cast<const BwdArgs*>(args), s);
    case kDqDelta: return run_dq<TIn, HD, CAUSAL, PREC, true>(*static_cast<const BwdArgs*>(args), s);
    default: return run_dkv<TIn, HD, CAUSAL, PREC>(*static_cast<const BwdArgs*>(args), s);
  }
}

template <typename TIn, int HD>
int run_stage_hd(int stage, const void* args, bool causal, int prec, hipStream_t s) {
  if constexpr (is_bf16<TIn>) {  // the split operand exists for bfloat16 only
    if (prec == 1)
      return causal ? run_stage<TIn, HD, true, 1>(stage, args, s) : run_stage<TIn, HD, false, 1>(stage, args, s);
  }
  return causal ? run_stage<TIn, HD, true, 0>(stage, args, s) : run_stage<TIn, HD, false, 0>(stage, args, s);
}

// Entry points of the per-dtype translation units.  prec: 0 single bf16
// operand, 1 split operand.  Return 0, -3 (head dim not built) or -5.
int stage_f32(int stage, int hd, const void* args, bool causal, hipStream_t s);
int stage_bf16(int stage, int hd, const void* args, bool causal, int prec, hipStream_t s);
int stage_f16(int stage, int hd, const void* args, bool causal, int prec, hipStream_t s);
int delta_f16(int hd, const BwdArgs& a, hipStream_t s);
int delta_f32(int hd, const BwdArgs& a, hipStream_t s);
int unfused_f32(int hd, const UnfusedArgs& a, bool causal, hipStream_t s);
int delta_bf16(int hd, const BwdArgs& a, hipStream_t s);

}  // namespace fa
