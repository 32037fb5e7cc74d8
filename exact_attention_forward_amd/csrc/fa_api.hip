// C ABI of the attention library: argument validation and dispatch.
// Declarations and the contract of every entry point are in include/fa.h.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.hpp"

static_assert(fa::kErrUnsupported == FA_ERR_UNSUPPORTED && fa::kErrLaunch == FA_ERR_LAUNCH,
              "launcher status codes must match the C ABI");

namespace {

struct Buf {
  const void* p;
  size_t bytes;
};

bool overlap(const Buf& a, const Buf& b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs must not overlap inputs or each other.
int check_alias(const Buf* in, int nin, const Buf* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(out[i], in[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptrs(const void* const* ps, int n) {
  for (int i = 0; i < n; ++i)
    if (ps[i] == nullptr) return FA_ERR_ARG;
  for (int i = 0; i < n; ++i)
    if (!aligned16(ps[i])) return FA_ERR_ALIGN;
  return FA_OK;
}

int supported(int hd, int dtype) {
  if (dtype == FA_F32) return hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128;
  if (dtype == FA_BF16 || dtype == FA_F16) return hd == 64 || hd == 128;
  return 0;
}

// Shape, dtype and precision checks shared by every entry point.
int check_common(int B, int H, int T, int hd, int dtype, int prec) {
  if (B < 1 || H < 1 || T < 1 || hd < 1) return FA_ERR_ARG;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_ARG;
  if (prec != FA_PREC_DEFAULT && prec != FA_PREC_BF16 && prec != FA_PREC_BF16X2) return FA_ERR_ARG;
  const double elems = (double)B * H * T * hd;
  if (elems >= 1099511627776.0) return FA_ERR_ARG;  // 2^40
  if ((double)B * H * T >= 2147483647.0) return FA_ERR_ARG;
  // the 32x32 forward keeps each thread's offsets within a 32-row key block
  // as 32-bit byte offsets: 32 rows of H * hd 16-bit elements must stay
  // under 4 GiB
  if ((double)H * hd >= 33554432.0) return FA_ERR_ARG;  // 2^25
  if (!supported(hd, dtype)) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && prec != FA_PREC_DEFAULT) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_scale(float scale, int causal) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  return FA_OK;
}

int prec_index(int prec) { return prec == FA_PREC_BF16X2 ? 1 : 0; }

int run(int stage, int hd, int dtype, int prec, bool causal, const void* args, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_F32) return fa::stage_f32(stage, hd, args, causal, s);
  if (dtype == FA_F16) return fa::stage_f16(stage, hd, args, causal, 0, s);
  return fa::stage_bf16(stage, hd, args, causal, prec_index(prec), s);
}

float log2e_scaled(float scale) { return (float)((double)scale * 1.4426950408889634); }

// Rows of D that fa_backward_nows keeps in the library's static device array.
constexpr size_t kScratchRows = size_t(1) << 22;

}  // namespace

// The D workspace of fa_backward_nows: one copy per device (each GPU the
// library runs on holds its own), for the life of the process.  In host code
// this name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, per device (scratch_on).
static __device__ __align__(256) float scratch[kScratchRows];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_addr[kMaxDevices];  // device address of `scratch`, per device id

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current.  nullptr if the runtime cannot provide it.
float* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    scratch_addr[dev] = static_cast<float*>(p);
  }
  return scratch_addr[dev];
}

// The device a stream launches on: the stream's own device, or the current
// device for the null stream.
int stream_device(void* stream, int* dev) {
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &d) != hipSuccess) return FA_ERR_LAUNCH;
    *dev = d;
    return FA_OK;
  }
  return hipGetDevice(dev) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_is_supported(int hd, fa_dtype dtype) { return supported(hd, dtype); }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_ARG: return "invalid argument";
    case FA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype or precision";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_TOO_LARGE: return "problem larger than the library's static workspace";
    default: return "unknown status";
  }
}

int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T, int hd,
               float scale, int causal, fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, o, lse};
  if ((st = check_ptrs(ptrs, 5))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}};
  const Buf out[] = {{o, n * 4}, {lse, (size_t)B * H * T * 4}};
  if ((st = check_alias(in, 3, out, 2))) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, T, log2e_scaled(scale)};
  return run(fa::kFwdAuto, hd, dtype, prec, causal != 0, &a, stream);
}

int fa_forward_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, float* ws, int B, int H,
                       int T, int hd, float scale, int causal, int nsplit, fa_dtype dtype, fa_precision prec,
                       void* stream) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  if (nsplit < 1 || nsplit > 64) return FA_ERR_ARG;
  if ((double)B * H > 65535.0) return FA_ERR_ARG;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T;
  if (nsplit == 1 && ws == nullptr) {
    // one range and no workspace: the plain forward, never split
    const void* ptrs[] = {q, k, v, o, lse};
    if ((st = check_ptrs(ptrs, 5))) return st;
    const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}};
    const Buf out[] = {{o, n * 4}, {lse, nr * 4}};
    if ((st = check_alias(in, 3, out, 2))) return st;
    fa::FwdArgs a{q, k, v, o, lse, B, H, T, log2e_scaled(scale)};
    return run(fa::kFwd, hd, dtype, prec, causal != 0, &a, stream);
  }
  const void* ptrs[] = {q, k, v, o, lse, ws};
  if ((st = check_ptrs(ptrs, 6))) return st;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}};
  const Buf out[] = {{o, n * 4}, {lse, nr * 4}, {ws, (size_t)nsplit * (n + nr) * 4}};
  if ((st = check_alias(in, 3, out, 3))) return st;
  fa::SplitArgs a{{q, k, v, ws, ws + (size_t)nsplit * n, B, H, T, log2e_scaled(scale)}, o, lse, nsplit};
  return run(fa::kFwdSplit, hd, dtype, prec, causal != 0, &a, stream);
}

int fa_forward_auto_splits(int B, int H, int T, int hd, int causal, fa_dtype dtype, fa_precision prec) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  fa::FwdArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, B, H, T, 0.f};
  return run(fa::kFwdSplits, hd, dtype, prec, causal != 0, &a, nullptr);
}

static int control_forward(int stage, const void* q, const void* k, const void* v, float* o, float* lse, int B,
                           int H, int T, int hd, float scale, int causal, fa_dtype dtype, void* stream) {
  int st = check_common(B, H, T, hd, dtype, FA_PREC_DEFAULT);
  if (st) return st;
  if (dtype == FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, o, lse};
  if ((st = check_ptrs(ptrs, 5))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}};
  const Buf out[] = {{o, n * 4}, {lse, (size_t)B * H * T * 4}};
  if ((st = check_alias(in, 3, out, 2))) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, T, log2e_scaled(scale)};
  return run(stage, hd, dtype, FA_PREC_DEFAULT, causal != 0, &a, stream);
}

int fa_forward_norescale(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T,
                         int hd, float scale, int causal, fa_dtype dtype, void* stream) {
  return control_forward(fa::kFwdNoRescale, q, k, v, o, lse, B, H, T, hd, scale, causal, dtype, stream);
}

int fa_forward_nomax(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int T, int hd,
                     float scale, int causal, fa_dtype dtype, void* stream) {
  return control_forward(fa::kFwdNoMax, q, k, v, o, lse, B, H, T, hd, scale, causal, dtype, stream);
}

int fa_forward_unfused(const void* q, const void* k, const void* v, float* o, float* scores, int B, int H, int T,
                       int hd, float scale, int causal, fa_dtype dtype, void* stream) {
  int st = check_common(B, H, T, hd, dtype, FA_PREC_DEFAULT);
  if (st) return st;
  if (dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((st = check_scale(scale, causal))) return st;
  if ((double)B * H > 65535.0 || (double)B * H * T * T >= 1099511627776.0) return FA_ERR_ARG;
  const void* ptrs[] = {q, k, v, o, scores};
  if ((st = check_ptrs(ptrs, 5))) return st;
  const size_t n = (size_t)B * T * H * hd;
  const Buf in[] = {{q, n * 4}, {k, n * 4}, {v, n * 4}};
  const Buf out[] = {{o, n * 4}, {scores, (size_t)B * H * T * T * 4}};
  if ((st = check_alias(in, 3, out, 2))) return st;
  fa::UnfusedArgs a{static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), o,
                    scores, B, H, T, scale};
  return fa::unfused_f32(hd, a, causal != 0, static_cast<hipStream_t>(stream));
}

int fa_backward_delta(const float* o, const void* dO, float* delta, int B, int H, int T, int hd, fa_dtype dtype,
                      void* stream) {
  int st = check_common(B, H, T, hd, dtype, FA_PREC_DEFAULT);
  if (st) return st;
  const void* ptrs[] = {o, dO, delta};
  if ((st = check_ptrs(ptrs, 3))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2;
  const Buf in[] = {{o, n * 4}, {dO, n * es}};
  const Buf out[] = {{delta, (size_t)B * H * T * 4}};
  if ((st = check_alias(in, 2, out, 1))) return st;
  fa::BwdArgs a{};
  a.o = o;
  a.dO = dO;
  a.delta = delta;
  a.B = B, a.H = H, a.T = T;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_F32) return fa::delta_f32(hd, a, s);
  return dtype == FA_F16 ? fa::delta_f16(hd, a, s) : fa::delta_bf16(hd, a, s);
}

static int check_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                    const float* delta, float* dq, int B, int H, int T, int hd, float scale, int causal,
                    fa_dtype dtype, fa_precision prec) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, lse, dO, delta, dq};
  if ((st = check_ptrs(ptrs, 7))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T * 4;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}, {lse, nr}, {dO, n * es}, {delta, nr}};
  const Buf out[] = {{dq, n * 4}};
  return check_alias(in, 6, out, 1);
}

static int check_dkv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                     const float* delta, float* dk, float* dv, int B, int H, int T, int hd, float scale,
                     int causal, fa_dtype dtype, fa_precision prec) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, lse, dO, delta, dk, dv};
  if ((st = check_ptrs(ptrs, 8))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T * 4;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}, {lse, nr}, {dO, n * es}, {delta, nr}};
  const Buf out[] = {{dk, n * 4}, {dv, n * 4}};
  return check_alias(in, 6, out, 2);
}

static fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const float* o, const float* lse,
                            const void* dO, float* dq, float* dk, float* dv, float* delta, int B, int H, int T,
                            float scale) {
  fa::BwdArgs a{q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, scale, log2e_scaled(scale)};
  return a;
}

int fa_backward_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                   const float* delta, float* dq, int B, int H, int T, int hd, float scale, int causal,
                   fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_dq(q, k, v, lse, dO, delta, dq, B, H, T, hd, scale, causal, dtype, prec);
  if (st) return st;
  fa::BwdArgs a = bwd_args(q, k, v, nullptr, lse, dO, dq, nullptr, nullptr, const_cast<float*>(delta), B, H, T, scale);
  return run(fa::kDq, hd, dtype, prec, causal != 0, &a, stream);
}

int fa_backward_dkv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                    const float* delta, float* dk, float* dv, int B, int H, int T, int hd, float scale,
                    int causal, fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_dkv(q, k, v, lse, dO, delta, dk, dv, B, H, T, hd, scale, causal, dtype, prec);
  if (st) return st;
  fa::BwdArgs a = bwd_args(q, k, v, nullptr, lse, dO, nullptr, dk, dv, const_cast<float*>(delta), B, H, T, scale);
  return run(fa::kDkv, hd, dtype, prec, causal != 0, &a, stream);
}

int fa_backward_dq_delta(const void* q, const void* k, const void* v, const float* o, const float* lse,
                         const void* dO, float* dq, float* delta, int B, int H, int T, int hd, float scale,
                         int causal, fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, delta};
  if ((st = check_ptrs(ptrs, 8))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T * 4;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}, {o, n * 4}, {lse, nr}, {dO, n * es}};
  const Buf out[] = {{dq, n * 4}, {delta, nr}};
  if ((st = check_alias(in, 6, out, 2))) return st;
  fa::BwdArgs a = bwd_args(q, k, v, o, lse, dO, dq, nullptr, nullptr, delta, B, H, T, scale);
  return run(fa::kDqDelta, hd, dtype, prec, causal != 0, &a, stream);
}

int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dO,
                float* dq, float* dk, float* dv, float* delta, int B, int H, int T, int hd, float scale, int causal,
                fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv, delta};
  if ((st = check_ptrs(ptrs, 10))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T * 4;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}, {o, n * 4}, {lse, nr}, {dO, n * es}};
  const Buf out[] = {{dq, n * 4}, {dk, n * 4}, {dv, n * 4}, {delta, nr}};
  if ((st = check_alias(in, 6, out, 4))) return st;
  if ((st = fa_backward_dq_delta(q, k, v, o, lse, dO, dq, delta, B, H, T, hd, scale, causal, dtype, prec, stream)))
    return st;
  return fa_backward_dkv(q, k, v, lse, dO, delta, dk, dv, B, H, T, hd, scale, causal, dtype, prec, stream);
}

int fa_backward_nows(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dO,
                     float* dq, float* dk, float* dv, int B, int H, int T, int hd, float scale, int causal,
                     fa_dtype dtype, fa_precision prec, void* stream) {
  int st = check_common(B, H, T, hd, dtype, prec);
  if (st) return st;
  if ((st = check_scale(scale, causal))) return st;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv};
  if ((st = check_ptrs(ptrs, 9))) return st;
  const size_t n = (size_t)B * T * H * hd, es = dtype == FA_F32 ? 4 : 2, nr = (size_t)B * H * T * 4;
  const Buf in[] = {{q, n * es}, {k, n * es}, {v, n * es}, {o, n * 4}, {lse, nr}, {dO, n * es}};
  const Buf out[] = {{dq, n * 4}, {dk, n * 4}, {dv, n * 4}};
  if ((st = check_alias(in, 6, out, 3))) return st;
  if ((size_t)B * H * T > kScratchRows) return FA_ERR_TOO_LARGE;
  int dev = -1;
  if ((st = stream_device(stream, &dev))) return st;
  float* delta = scratch_on(dev);
  if (delta == nullptr) return FA_ERR_LAUNCH;
  // D needs no clearing: the dQ stage writes every row of it before the
  // dK/dV stage reads it.
  return fa_backward(q, k, v, o, lse, dO, dq, dk, dv, delta, B, H, T, hd, scale, causal, dtype, prec, stream);
}

}  // extern "C"
