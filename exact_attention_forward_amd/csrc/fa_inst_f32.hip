// float32 instantiations: head dims 8, 16, 32, 64, 128.
#include "fa_launch.hpp"

namespace fa {

int stage_f32(int stage, int hd, const void* args, bool causal, hipStream_t s) {
  switch (hd) {
    case 8: return run_stage_hd<float, 8>(stage, args, causal, 0, s);
    case 16: return run_stage_hd<float, 16>(stage, args, causal, 0, s);
    case 32: return run_stage_hd<float, 32>(stage, args, causal, 0, s);
    case 64: return run_stage_hd<float, 64>(stage, args, causal, 0, s);
    case 128: return run_stage_hd<float, 128>(stage, args, causal, 0, s);
    default: return kErrUnsupported;
  }
}

int delta_f32(int hd, const BwdArgs& a, hipStream_t s) {
  switch (hd) {
    case 8: return run_delta<float, 8>(a, s);
    case 16: return run_delta<float, 16>(a, s);
    case 32: return run_delta<float, 32>(a, s);
    case 64: return run_delta<float, 64>(a, s);
    case 128: return run_delta<float, 128>(a, s);
    default: return kErrUnsupported;
  }
}

int unfused_f32(int hd, const UnfusedArgs& a, bool causal, hipStream_t s) {
  switch (hd) {
    case 8: return run_unfused<8>(a, causal, s);
    case 16: return run_unfused<16>(a, causal, s);
    case 32: return run_unfused<32>(a, causal, s);
    case 64: return run_unfused<64>(a, causal, s);
    case 128: return run_unfused<128>(a, causal, s);
    default: return kErrUnsupported;
  }
}

}  // namespace fa
