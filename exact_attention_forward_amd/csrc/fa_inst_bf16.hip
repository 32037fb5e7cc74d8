// bfloat16 instantiations: head dims 64 and 128, single and split operands.
#include "fa_launch.hpp"

namespace fa {

int stage_bf16(int stage, int hd, const void* args, bool causal, int prec, hipStream_t s) {
  switch (hd) {
    case 64: return run_stage_hd<bf16_t, 64>(stage, args, causal, prec, s);
    case 128: return run_stage_hd<bf16_t, 128>(stage, args, causal, prec, s);
    default: return kErrUnsupported;
  }
}

int delta_bf16(int hd, const BwdArgs& a, hipStream_t s) {
  switch (hd) {
    case 64: return run_delta<bf16_t, 64>(a, s);
    case 128: return run_delta<bf16_t, 128>(a, s);
    default: return kErrUnsupported;
  }
}

}  // namespace fa
