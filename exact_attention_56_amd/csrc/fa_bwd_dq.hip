// fa_bwd_dq.hip - instantiates the dQ pass of the backward (headdim 64 and 128, bf16
// and fp16).  A translation unit of its own so that it can keep its accumulators in
// arch VGPRs (two waves per SIMD) while the dK/dV pass uses the accumulation registers.
#include "fa_bwd_kernel.h"

namespace fa {
hipError_t launch_dq_d64(const BwdParams& p, hipStream_t stream) {
  return p.f16 ? launch_dq_hd<64, _Float16>(p, stream) : launch_dq_hd<64, __bf16>(p, stream);
}
hipError_t launch_dq_d128(const BwdParams& p, hipStream_t stream) {
  return p.f16 ? launch_dq_hd<128, _Float16>(p, stream) : launch_dq_hd<128, __bf16>(p, stream);
}
}  // namespace fa
