// fa_fwd_d64.hip - instantiates the forward kernels for headdim 64.
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_d64(const FwdParams& p, bool split, hipStream_t stream) {
  return launch_fwd_hd<64>(p, split, stream);
}
hipError_t launch_fwd_decode_d64(const FwdParams& p, hipStream_t stream) {
  return launch_fwd_decode_hd<64>(p, stream);
}
}  // namespace fa
