// fa_fwd_d256.hip - instantiates the forward kernels for headdim 256.
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_d256(const FwdParams& p, bool split, hipStream_t stream) {
  return launch_fwd_hd<256>(p, split, stream);
}
}  // namespace fa
