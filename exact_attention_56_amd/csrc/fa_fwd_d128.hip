// fa_fwd_d128.hip - instantiates the forward kernels for headdim 128.
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_d128(const FwdParams& p, bool split, hipStream_t stream) {
  return launch_fwd_hd<128>(p, split, stream);
}
hipError_t launch_fwd_decode_d128(const FwdParams& p, hipStream_t stream) {
  return launch_fwd_decode_hd<128>(p, stream);
}
}  // namespace fa
