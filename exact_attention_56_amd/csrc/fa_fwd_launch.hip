// fa_fwd_launch.hip - headdim dispatch of the matrix-core forward kernels.
#include "fa_fwd_kernel.h"

namespace fa {

// Host-side launcher used by the C ABI layer.  Arguments are already validated.
hipError_t launch_fwd(const FwdParams& p, int headdim, bool split, hipStream_t stream) {
  switch (headdim) {
    case 64: return launch_fwd_d64(p, split, stream);
    case 128: return launch_fwd_d128(p, split, stream);
    case 256: return launch_fwd_d256(p, split, stream);
    default: return hipErrorInvalidValue;
  }
}

long fwd_num_blocks(const FwdParams& p, bool split) {
  return (long)p.batch * p.nheads * p.num_q_tiles * (split ? p.num_splits : 1);
}

}  // namespace fa
