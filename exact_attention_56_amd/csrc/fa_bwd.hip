// fa_bwd.hip - instantiates the dK/dV pass of the backward (headdim 64, 128 and 256,
// bf16 and fp16; the dQ pass too at 256) and launches the two passes in order on one
// stream: dQ (which also writes D), then dK/dV (padded or packed batches, grouped K/V
// heads).
#include "fa_bwd_kernel.h"

namespace fa {

template <int HD, typename E>
static hipError_t launch_bwd_hd(const BwdParams& p, hipStream_t stream) {
  // dQ first: besides dQ it writes D = rowsum(dO o O) of every query row, which the
  // dK/dV pass reads, so dK/dV must not start before it (one stream: it does not)
  hipError_t e;
  if constexpr (HD == 256)
    e = launch_dq_hd<256, E>(p, stream);  // accumulators in AGPRs: compiled here
  else
    e = HD == 64 ? launch_dq_d64(p, stream) : launch_dq_d128(p, stream);
  if (e != hipSuccess) return e;
  const bool alibi = p.alibi != nullptr;
  const int kv_items = p.batch * p.nheads_k * p.num_k_tiles;
  if (alibi)
    hipLaunchKernelGGL((dkdv_kernel<HD, true, E>), dim3(kv_items), dim3(256), 0, stream, p, kv_items);
  else
    hipLaunchKernelGGL((dkdv_kernel<HD, false, E>), dim3(kv_items), dim3(256), 0, stream, p, kv_items);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_bwd_e(const BwdParams& p, int headdim, hipStream_t stream) {
  switch (headdim) {
    case 64: return launch_bwd_hd<64, E>(p, stream);
    case 128: return launch_bwd_hd<128, E>(p, stream);
    case 256: return launch_bwd_hd<256, E>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdParams& p, int headdim, hipStream_t stream) {
  return p.f16 ? launch_bwd_e<_Float16>(p, headdim, stream) : launch_bwd_e<__bf16>(p, headdim, stream);
}

}  // namespace fa
