// fa_bwd.hip - instantiates the delta and dK/dV passes of the backward (headdim 64,
// 128 and 256, bf16 and fp16; the dQ pass too at 256) and launches the three passes in
// order on one stream:
// delta, dK/dV, dQ (padded or packed batches, grouped K/V heads).
#include "fa_bwd_kernel.h"

namespace fa {

template <int HD, typename E>
static hipError_t launch_bwd_hd(const BwdParams& p, hipStream_t stream) {
  // delta runs over rows of [rows, H, D]; a packed batch is one sequence of total_q rows
  // for it (its [H, total_q] output is then the [1, H, total_q] layout)
  BwdParams pd = p;
  if (p.cu_q != nullptr) {
    pd.batch = 1;
    pd.seqlen_q = (int)p.lse_head_stride;
  }
  const long rows = (long)pd.batch * pd.seqlen_q * pd.nheads;
  const int rows_per_block = delta_rows_per_block(HD);
  hipLaunchKernelGGL((delta_kernel<HD, E>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(256),
                     0, stream, pd, rows);
  // dK/dV must not run on a delta that was never written
  const hipError_t ed = hipGetLastError();
  if (ed != hipSuccess) return ed;
  const bool alibi = p.alibi != nullptr;
  const int kv_items = p.batch * p.nheads_k * p.num_k_tiles;
  if (alibi)
    hipLaunchKernelGGL((dkdv_kernel<HD, true, E>), dim3(kv_items), dim3(256), 0, stream, p, kv_items);
  else
    hipLaunchKernelGGL((dkdv_kernel<HD, false, E>), dim3(kv_items), dim3(256), 0, stream, p, kv_items);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (HD == 256) return launch_dq_hd<256, E>(p, stream);  // accumulators in AGPRs: compiled here
  return HD == 64 ? launch_dq_d64(p, stream) : launch_dq_d128(p, stream);
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
