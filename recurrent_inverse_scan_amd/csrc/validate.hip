// Opt-in NaN/Inf pre-check of the scan inputs.  Source: "Mathematical
// Primitives", section 1 (finite-state enforcement before evaluation).
// Also the last step of the chunked schedule's statistics.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_seq.h"

namespace vla {

namespace {

__global__ void clear_flag_kernel(int32_t* flag) { *flag = 0; }

template <typename T>
__global__ void __launch_bounds__(256) nonfinite_kernel(const T* __restrict__ p, int64_t n, int32_t* flag) {
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    bad |= !isfinite(Elem<T>::load(p + i));
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
}

// stats[c][2] |= the non-finite flag that the chunked schedule's passes left
// in chain_info[c].
__global__ void __launch_bounds__(256) stats_finalize_kernel(int32_t* __restrict__ stats,
                                                             const int32_t* __restrict__ chain_info, int chains) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < chains && chain_info[c * 4 + kInfoNonfinite]) stats[c * 4 + 2] = 1;
}

}  // namespace

hipError_t launch_stats_finalize(int32_t* stats, const int32_t* chain_info, int chains, hipStream_t stream) {
  if (!stats || chains <= 0) return hipSuccess;
  hipLaunchKernelGGL(stats_finalize_kernel, dim3((chains + 255) / 256), dim3(256), 0, stream, stats, chain_info,
                     chains);
  return hipGetLastError();
}

hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, stream, flag);
  return hipGetLastError();
}

hipError_t launch_nonfinite_check(const void* p, int64_t n, bool bf16, int32_t* flag, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 4096 ? want : 4096);
  if (bf16)
    hipLaunchKernelGGL(nonfinite_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p), n, flag);
  else
    hipLaunchKernelGGL(nonfinite_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const float*>(p), n, flag);
  return hipGetLastError();
}

}  // namespace vla
