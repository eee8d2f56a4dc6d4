// Opt-in NaN/Inf pre-check of the scan inputs.  Source: "Mathematical
// Primitives", section 1 (finite-state enforcement before evaluation).
#include "vla_common.h"
#include "vla_kernels.h"

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

}  // namespace

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
