// Input pre-passes: the opt-in NaN/Inf pre-check of the scan inputs (source:
// "Mathematical Primitives", section 1, finite-state enforcement before
// evaluation) and the gather of strided q, k, v into contiguous rows.  Also
// the last step of the chunked schedule's statistics.
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

// q, k, v (blockIdx.y = 0, 1, 2) from strided [B, H, T, d] views into
// contiguous [B, H, T, d] rows at dst (three tensors back to back), one
// 16-byte piece per thread and step.  Strides are in elements and keep every
// row 16-byte aligned (checked on the host).
__global__ void __launch_bounds__(256) gather_rows_kernel(GatherArgs g) {
  const char* src = blockIdx.y == 0 ? g.q : (blockIdx.y == 1 ? g.k : g.v);
  uint4* dst = reinterpret_cast<uint4*>(g.dst + static_cast<int64_t>(blockIdx.y) * g.rows * g.row_bytes);
  const int vpr = g.row_bytes / 16;
  const int64_t nvec = g.rows * vpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < nvec;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t row = i / vpr;
    const int piece = static_cast<int>(i - row * vpr);
    const int64_t t = row % g.T, chain = row / g.T;
    const int64_t b = chain / g.H, h = chain - b * g.H;
    const int64_t off = (b * g.stride_b + h * g.stride_h + t * g.stride_t) * g.elem_bytes + 16 * piece;
    dst[i] = *reinterpret_cast<const uint4*>(src + off);
  }
}

// Feature map ELU(x) + 1 (ELU with alpha = 1) of q_raw and k_raw
// (blockIdx.y = 0, 1) into q and k, in the storage dtype (round to nearest
// even for bfloat16): "Variational Linear Attention (VLA)" README, v3 notes
// item 1.
template <typename T>
__global__ void __launch_bounds__(256) feature_map_kernel(const T* __restrict__ q_raw, const T* __restrict__ k_raw,
                                                          T* __restrict__ q, T* __restrict__ k, int64_t n) {
  const T* src = blockIdx.y == 0 ? q_raw : k_raw;
  T* dst = blockIdx.y == 0 ? q : k;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const float x = Elem<T>::load(src + i);
    Elem<T>::store(dst + i, (x > 0.f ? x : expm1f(x)) + 1.f);
  }
}

}  // namespace

hipError_t launch_feature_map(const void* q_raw, const void* k_raw, void* q, void* k, int64_t n, bool bf16,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  if (bf16)
    hipLaunchKernelGGL(feature_map_kernel<uint16_t>, dim3(grid, 2), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q_raw), static_cast<const uint16_t*>(k_raw),
                       static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), n);
  else
    hipLaunchKernelGGL(feature_map_kernel<float>, dim3(grid, 2), dim3(256), 0, stream,
                       static_cast<const float*>(q_raw), static_cast<const float*>(k_raw), static_cast<float*>(q),
                       static_cast<float*>(k), n);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const GatherArgs& g, hipStream_t stream) {
  const int64_t nvec = g.rows * (g.row_bytes / 16);
  if (nvec <= 0) return hipSuccess;
  const int64_t want = (nvec + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid, 3), dim3(256), 0, stream, g);
  return hipGetLastError();
}

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
