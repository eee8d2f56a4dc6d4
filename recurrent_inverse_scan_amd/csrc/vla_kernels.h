// Internal kernel-launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

// Everything a scan kernel needs; pointers are device pointers.
struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* u;
  const float* A0;   // nullable: identity
  const float* S0;   // nullable: zero
  const float* n0;   // nullable: zero
  void* o;
  float* A_T;
  float* S_T;
  float* n_T;
  int32_t* stats;    // nullable
  int32_t T;
  int32_t r;
  float eps;
  int32_t nudge_period;   // 0 = off
  int32_t nudge_phase0;   // (t0 + 1) mod nudge_period: 0 means token 0 is nudged
  float cap;
  int32_t cap_on;
  float den_eps;
};

hipError_t launch_scan_sequential(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream);

hipError_t launch_project_u(int64_t rows, int d, int r, bool in_bf16, bool out_bf16, const void* W,
                            const void* kraw, void* u, hipStream_t stream);

// Sets *flag (device int) to 1 if any of the n elements at the given buffers
// is NaN or Inf; *flag must be cleared first with launch_clear_flag.
hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream);
hipError_t launch_nonfinite_check(const void* p, int64_t n, bool bf16, int32_t* flag, hipStream_t stream);

}  // namespace vla
