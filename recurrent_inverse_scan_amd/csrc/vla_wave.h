// Wave-wide sum by DPP alone, for the sequential kernels.
#pragma once

#include "vla_common.h"

namespace vla {

// Row sums, then the gfx9 row broadcasts (lane 15 of rows 0 and 2 into rows 1
// and 3, then lane 31 into rows 2 and 3), so lane 63 holds the total; one
// readlane makes it wave-uniform.  The order of the additions is fixed, so
// every wave that reduces the same values gets the same bits.
__device__ __forceinline__ float wave_total(float x) {
  x = group_sum<16>(x);
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast15, 0xA, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast31, 0xC, 0xF, false));
  return readlane_f(x, 63);
}

}  // namespace vla
