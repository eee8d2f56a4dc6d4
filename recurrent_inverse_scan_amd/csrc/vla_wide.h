// Launch interface of the d = 128 blocked inverse pass (inverse_wy128.hip).
#pragma once
#include "vla_kernels.h"

namespace vla {

// The inverse pass of chunks [chunk_lo, chunk_lo + chunk_cnt) in blocked
// Woodbury form on the matrix cores: d = 128, bf16 storage, additive update,
// r = 1..4; writes alpha_hat and, from each chain's last chunk, A_T.  A guard
// fire flags the chain for the sequential fallback.
hipError_t launch_inverse_wy128(const ScanArgs& a, const float* a_start, float* alpha_out, int32_t* chain_info,
                                int chunk_len, int nchunks, int chunk_lo, int chunk_cnt, int chains,
                                hipStream_t stream);

}  // namespace vla
