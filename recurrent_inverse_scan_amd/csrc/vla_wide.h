// Launch interface of the d = 128 blocked inverse pass (inverse_wy128.hip).
#pragma once
#include "vla_kernels.h"

namespace vla {

// Chunk-start inverses at d = 128 of chunks (c_lo + i) c_step, i = 0 ..
// c_cnt - 1, of every chain (the starts of the inverse pass's spans).
hipError_t launch_chunk_start128(const ChunkPlan& pl, int c_lo, int c_cnt, int c_step, hipStream_t stream);

// The inverse pass in blocked Woodbury form on the matrix cores: d = 128,
// bf16 storage, additive update, r = 1..4.  One workgroup per span of cm
// consecutive chunks (spans [inv_lo, inv_lo + inv_cnt) of every chain, span j
// starting at chunk j cm, whose start inverse a_start must hold); writes
// alpha_hat and, from each chain's last span, A_T.  A guard fire flags the
// chain for the sequential fallback.
hipError_t launch_inverse_wy128(const ScanArgs& a, const float* a_start, float* alpha_out, int32_t* chain_info,
                                int chunk_len, int nchunks, int cm, int inv_lo, int inv_cnt, int chains,
                                hipStream_t stream);

}  // namespace vla
