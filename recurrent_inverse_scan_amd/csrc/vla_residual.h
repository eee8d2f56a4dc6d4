// Internal launch interface of the residual update's time-parallel state
// pass (residual_pass.hip), between the C ABI layer and its kernels.
#pragma once
#include "vla_kernels.h"

namespace vla {

// Time-parallel state pass of the residual update (d = 64, blocks of 64
// tokens); buffers in the workspace, see residual_pass.hip.
struct ResPlan {
  int T, nblk;
  int bf16;              // storage of q, k, v, o
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* alpha;    // [chains][T][64] unit gates from the inverse pass
  float* W;              // [chains][nblk][64][64] (I + L)^{-1} K_hat
  float* U;              // [chains][nblk][64][64] (I + L)^{-1} V
  uint16_t* NTF;         // [chains][nblk][2][2][2][3][64][8] N^T as split bf16 matrix-core operands
  float* QT;             // [chains][nblk][4 tiles][4][64 lanes][4] Q^T in accumulator order
  float* ksum;           // [chains][nblk][64] sum of the block's keys
  float* Ssnap;          // [chains][nblk][64][64] S at each block start
  float* nblock;         // [chains][nblk][64] normaliser at each block start
  int32_t* exact;        // [chains][nblk] the block needs the per-token cap test
};
// Block ranges [b_lo, b_lo + nb) of every chain; at most max_wg workgroups
// if max_wg > 0 (grid-stride).
hipError_t launch_res_prep(const ResPlan& pl, int chains, int b_lo, int nb, int max_wg, hipStream_t stream);
// Block-start normalisers of blocks [b_lo, b_hi) from n at b_lo (n_in,
// [chains][64]); n at b_hi goes to n_out (which must not alias n_in).
hipError_t launch_res_nprefix(const ResPlan& pl, int b_lo, int b_hi, const float* n_in, float* n_out, int chains,
                              hipStream_t stream);
// The chain kernel over blocks [b_lo, b_hi) from S_in (chain c at
// S_in + c * S_in_stride).  The last segment writes S_T and stats (guard count
// and non-finite flag from chain_info; no cap fires: a token over the cap
// makes the readout flag the chain for the fallback); the others leave S at
// b_hi in that block's snapshot.
hipError_t launch_res_chain(const ResPlan& pl, int b_lo, int b_hi, const float* S_in, int64_t S_in_stride,
                            float* S_T, int32_t* stats, const int32_t* chain_info, int last, int chains,
                            hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);
// Where the sequential fallback restarts a chain (see vla_res_restart_kernel).
struct ResRestart {
  int chunk_len, nchunks;
  const float* Ac;       // [chains][nchunks][64][64] chunk-start inverses
  float* A_init;         // [chains][64][64], overwritten for restarted chains
  float* S_init;
  float* n_init;         // [chains][64]
  int32_t* chain_info;   // [chains][4]
};
hipError_t launch_res_restart(const ResPlan& pl, const ResRestart& rs, int chains, hipStream_t stream);
hipError_t launch_res_readout(const ResPlan& pl, float den_eps, float cap, int cap_on, int chains, int b_lo, int nb,
                              int max_wg, int32_t* chain_info, hipStream_t stream);

}  // namespace vla
