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

// Whole recurrence, one workgroup per chain.  only_if (nullable) restricts
// the run to chains whose flag is nonzero.
hipError_t launch_scan_sequential(const ScanArgs& a, int d, bool bf16, int chains, const int32_t* only_if,
                                  hipStream_t stream);

// State recurrence only (S, n, cap, readout) from precomputed alpha_hat.
hipError_t launch_scan_state_only(const ScanArgs& a, const float* alpha, int32_t* chain_info, int d,
                                  bool bf16, int chains, hipStream_t stream);

// Time-parallel inverse schedule (d = 64): buffers live in the caller's
// workspace; see chunked.hip.
struct ChunkPlan {
  int chains, T, r;
  int L;          // tokens per chunk
  int nchunks;    // ceil(T / L)
  int nperiods;   // nudge periods touched by this call
  int o, q;       // t0 / L and nudge_period / L (q = 0: no nudge)
  float eps;
  float* A_init;  // snapshots of the initial state [chains][64][64], [chains][64][64], [chains][64]
  float* S_init;
  float* n_init;
  int32_t* chain_info;  // [chains][4]
  float* G;       // [chains][nchunks][64][64]
  double* Gpre;   // [chains][nchunks][64][64] Gram sum of the earlier chunks of the chunk's period
  double* Gtot;   // [chains][nperiods][64][64] Gram sum of each period
  double* ND;     // [chains][nperiods][2][64][64]
  float* Ac;      // [chains][nchunks][64][64]
  float* alpha;   // [chains][T][64]
};

// Snapshot of the initial state, per-chunk Gram matrices, the (N, D) chain and
// the chunk-start inverses.
hipError_t launch_chunk_prologue(const ChunkPlan& pl, const float* A0, const float* S0, const float* n0,
                                 const void* u, bool bf16, hipStream_t stream);

// Blocked state pass (d = 64, blocks of 64 tokens); buffers in the workspace.
struct StatePlan {
  int T, nblk;
  int bf16;              // storage of q, k, v, o
  const void* v;
  const float* alpha;    // [chains][T][64] alpha_hat from the inverse pass
  float* Kmat;           // [chains][nblk][68][64] row prefix sums over s<j of K(t,s) = (v_t.v_s)(alpha_t.alpha_s),
                         // then rows K(t,t), sum_s K(t,s), sum_t k_t and one padding row
  float* Kcross;         // [chains][nblk][64][64] (v_t.v_s)(alpha_t.alpha_s), s in the previous block
  void* VT;              // [chains][nblk][512][8] v regrouped as matrix-core operands (storage dtype)
  float* AT;             // [chains][nblk][512][8] alpha_hat regrouped the same way
  float* Xsnap;          // [chains][nblk][64][64] S at each block start
  float* wsig;           // [chains][T][2] block-local log2 scales: log2 sigma_{t-1}, log2 sigma_t
  float* ld;             // [chains][T] sum_{s<=t in block} k_s.q_t
  float* nblock;         // [chains][nblk][64] normaliser at each block start
};

// Prep (parallel), chain (one workgroup per chain) and readout (parallel):
// writes o, S_T, n_T and stats (guard count and inverse-pass non-finite flag
// taken from chain_info).  Non-null events are recorded on the stream right
// before and after the chain kernel.
hipError_t launch_state_pass(const StatePlan& pl, const ScanArgs& a, int32_t* chain_info, int chains,
                             hipStream_t stream, hipEvent_t chain_start = nullptr, hipEvent_t chain_stop = nullptr);

// Inverse recurrence of every chunk from its chunk-start inverse; writes
// alpha_hat and, from each chain's last chunk, A_T.
hipError_t launch_scan_inverse_chunks(const ScanArgs& a, const float* a_start, float* alpha_out,
                                      int32_t* chain_info, int chunk_len, int nchunks, int d, bool bf16, int chains,
                                      hipStream_t stream);

hipError_t launch_project_u(int64_t rows, int d, int r, bool in_bf16, bool out_bf16, const void* W,
                            const void* kraw, void* u, hipStream_t stream);

// Sets *flag (device int) to 1 if any of the n elements at the given buffers
// is NaN or Inf; *flag must be cleared first with launch_clear_flag.
hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream);
hipError_t launch_nonfinite_check(const void* p, int64_t n, bool bf16, int32_t* flag, hipStream_t stream);

}  // namespace vla
