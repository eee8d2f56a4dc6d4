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
  int32_t residual;       // nonzero: residual (delta-rule) state update; full recurrence only
  // Fused prologue (two-wave kernel only): q and k hold the raw inputs, the
  // kernel applies ELU+1 to them and projects u = normalize(W_u[i] k_raw)
  // itself; u is unused.  Features and u are rounded to the storage dtype.
  int32_t fused;
  const void* W_u;        // [r][d][d] in the storage dtype
};

// Sequential scan with the fused prologue (d <= 64, the two-wave kernel).
hipError_t launch_scan_split_fused(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream);

// Whole recurrence, one workgroup per chain.  only_if (nullable) restricts
// the run to chains whose flag is nonzero.
hipError_t launch_scan_sequential(const ScanArgs& a, int d, bool bf16, int chains, const int32_t* only_if,
                                  hipStream_t stream);

// Time-parallel inverse schedule (d = 64, and d = 128 with bf16 storage):
// buffers live in the caller's workspace; see chunked.hip.  Matrices below
// are d x d (shown for d = 64).
struct ChunkPlan {
  int chains, T, r, d;
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

// Snapshot of the initial state, per-chunk Gram matrices, their per-period
// prefixes and the (N, D) chain.
hipError_t launch_chunk_prologue(const ChunkPlan& pl, const float* A0, const float* S0, const float* n0,
                                 const void* u, bool bf16, hipStream_t stream);

// Chunk-start inverses of chunks [c_lo, c_lo + c_cnt).
hipError_t launch_chunk_start(const ChunkPlan& pl, int c_lo, int c_cnt, hipStream_t stream);

// Blocked state pass (d = 64, blocks of 64 tokens); buffers in the workspace.
struct StatePlan {
  int T, nblk;
  int bf16;              // storage of q, k, v, o
  const void* v;
  const float* alpha;    // [chains][T][64] alpha_hat from the inverse pass
  float* Kmat;           // [chains][nblk][2304] lower triangle of the row prefix sums over s<j of
                         // K(t,s) = (v_t.v_s)(alpha_t.alpha_s) (row t's j = 0..t at t(t+1)/2 + j), then
                         // K(t,t), sum_s K(t,s), sum_t k_t (64 each) and padding
  float* Kcross;         // [chains][nblk][64][64] (v_t.v_s)(alpha_t.alpha_s), s in the previous block
  void* VT;              // [chains][nblk][512][8] v regrouped as matrix-core operands (storage dtype)
  float* AT;             // [chains][nblk][512][8] alpha_hat regrouped the same way
  float* Xsnap;          // [chains][nblk][64][64] S at each block start
  float* wsig;           // [chains][T][2] block-local log2 scales: log2 sigma_{t-1}, log2 sigma_t
  float* ld;             // [chains][T] sum_{s<=t in block} k_s.q_t
  float* nblock;         // [chains][nblk][64] normaliser at each block start
};

// One segment of the chain kernel: blocks [b_lo, b_hi), b_lo even, continuing
// from S and n at block b_lo.  A segment that does not end the sequence leaves
// S at b_hi in Xsnap, n in n_carry and its counters for the next one; the last
// writes S_T, n_T and stats (guard count and non-finite flag of the inverse
// pass taken from chain_info).
constexpr int kMaxParaSegs = 16;
struct ChainSeg {
  int b_lo, b_hi;
  const float* S_in;      // S at block b_lo, chain c at S_in + c * S_in_stride
  int64_t S_in_stride;
  const float* n_in;      // n at block b_lo, chain c at n_in + c * n_in_stride
  int64_t n_in_stride;
  float* n_carry;         // [chains][64] n after block b_hi - 1
  int32_t* counters;      // [chains][2] cap fires so far and the first cap step (-1: none)
  int last;
  // Parallel-in-time mode (pr != 0): all segments of every chain at once;
  // workgroup x runs segment x / chains of chain x % chains over blocks
  // [bnd[seg], bnd[seg + 1]), from S_in + (c * nseg + seg) * 4096 and
  // n_in + (c * nseg + seg) * 64, and leaves S at the segment's end in F and
  // (log2 sigma over the segment, cap fires, first cap step) in rec.
  int pr, nseg;
  int bnd[kMaxParaSegs + 1];
  float* F;               // [chains][nseg][64][64]
  float* rec;             // [chains][nseg][4]
  const int32_t* conv;    // [chains]: nonzero once the chain's segment starts have converged
  const int32_t* active;  // [chains][nseg] (nullable): zero skips the segment (its start has not moved)
};

// Parallel-in-time state pass (state_pass.hip): the segment starts' sweep
// between chain-kernel passes, the normaliser at the segment starts, and the
// per-chain statistics.
struct ParaPlan {
  int chains, nseg, iter_last;   // iter_last: this sweep is the last one allowed
  int bnd[kMaxParaSegs + 1];
  const float* S_init;   // [chains][64][64]
  float* Sit;            // [chains][nseg][64][64] segment starts of the next pass
  const float* F;        // [chains][nseg][64][64]
  const float* rec;      // [chains][nseg][4]
  int32_t* conv;         // [chains]
  int32_t* active;       // [chains][nseg]: segments whose start moved, to run in the next pass
  int32_t* chain_info;   // [chains][4]: the fallback flag is set if a chain does not converge
  float cap, tol, tol_skip;
  int cap_on;
  float* P;              // [chains][nseg][kParaSub][64][64]: plain sums of v alpha_hat^T over the
                         // sub-steps of each segment (the first sweep's input)
};
constexpr int kParaSub = 4;   // sub-steps per segment of the first sweep
hipError_t launch_para_init(const ParaPlan& pp, const StatePlan& pl, const float* n_init, float* n_seg,
                            hipStream_t stream);
// The plain sums pp.P (one workgroup per chain, segment and sub-step).
hipError_t launch_para_sums(const ParaPlan& pp, const StatePlan& pl, hipStream_t stream);
hipError_t launch_para_sweep(const ParaPlan& pp, int first, hipStream_t stream);
hipError_t launch_para_stats(const ParaPlan& pp, const float* S_T, const float* n_T, int32_t* stats,
                             hipStream_t stream);

// Prep and readout of blocks [b_lo, b_lo + nb) of every chain (parallel, at
// most max_wg workgroups if max_wg > 0); the readout flags non-finite outputs
// in chain_info.
hipError_t launch_state_prep(const StatePlan& pl, const ScanArgs& a, int chains, int b_lo, int nb, int max_wg,
                             hipStream_t stream);
hipError_t launch_state_readout(const StatePlan& pl, const ScanArgs& a, int32_t* chain_info, int chains, int b_lo,
                                int nb, int max_wg, hipStream_t stream);
// The chain kernel over one segment (one workgroup per chain), or in
// parallel-in-time mode over all segments (chains * nseg workgroups).
// Non-null events are recorded on the stream right before and after it.
hipError_t launch_state_chain(const StatePlan& pl, const ChainSeg& sg, const ScanArgs& a, const int32_t* chain_info,
                              int chains, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

// State pass at d = 128 without the cap (linear_state.hip): additive update,
// bf16 storage, chunks of kLinChunk tokens.
constexpr int kLinChunk = 256;
struct LinPlan {
  int chains, T, ncs;      // ncs = ceil(T / kLinChunk)
  const void* q;           // [chains][T][128] bf16
  const void* k;
  const void* v;
  void* o;
  const float* alpha;      // [chains][T][128] alpha_hat from the inverse pass
  float* dS;               // [chains][ncs][128][128]: chunk sums, then the chunk-start S
  float* dn;               // [chains][ncs][128]: the same for n
  const float* S_init;     // [chains][128][128]
  const float* n_init;     // [chains][128]
  float* S_T;
  float* n_T;
  int32_t* chain_info;     // [chains][4]: guard fires and flags of the inverse pass
  int32_t* stats;          // nullable
  float den_eps;
};
hipError_t launch_linear_state(const LinPlan& lp, hipStream_t stream);

// Inverse recurrence of chunks [chunk_lo, chunk_lo + chunk_cnt) from their
// chunk-start inverses; writes alpha_hat and, from each chain's last chunk, A_T.
hipError_t launch_scan_inverse_chunks(const ScanArgs& a, const float* a_start, float* alpha_out,
                                      int32_t* chain_info, int chunk_len, int nchunks, int chunk_lo, int chunk_cnt,
                                      int d, bool bf16, int chains, hipStream_t stream);

// The same pass in blocked form on the matrix cores (inverse_wy.hip): d = 64,
// r = 1 only, bf16 or fp32 storage.
hipError_t launch_inverse_wy(const ScanArgs& a, const float* a_start, float* alpha_out, int32_t* chain_info,
                             int chunk_len, int nchunks, int chunk_lo, int chunk_cnt, bool bf16, int chains,
                             hipStream_t stream);

hipError_t launch_project_u(int64_t rows, int d, int r, bool in_bf16, bool out_bf16, const void* W,
                            const void* kraw, void* u, hipStream_t stream);

// Sets *flag (device int) to 1 if any of the n elements at the given buffers
// is NaN or Inf; *flag must be cleared first with launch_clear_flag.
hipError_t launch_clear_flag(int32_t* flag, hipStream_t stream);

// Strided q, k, v views gathered into contiguous rows (see gather_rows_kernel).
struct GatherArgs {
  const char* q;
  const char* k;
  const char* v;
  char* dst;             // three [rows][row_bytes] tensors back to back
  int64_t rows;          // B * H * T
  int64_t T, H;
  int64_t stride_b, stride_h, stride_t;   // elements
  int32_t elem_bytes;    // 2 or 4
  int32_t row_bytes;     // d * elem_bytes, a multiple of 16
};
hipError_t launch_gather_rows(const GatherArgs& g, hipStream_t stream);

// q = ELU(q_raw) + 1 and k = ELU(k_raw) + 1 over n elements each, in the storage dtype.
hipError_t launch_feature_map(const void* q_raw, const void* k_raw, void* q, void* k, int64_t n, bool bf16,
                              hipStream_t stream);

// Backward pass (backward.hip): inputs, cotangents, gradients and the tape.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* u;
  const float* A0;    // nullable: I
  const float* S0;    // nullable: 0
  const float* n0;    // nullable: 0
  const float* go;    // [chains][T][d] fp32
  const float* gAT;   // nullable cotangents of the final state
  const float* gST;
  const float* gnT;
  float* gq;          // [chains][T][d]
  float* gk;
  float* gv;
  float* gu;          // [chains][T][r][d]
  float* gA0;         // [chains][d][d]
  float* gS0;
  float* gn0;         // [chains][d]
  int32_t T, r;
  float eps;
  int32_t nudge_period, nudge_phase0;
  int32_t cap_on;
  float cap, den_eps;
  // tape and checkpoints (workspace)
  float* ckA;
  float* ckS;
  float* ckn;
  float* sbuf;
  float* tz;
  float* tdelta;
  float* tfire;
  float* tah;
  float* tan_;
  float* tc;
};
size_t bwd_workspace_bytes(int64_t chains, int T, int d, int r);
void bwd_carve(BwdArgs& a, void* ws, int64_t chains, int T, int d, int r);
hipError_t launch_backward(const BwdArgs& a, int d, bool bf16, int chains, hipStream_t stream);
// stats[c][2] |= chain_info[c] non-finite flag (stats nullable).
hipError_t launch_stats_finalize(int32_t* stats, const int32_t* chain_info, int chains, hipStream_t stream);
hipError_t launch_nonfinite_check(const void* p, int64_t n, bool bf16, int32_t* flag, hipStream_t stream);

}  // namespace vla
