// Register-tile layout, LDS vector helpers and the HBM -> LDS token stager
// shared by the scan kernels.
#pragma once
#include "vla_common.h"

namespace vla {

// kFull: the whole recurrence.  kStateOnly: S, n, cap and readout from a
// precomputed alpha_hat.  kInverseOnly: the inverse recurrence over one chunk
// of tokens from a precomputed chunk-start inverse, writing alpha_hat.
enum class SeqMode { kFull, kStateOnly, kInverseOnly };

// Per-chain bookkeeping of the time-parallel schedule, int32 [chains][4].
constexpr int kInfoGuard = 0;      // guard fires in the inverse pass
constexpr int kInfoFallback = 1;   // nonzero: redo this chain sequentially
constexpr int kInfoNonfinite = 2;  // a non-finite alpha_hat or inverse appeared
// Residual update with the cap: nblk - (first block with a token over the
// cap), 0 = none; the restart set-up then turns it into the token from which
// the sequential fallback reruns the chain.
constexpr int kInfoRestart = 3;

struct SeqExtra {
  const float* alpha;         // kStateOnly: alpha_hat per token, [chains][T][d] fp32
  float* alpha_out;           // kInverseOnly: same layout, written
  const float* a_start;       // kInverseOnly: chunk-start inverses [chains][nchunks][d][d]
  int32_t* chain_info;        // kStateOnly/kInverseOnly: [chains][4], see kInfo*
  const int32_t* only_if;     // kFull: chain_info of a time-parallel run; only chains
                              // with the fallback flag set run (nullable: all run)
  int32_t chunk_len;          // kInverseOnly: tokens per chunk
  int32_t nchunks;            // kInverseOnly: chunks per chain
  int32_t chunk_lo;           // kInverseOnly: this launch runs chunks [chunk_lo, chunk_lo + chunk_cnt)
  int32_t chunk_cnt;
};

constexpr int kMaxStageVecs = 8;   // 16-byte staging registers per thread

// NW waves split d rows into slabs of RW; a wave's lanes form RG row groups of
// CG lanes; each lane owns R rows and C columns (float4-interleaved).
template <int D, int NW, int CG>
struct TileLayout {
  static constexpr int kThreads = 64 * NW;
  static constexpr int RW = D / NW;
  static constexpr int RG = 64 / CG;
  static constexpr int R = RW / RG;
  static constexpr int C = D / CG;
  static_assert(RW % RG == 0 && R >= 1, "each lane needs at least one row");
  static_assert(C % 4 == 0, "columns come in float4 blocks");
};

// This lane's C columns of an LDS vector: j = (m*CG + cg)*4 + e.
template <int CG, int C>
__device__ __forceinline__ void lds_cols(const float* vec, int cg, float (&out)[C]) {
#pragma unroll
  for (int m = 0; m < C / 4; ++m) {
    const float4 x = *reinterpret_cast<const float4*>(vec + (m * CG + cg) * 4);
    out[4 * m + 0] = x.x; out[4 * m + 1] = x.y; out[4 * m + 2] = x.z; out[4 * m + 3] = x.w;
  }
}

// R consecutive entries of an LDS vector.
template <int R>
__device__ __forceinline__ void lds_rows(const float* vec, float (&out)[R]) {
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(vec + 4 * i);
      out[4 * i + 0] = x.x; out[4 * i + 1] = x.y; out[4 * i + 2] = x.z; out[4 * i + 3] = x.w;
    }
  } else if constexpr (R == 2) {
    const float2 x = *reinterpret_cast<const float2*>(vec);
    out[0] = x.x; out[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) out[i] = vec[i];
  }
}

template <int R>
__device__ __forceinline__ void lds_store_rows(float* vec, const float (&in)[R]) {
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i)
      *reinterpret_cast<float4*>(vec + 4 * i) = make_float4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
  } else if constexpr (R == 2) {
    *reinterpret_cast<float2*>(vec) = make_float2(in[0], in[1]);
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) vec[i] = in[i];
  }
}

// A += s*I on this lane's tile (rows row0.., interleaved columns).
template <int R, int C, int CG, int RA, int CA>
__device__ __forceinline__ void add_to_diagonal(float (&A)[RA][CA], int row0, int cg, float s) {
#pragma unroll
  for (int ii = 0; ii < R; ++ii)
#pragma unroll
    for (int m = 0; m < C / 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (row0 + ii == (m * CG + cg) * 4 + e) A[ii][4 * m + e] += s;
}

// Row streams of a token: rows 0..nfix-1 come from fix0..fix2 (stride D per
// token); rows nfix..n-1 are the r penalty directions, row nfix+i of token t
// at ubase + i*D + t*ustride.  Plain members (no arrays) keep the selection
// in registers.
template <typename T, int D>
struct RowSource {
  int n, nfix;
  const T* fix0;
  const T* fix1;
  const T* fix2;
  const T* ubase;
  int64_t ustride;

  __device__ __forceinline__ const T* row(int vv, int t) const {
    if (vv >= nfix) return ubase + (vv - nfix) * D + t * ustride;
    // Arithmetic select: a conditional chain here becomes a lookup table in
    // scratch memory.
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(fix0);
    const uintptr_t p = a0 + static_cast<uintptr_t>(vv == 1) * (reinterpret_cast<uintptr_t>(fix1) - a0) +
                        static_cast<uintptr_t>(vv == 2) * (reinterpret_cast<uintptr_t>(fix2) - a0);
    return reinterpret_cast<const T*>(p) + static_cast<int64_t>(t) * D;
  }
};

// Streams TT tokens of row streams from HBM into an LDS stage [TT][n][D] of
// float32 (bf16 widened exactly).  Each thread moves up to SLOTS (at most
// kMaxStageVecs) 16-byte vectors; the caller sizes the stage to fit.  Tokens
// at or past T read as 0.
template <typename TSrc, int D, int NTH, int SLOTS = kMaxStageVecs>
struct Stager {
  static constexpr int EPV = Elem<TSrc>::kPer16B;
  static constexpr int VPR = D / EPV;
  static_assert(SLOTS >= 1 && SLOTS <= kMaxStageVecs, "staging slots");
  uint4 reg[SLOTS];

  __device__ __forceinline__ void load(const RowSource<TSrc, D> s, int tb, int TT, int T, int tid) {
    const int nvec = TT * s.n * VPR;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int e = tid + j * NTH;
      reg[j] = make_uint4(0, 0, 0, 0);
      if (e < nvec) {
        const int rho = e / VPR, c = e % VPR;
        const int tt = rho / s.n, vv = rho - tt * s.n;
        const int t = tb + tt;
        if (t < T) reg[j] = *reinterpret_cast<const uint4*>(s.row(vv, t) + c * EPV);
      }
    }
  }

  // Rows land at stage + (token * rows_per_token + row) * D; rows_per_token
  // defaults to n (the rows loaded per token) and may be larger, leaving the
  // remaining rows of each token for the caller to fill.
  __device__ __forceinline__ void store(float* stage, int TT, int n, int tid, int rows_per_token = 0) const {
    const int nvec = TT * n * VPR;
    const int rpt = rows_per_token > 0 ? rows_per_token : n;
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int e = tid + j * NTH;
      if (e < nvec) {
        const int rho = e / VPR, c = e % VPR;
        const int orow = rpt == n ? rho : (rho / n) * rpt + rho % n;
        float* dst = stage + orow * D + c * EPV;
        if constexpr (EPV == 4) {
          *reinterpret_cast<uint4*>(dst) = reg[j];
        } else {
          const uint32_t w[4] = {reg[j].x, reg[j].y, reg[j].z, reg[j].w};
          float f[8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            f[2 * h] = __uint_as_float(w[h] << 16);
            f[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
          }
          *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
    }
  }
};

// Rows per token streamed in the input dtype: q, k, v, u_1..u_r (kFull);
// q, k, v (kStateOnly); k, u_1..u_r (kInverseOnly).
template <typename TIn, int D, int NW>
__host__ __device__ constexpr int seq_rows_per_token(SeqMode m, int r) {
  return m == SeqMode::kFull ? 3 + r : (m == SeqMode::kStateOnly ? 3 : 1 + r);
}

// Tokens per LDS stage: one stage fits the staging registers of every row
// stream, and the two stages stay within 48 KiB.
template <typename TIn, int D, int NW>
__host__ __device__ constexpr int seq_stage_tokens(SeqMode m, int r) {
  const bool state_only = m == SeqMode::kStateOnly;
  const int nv = seq_rows_per_token<TIn, D, NW>(m, r);  // rows per token in TIn
  const int nf = nv + (state_only ? 1 : 0);              // fp32 rows per token in LDS
  constexpr int VPR = D / Elem<TIn>::kPer16B;
  int cap = (kMaxStageVecs * 64 * NW) / (nv * VPR);
  if (state_only) {
    const int cap_a = (kMaxStageVecs * 64 * NW) / (D / 4);
    cap = cap < cap_a ? cap : cap_a;
  }
  const int lds_cap = (48 * 1024) / (2 * nf * D * static_cast<int>(sizeof(float)));
  cap = cap < lds_cap ? cap : lds_cap;
  return cap >= 8 ? 8 : (cap < 1 ? 1 : cap);
}

// Staging slots per thread that every rank r <= 4 needs: a stage holds at
// most 8 tokens of at most the mode's rows at r = 4, and never more vectors
// than kMaxStageVecs per thread (seq_stage_tokens caps it there).
template <typename TIn, int D, int NW>
__host__ __device__ constexpr int seq_stage_slots(SeqMode m) {
  const int nvmax = seq_rows_per_token<TIn, D, NW>(m, 4);
  const int vecs = 8 * nvmax * (D / Elem<TIn>::kPer16B);
  const int slots = (vecs + 64 * NW - 1) / (64 * NW);
  return slots < kMaxStageVecs ? slots : kMaxStageVecs;
}

template <typename TIn, int D, int NW>
inline size_t seq_lds_bytes(SeqMode m, int r) {
  const int TT = seq_stage_tokens<TIn, D, NW>(m, r);
  const int nf = seq_rows_per_token<TIn, D, NW>(m, r) + (m == SeqMode::kStateOnly ? 1 : 0);
  return sizeof(float) * (2 * TT * nf * D + 4 * D + 2 * NW * 4);
}

}  // namespace vla
