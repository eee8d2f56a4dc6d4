// Time-parallel ("chunked") schedule of the VLA inverse recurrence, d = 64.
//
// The pages fuse all T steps in one launch and mention a parallel
// Blelloch-style formulation ("Variational Linear Attention: Stable
// Associative Memory for Long-Context Transformers", technical summary 2.4).
// This schedule is exact in exact arithmetic and built on the structure of
// the penalty matrix ("Mathematical Primitives", section 2, theoretical
// derivation): while no guard fires, A_t = M_t^{-1} with M_t = M_{t-1} +
// u_t u_t^T, so the penalty over a chunk of L tokens adds the Gram matrix
// G_c = sum u u^T.  The periodic nudge A <- A + eps*I is not additive in M;
// writing A = N D^{-1}, both steps are linear in (N, D):
//     rank-1 update:  D <- D + u u^T N
//     nudge:          N <- N + eps D
// so each chain carries (N, D) across chunks with one d x d x d product per
// nudge period, and every chunk-start inverse A_c = N_p (D_p + Gpre_c N_p)^{-1}
// follows in parallel.  From A_c, the existing sequential inverse recurrence
// runs each chunk independently (kInverseOnly mode).
//
// Kernels, in stream order:
//   vla_chunk_gram_kernel   G_c for every chunk (MFMA, fp32 accumulation)
//   vla_chunk_scan_kernel   fp64 prefix sums of G inside each nudge period and
//                           each period's total, in parallel over elements
//   vla_chunk_chain_kernel  per chain and column block, sequential over
//                           periods, fp64: (N, D) at every period start
//   vla_chunk_start_kernel  per chunk, fp64: A_c by blocked Gauss-Jordan
//                           elimination of [ D_c^T | N_p^T ] on the fp64
//                           matrix cores; a non-positive pivot flags the
//                           chain for the sequential fallback
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_seq.h"

namespace vla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;            // head dimension of this schedule
constexpr int kChunkThreads = 256;

__global__ void snapshot_kernel(const float* __restrict__ A0, const float* __restrict__ S0,
                                const float* __restrict__ n0, float* __restrict__ A_copy,
                                float* __restrict__ S_copy, float* __restrict__ n_copy,
                                int32_t* __restrict__ chain_info, int64_t chains) {
  const int64_t mat = chains * kD * kD;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < mat;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = i % (kD * kD);
    A_copy[i] = A0 ? A0[i] : ((e / kD) == (e % kD) ? 1.f : 0.f);
    S_copy[i] = S0 ? S0[i] : 0.f;
    if (i < chains * kD) n_copy[i] = n0 ? n0[i] : 0.f;
    if (i < chains * 4) chain_info[i] = 0;
  }
}

// Period index of chunk c: the number of nudges at the ends of chunks < c.
// Chunk c ends at global token index t0 + (c+1)L, so with o = t0/L and
// q = P/L a nudge follows chunk c' when (o + c' + 1) % q == 0.
__device__ __forceinline__ int period_of(int c, int o, int q) {
  return q > 0 ? (o + c) / q - o / q : 0;
}

// ---- Gram matrices ---------------------------------------------------------
// One workgroup per (chain, chunk); wave w accumulates 32x32 tiles of
// G = U^T U, U the chunk's rows of u ([L*r, 64], contiguous).
template <typename TIn>
__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_gram_kernel(const TIn* __restrict__ u, float* __restrict__ G, int T, int r, int L, int nchunks) {
  const int64_t chain = blockIdx.x / nchunks;
  const int c = blockIdx.x % nchunks;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t_lo = c * L, t_hi = min(T, t_lo + L);
  const int nrows = (t_hi - t_lo) * r;
  const TIn* U = u + (chain * T + t_lo) * static_cast<int64_t>(r) * kD;
  const int ib = w >> 1, jb = w & 1;     // 4 waves, 2x2 tiles
  const int fa = ib * 32 + (lane & 31), fb = jb * 32 + (lane & 31);
  f32x16 acc = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(TIn) == 2) {
    const int koff = 8 * (lane >> 5);
    for (int k0 = 0; k0 < nrows; k0 += 16) {
      uint16_t av[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = k0 + koff + e;
        const bool ok = k < nrows;
        av[e] = ok ? U[static_cast<int64_t>(k) * kD + fa] : uint16_t(0);
        bv[e] = ok ? U[static_cast<int64_t>(k) * kD + fb] : uint16_t(0);
      }
      const uint4 ap = make_uint4(av[0] | (uint32_t(av[1]) << 16), av[2] | (uint32_t(av[3]) << 16),
                                  av[4] | (uint32_t(av[5]) << 16), av[6] | (uint32_t(av[7]) << 16));
      const uint4 bp = make_uint4(bv[0] | (uint32_t(bv[1]) << 16), bv[2] | (uint32_t(bv[3]) << 16),
                                  bv[4] | (uint32_t(bv[5]) << 16), bv[6] | (uint32_t(bv[7]) << 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ap), __builtin_bit_cast(bf16x8, bp),
                                                     acc, 0, 0, 0);
    }
  } else {
    const int koff = lane >> 5;
    for (int k0 = 0; k0 < nrows; k0 += 2) {
      const int k = k0 + koff;
      const bool ok = k < nrows;
      const float a = ok ? U[static_cast<int64_t>(k) * kD + fa] : 0.f;
      const float b = ok ? U[static_cast<int64_t>(k) * kD + fb] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
  }
  float* g = G + (chain * nchunks + c) * kD * kD;
  const int col = jb * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int row = ib * 32 + 8 * (s / 4) + 4 * (lane >> 5) + (s % 4);
    g[row * kD + col] = acc[s];
  }
}

// ---- Gram prefixes ----------------------------------------------------------
// Segmented exclusive prefix over the chunks of each nudge period, in fp64:
// Gpre_c = sum of G_c' over the earlier chunks c' of c's period, and Gtot_p =
// the whole period's sum.  One thread per (chain, matrix element); the chunk
// loop is sequential only through the running sum, so loads are issued eight
// chunks ahead.
__global__ void __launch_bounds__(256)
vla_chunk_scan_kernel(const float* __restrict__ G, double* __restrict__ Gpre, double* __restrict__ Gtot,
                      int64_t chains, int nchunks, int nperiods, int o, int q) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= chains * kD * kD) return;
  const int64_t chain = idx / (kD * kD);
  const int e = static_cast<int>(idx % (kD * kD));
  const float* g = G + chain * nchunks * kD * kD + e;
  double* gp = Gpre + chain * nchunks * kD * kD + e;
  double* gt = Gtot + chain * nperiods * kD * kD + e;
  double acc = 0.0;
  int p = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 8) {
    float gv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) gv[k] = (c0 + k < nchunks) ? g[static_cast<int64_t>(c0 + k) * kD * kD] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = c0 + k;
      if (c < nchunks) {
        const int pc = period_of(c, o, q);
        if (pc != p) {
          gt[static_cast<int64_t>(p) * kD * kD] = acc;
          acc = 0.0;
          p = pc;
        }
        gp[static_cast<int64_t>(c) * kD * kD] = acc;
        acc += static_cast<double>(gv[k]);
      }
    }
  }
  gt[static_cast<int64_t>(p) * kD * kD] = acc;
}

// ---- (N, D) chain ---------------------------------------------------------
// Between periods p and p+1: D += Gtot_p N, then the nudge N += eps D.  Both
// steps act on each column of (N, D) separately, so a chain runs as
// kNdSplit independent workgroups, one per block of 64/kNdSplit = 4 columns.
// The four waves of a workgroup each take a quarter of the product's inner
// dimension (thread (q, rb, c): rows 4 rb.. of column c, inner indices
// 16 q..); the waves' partial sums meet in LDS, where the first wave, which
// owns (N, D), adds them.  The period's Gram total is symmetric, so it is
// staged in LDS as it is stored (row m serves as column m: no transposed
// stores); the next one is loaded while the current product runs, and the
// LDS buffers alternate between periods, so a period needs two barriers.
constexpr int kNdSplit = 16;
constexpr int kNdCols = kD / kNdSplit;   // 4
// fp64 LDS rows of 68 doubles: 16-byte aligned, so a thread's four
// consecutive entries move as two 16-byte accesses.
constexpr int kPadG = kD + 4;
// fp64 LDS rows padded to 65 doubles (the chunk-start kernel's staging).
constexpr int kPad = kD + 1;

__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_chain_kernel(const double* __restrict__ Gtot, const float* __restrict__ A0, double* __restrict__ ND,
                       int nperiods, double eps) {
  __shared__ double sG[2][kD * kPadG];         // sG[m * kPadG + i] = Gtot[m][i] = Gtot[i][m]
  __shared__ double sN[2][kD * kNdCols];       // sN[m * kNdCols + c] = N[m][c0 + c]
  __shared__ double sP[2][4][kD * kNdCols];    // partial products of each wave
  const int64_t chain = blockIdx.x / kNdSplit;
  const int c0 = (blockIdx.x % kNdSplit) * kNdCols;
  const int t = threadIdx.x, q = t >> 6, rb = (t & 63) >> 2, cc = t & 3;
  const int col = c0 + cc;
  const bool owner = q == 0;   // wave-uniform
  double N[4], Dm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = 4 * rb + i;
    N[i] = static_cast<double>(A0[(chain * kD + gi) * kD + col]);
    Dm[i] = gi == col ? 1.0 : 0.0;
  }
  auto store_nd = [&](int p) {
    double* nd = ND + (chain * nperiods + p) * 2 * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nd[(4 * rb + i) * kD + col] = N[i];
      nd[kD * kD + (4 * rb + i) * kD + col] = Dm[i];
    }
  };
  // Staging of the 64x64 total: thread t loads rows 4*(t/16).., columns
  // 4*(t%16)..; two register sets, so each total is loaded two periods ahead.
  const int sr = t >> 4, sc = t & 15;
  double ga[16], gb[16];
  auto load_g = [&](double (&g)[16], int p) {
    if (p + 1 >= nperiods) return;   // the last period's total is not needed
    const double* gt = Gtot + (chain * nperiods + p) * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) g[4 * i + j] = gt[(4 * sr + i) * kD + 4 * sc + j];
  };
  auto advance = [&](double (&g)[16], int p) {
    // Buffers of parity p & 1: their last readers were in period p - 2, which
    // every wave finished before the previous period's second barrier.
    double* G = sG[p & 1];
    double* Ns = sN[p & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) G[(4 * sr + i) * kPadG + 4 * sc + j] = g[4 * i + j];
    if (owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Ns[(4 * rb + i) * kNdCols + cc] = N[i];
    }
    __syncthreads();
    load_g(g, p + 2);
    double part[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int m = 16 * q; m < 16 * q + 16; ++m) {
      const double nm = Ns[m * kNdCols + cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = fma(G[m * kPadG + 4 * rb + i], nm, part[i]);
    }
    double (*P)[kD * kNdCols] = sP[p & 1];
    if (!owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) P[q][(4 * rb + i) * kNdCols + cc] = part[i];
    }
    __syncthreads();
    if (owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (4 * rb + i) * kNdCols + cc;
        Dm[i] += (part[i] + P[1][e]) + (P[2][e] + P[3][e]);
        N[i] = fma(eps, Dm[i], N[i]);
      }
      store_nd(p + 1);
    }
  };
  if (owner) store_nd(0);
  load_g(ga, 0);
  load_g(gb, 1);
  for (int p = 0; p + 1 < nperiods; p += 2) {
    advance(ga, p);
    if (p + 2 < nperiods) advance(gb, p + 1);
  }
}

// ---- chunk-start inverses ---------------------------------------------------
// One workgroup (four waves) per (chain, chunk).  W = [ D_c^T | N_p^T ] (64 x
// 128, fp64) lives in registers as 16 x 16 matrix-core tiles: wave w holds
// rows 16 w .. 16 w + 15, tiles ct = 0..3 of the left block and 4..7 of the
// right.  D_c^T = D_p^T + N_p^T Gpre_c^T on the fp64 matrix cores.  Gauss-
// Jordan elimination without pivoting then turns W into [ I | A_c^T ], in
// panels of 16 columns: wave p inverts its pivot block W11 (one pivot at a
// time, with cross-lane broadcasts) and forms R = W11^-1 W[panel rows]; every
// other wave w then subtracts C_w R (C_w its rows of the panel's columns).
// Both products run on the matrix cores.  A non-positive or non-finite pivot
// flags the chain for the sequential fallback.
//
// v_mfma_f64_16x16x4f64, wave64, D = A B + C with A 16x4, B 4x16:
//   A operand  lane l holds A[l % 16][l / 16]
//   B operand  lane l holds B[l / 16][l % 16]
//   C / D      lane l slot i holds D[4 i + l / 16][l % 16]
typedef double d4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ d4 mfma64(double a, double b, d4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
constexpr int kRPad = 2 * kD + 1;   // row stride (doubles) of the finished panel rows R

// Panel P of the elimination (compile time, so every tile index is too).
// Wave P inverts its pivot block W11 by Gauss-Jordan on [ W11 | I ] (one
// pivot at a time, two tiles), then forms R = W11^-1 W[panel rows] for the
// tiles right of the panel on the matrix cores; the other waves subtract
// C_w R.  sI is the wave's 16 x 17 staging tile for transposed operand reads.
template <int P>
__device__ __forceinline__ void gj_panel(d4 (&W)[8], int w, int g, int col, double* sR, double* sI, bool& ok) {
  if (w == P) {   // wave-uniform
    d4 inv_t;     // becomes W11^-1
#pragma unroll
    for (int i = 0; i < 4; ++i) inv_t[i] = (4 * i + g == col) ? 1.0 : 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      // Row k of the block sits in lanes 16 (k % 4) .., slot k / 4; the
      // pivot is its entry in column k.
      const double piv = readlane_d(W[P][k >> 2], 16 * (k & 3) + k);
      ok = ok && (piv > 0.0) && isfinite(piv);
      // 1/piv: the hardware reciprocal refined by one Newton step.
      double inv = __builtin_amdgcn_rcp(piv);
      inv = fma(inv, fma(-piv, inv, 1.0), inv);
      double f[4];   // column k of this lane's rows 4 i + g
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = __shfl(W[P][i], 16 * g + k, 64);
      const double ra = __shfl(W[P][k >> 2], 16 * (k & 3) + col, 64) * inv;
      const double rb = __shfl(inv_t[k >> 2], 16 * (k & 3) + col, 64) * inv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool own = 4 * i + g == k;
        W[P][i] = own ? ra : fma(-f[i], ra, W[P][i]);
        inv_t[i] = own ? rb : fma(-f[i], rb, inv_t[i]);
      }
    }
    // R = W11^-1 W[panel rows] tile by tile: the A operand of k step kk is
    // W11^-1[l % 16][4 kk + l / 16] (a transposed read), the B operand is
    // rows 4 kk + l / 16 of the tile, which is slot kk of this lane.
#pragma unroll
    for (int i = 0; i < 4; ++i) sI[(4 * i + g) * 17 + col] = inv_t[i];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // one wave: its own LDS writes first
    double a[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = sI[col * 17 + 4 * kk + g];
#pragma unroll
    for (int ct = P + 1; ct < 8; ++ct) {
      d4 r = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) r = mfma64(a[kk], W[ct][kk], r);
      W[ct] = r;
#pragma unroll
      for (int i = 0; i < 4; ++i) sR[(4 * i + g) * kRPad + 16 * ct + col] = r[i];
    }
  } else {
    // This wave's rows of the panel's columns, staged for the transposed read.
#pragma unroll
    for (int i = 0; i < 4; ++i) sI[(4 * i + g) * 17 + col] = W[P][i];
  }
  __syncthreads();
  if (w != P) {
    double a[4];   // A operand of k step kk: -C[l % 16][4 kk + l / 16]
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = -sI[col * 17 + 4 * kk + g];
#pragma unroll
    for (int ct = P + 1; ct < 8; ++ct)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) W[ct] = mfma64(a[kk], sR[(4 * kk + g) * kRPad + 16 * ct + col], W[ct]);
  }
  __syncthreads();   // sR and sI are rewritten by the next panel
}

__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_start_kernel(const double* __restrict__ Gpre, const double* __restrict__ ND, float* __restrict__ Ac,
                       int32_t* __restrict__ chain_info, int nchunks, int nperiods, int o, int q, int c_lo, int c_cnt) {
  // 66.6 KiB of LDS: N_p and Gpre_c rows (padded); after the product the
  // second half holds the finished panel rows and the per-wave panel-column
  // tiles, and at the end the first half holds the result block.
  __shared__ double sN[kD * kPad];
  __shared__ double sG[kD * kPad];
  double* sR = sG;                          // [16][kRPad]
  double* sIw = sG + 16 * kRPad;            // [4 waves][16][17]
  const int64_t chain = blockIdx.x / c_cnt;
  const int c = c_lo + static_cast<int>(blockIdx.x % c_cnt);
  const int p = period_of(c, o, q);
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const double* Np = ND + (chain * nperiods + p) * 2 * kD * kD;
  const double* Dp = Np + kD * kD;
  const double* gp = Gpre + (chain * nchunks + c) * kD * kD;
  // The first chunk of a period has no Gram prefix: D_c = D_p.
  const bool has_pre = c > 0 && (q == 0 || (o + c) % q != 0);

  // Every global load first (one round of latency), then the LDS stores.
  constexpr int kPer = kD * kD / kChunkThreads;   // 16 elements per thread
  double rn[kPer], rg[kPer], dp[16];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    rn[j] = Np[t + kChunkThreads * j];
    rg[j] = has_pre ? gp[t + kChunkThreads * j] : 0.0;
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)   // D_p^T, this lane's entries of the left block
#pragma unroll
    for (int i = 0; i < 4; ++i) dp[4 * ct + i] = Dp[(16 * ct + col) * kD + 16 * w + 4 * i + g];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = t + kChunkThreads * j, i = e / kD, jj = e % kD;
    sN[i * kPad + jj] = rn[j];
    if (has_pre) sG[i * kPad + jj] = rg[j];
  }
  __syncthreads();

  d4 W[8];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {   // right block: N_p^T
#pragma unroll
    for (int i = 0; i < 4; ++i) W[4 + qb][i] = sN[(16 * qb + col) * kPad + 16 * w + 4 * i + g];
  }
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {   // left block: D_p^T + N_p^T Gpre_c^T
    d4 acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = dp[4 * ct + i];
    if (has_pre) {
#pragma unroll 4
      for (int kk = 0; kk < kD / 4; ++kk)
        acc = mfma64(sN[(4 * kk + g) * kPad + 16 * w + col], sG[(16 * ct + col) * kPad + 4 * kk + g], acc);
    }
    W[ct] = acc;
  }
  __syncthreads();   // sG is reused below

  bool ok = true;
  double* sI = sIw + w * 16 * 17;
  gj_panel<0>(W, w, g, col, sR, sI, ok);
  gj_panel<1>(W, w, g, col, sR, sI, ok);
  gj_panel<2>(W, w, g, col, sR, sI, ok);
  gj_panel<3>(W, w, g, col, sR, sI, ok);
  if (!ok && lane == 0) atomicOr(chain_info + chain * 4 + kInfoFallback, 1);

  // The result block (A_c^T, equal to A_c in exact arithmetic), symmetrised.
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sN[(16 * w + 4 * i + g) * kPad + 16 * qb + col] = W[4 + qb][i];
  __syncthreads();
  float* ac = Ac + (chain * nchunks + c) * kD * kD;
  for (int e = t; e < kD * kD; e += kChunkThreads) {
    const int i = e / kD, j = e % kD;
    ac[e] = static_cast<float>(0.5 * (sN[i * kPad + j] + sN[j * kPad + i]));
  }
}

}  // namespace

hipError_t launch_chunk_prologue(const ChunkPlan& pl, const float* A0, const float* S0, const float* n0,
                                 const void* u, bool bf16, hipStream_t stream) {
  const int64_t mat = static_cast<int64_t>(pl.chains) * kD * kD;
  const int64_t want = (mat + 255) / 256;
  const unsigned sgrid = static_cast<unsigned>(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(snapshot_kernel, dim3(sgrid), dim3(256), 0, stream, A0, S0, n0, pl.A_init, pl.S_init,
                     pl.n_init, pl.chain_info, static_cast<int64_t>(pl.chains));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned units = static_cast<unsigned>(pl.chains * pl.nchunks);
  if (bf16)
    hipLaunchKernelGGL(vla_chunk_gram_kernel<uint16_t>, dim3(units), dim3(kChunkThreads), 0, stream,
                       static_cast<const uint16_t*>(u), pl.G, pl.T, pl.r, pl.L, pl.nchunks);
  else
    hipLaunchKernelGGL(vla_chunk_gram_kernel<float>, dim3(units), dim3(kChunkThreads), 0, stream,
                       static_cast<const float*>(u), pl.G, pl.T, pl.r, pl.L, pl.nchunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const int64_t n = static_cast<int64_t>(pl.chains) * kD * kD;
    hipLaunchKernelGGL(vla_chunk_scan_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       pl.G, pl.Gpre, pl.Gtot, static_cast<int64_t>(pl.chains), pl.nchunks, pl.nperiods, pl.o, pl.q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(vla_chunk_chain_kernel, dim3(pl.chains * kNdSplit), dim3(kChunkThreads), 0, stream, pl.Gtot,
                     pl.A_init, pl.ND, pl.nperiods, static_cast<double>(pl.eps));
  return hipGetLastError();
}

hipError_t launch_chunk_start(const ChunkPlan& pl, int c_lo, int c_cnt, hipStream_t stream) {
  if (c_cnt <= 0) return hipSuccess;
  hipLaunchKernelGGL(vla_chunk_start_kernel, dim3(static_cast<unsigned>(pl.chains * c_cnt)), dim3(kChunkThreads), 0,
                     stream, pl.Gpre, pl.ND, pl.Ac, pl.chain_info, pl.nchunks, pl.nperiods, pl.o, pl.q, c_lo, c_cnt);
  return hipGetLastError();
}

}  // namespace vla
