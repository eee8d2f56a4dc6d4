// Time-parallel ("chunked") schedule of the VLA inverse recurrence, d = 64
// and d = 128.
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
//                           each period's total, in parallel over periods and
//                           elements
//   vla_chunk_chain_kernel  per chain and column block, sequential over
//                           periods, fp64: (N, D) at every period start
//   vla_chunk_start_kernel  per chunk, fp64: A_c by blocked Gauss-Jordan
//                           elimination of [ D_c^T | N_p^T ] on the fp64
//                           matrix cores; a non-positive pivot flags the
//                           chain for the sequential fallback
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_wide.h"
#include "vla_seq.h"

namespace vla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;            // head dimension of this schedule
constexpr int kChunkThreads = 256;

template <int D>
__global__ void snapshot_kernel(const float* __restrict__ A0, const float* __restrict__ S0,
                                const float* __restrict__ n0, float* __restrict__ A_copy,
                                float* __restrict__ S_copy, float* __restrict__ n_copy,
                                int32_t* __restrict__ chain_info, int64_t chains) {
  const int64_t mat = chains * D * D;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < mat;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = i % (D * D);
    A_copy[i] = A0 ? A0[i] : ((e / D) == (e % D) ? 1.f : 0.f);
    S_copy[i] = S0 ? S0[i] : 0.f;
    if (i < chains * D) n_copy[i] = n0 ? n0[i] : 0.f;
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
// the whole period's sum.  One thread per (chain, period, matrix element),
// sequential over the period's chunks.  A period's first chunk has no prefix
// (the chunk-start kernels read none for it), so nothing is written there.
template <int D>
__global__ void __launch_bounds__(256)
vla_chunk_scan_kernel(const float* __restrict__ G, double* __restrict__ Gpre, double* __restrict__ Gtot,
                      int nchunks, int nperiods, int o, int q) {
  // Grid: x = (chain, period), y = slices of 1024 matrix elements, four
  // consecutive ones per thread (one 16-byte load per chunk), so the bases
  // below are wave-uniform and each wave keeps 4 KiB of loads in flight.
  const int64_t cp = blockIdx.x;
  const int p = static_cast<int>(cp % nperiods);
  const int64_t chain = cp / nperiods;
  const int e = 4 * (blockIdx.y * 256 + threadIdx.x);
  // Chunks of period p: those c with period_of(c) = p.
  int c_lo = 0, c_hi = nchunks;
  if (q > 0) {
    const int base = (o / q + p) * q - o;
    c_lo = max(0, base);
    c_hi = min(nchunks, base + q);
  }
  const float* g = G + (chain * nchunks + c_lo) * D * D + e;
  double* gp = Gpre + (chain * nchunks + c_lo) * D * D + e;
  const int n = c_hi - c_lo;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i0 = 0; i0 < n; i0 += 4) {
    float4 gv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      gv[k] = i0 + k < n ? *reinterpret_cast<const float4*>(g + static_cast<int64_t>(i0 + k) * D * D)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = i0 + k;
      if (i < n) {
        if (i > 0) {
          double2* dst = reinterpret_cast<double2*>(gp + static_cast<int64_t>(i) * D * D);
          dst[0] = make_double2(acc[0], acc[1]);
          dst[1] = make_double2(acc[2], acc[3]);
        }
        acc[0] += static_cast<double>(gv[k].x);
        acc[1] += static_cast<double>(gv[k].y);
        acc[2] += static_cast<double>(gv[k].z);
        acc[3] += static_cast<double>(gv[k].w);
      }
    }
  }
  double2* dt = reinterpret_cast<double2*>(Gtot + cp * D * D + e);
  dt[0] = make_double2(acc[0], acc[1]);
  dt[1] = make_double2(acc[2], acc[3]);
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
// Row stride (doubles) of the finished panel rows R with NT tiles per row.
template <int NT>
constexpr int rpad() { return 16 * NT + 1; }
constexpr int kRPad = rpad<8>();

// Panel P of the elimination (compile time, so every tile index is too).
// Wave P inverts its pivot block W11 by Gauss-Jordan on [ W11 | I ] (one
// pivot at a time, two tiles), then forms R = W11^-1 W[panel rows] for the
// tiles right of the panel on the matrix cores; the other waves subtract
// C_w R.  sI is the wave's 16 x 17 staging tile for transposed operand reads.
template <int NT, int P>
__device__ __forceinline__ void gj_panel(d4 (&W)[NT], int w, int g, int col, double* sR, double* sI, bool& ok) {
  constexpr int kRP = rpad<NT>();
  if (w == P) {   // wave-uniform
    d4 inv_t;     // becomes W11^-1
#pragma unroll
    for (int i = 0; i < 4; ++i) inv_t[i] = (4 * i + g == col) ? 1.0 : 0.0;
    auto rcp64 = [](double x) {   // the hardware reciprocal refined by one Newton step
      const double r = __builtin_amdgcn_rcp(x);
      return fma(r, fma(-x, r, 1.0), r);
    };
    // Two pivots per round of cross-lane reads.  Row k of the block sits in
    // lanes 16 (k % 4) .., slot k / 4 (rows k and k + 1 share the slot); the
    // lanes fetch columns k and k + 1 of their rows and rows k and k + 1 at
    // their column as they stand before pivot k, then apply pivot k to their
    // copies of column and row k + 1 themselves (the same operations, in the
    // same order, as one pivot at a time).
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      const int sk = k >> 2, lk = 16 * (k & 3), lk1 = 16 * ((k + 1) & 3);
      const double pa = readlane_d(W[P][sk], lk + k), pb = readlane_d(W[P][sk], lk + k + 1);
      const double pc = readlane_d(W[P][sk], lk1 + k), pd = readlane_d(W[P][sk], lk1 + k + 1);
      double fk[4], fk1[4];   // columns k and k + 1 of this lane's rows 4 i + g
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fk[i] = __shfl(W[P][i], 16 * g + k, 64);
        fk1[i] = __shfl(W[P][i], 16 * g + k + 1, 64);
      }
      const double Rk = __shfl(W[P][sk], lk + col, 64), Rk1 = __shfl(W[P][sk], lk1 + col, 64);
      const double Ik = __shfl(inv_t[sk], lk + col, 64), Ik1 = __shfl(inv_t[sk], lk1 + col, 64);
      ok = ok && (pa > 0.0) && isfinite(pa);
      const double ia = rcp64(pa);
      const double ra = Rk * ia, rb = Ik * ia;       // row k after pivot k
      const double bk = pb * ia;                      // its entry in column k + 1
      const double pd1 = fma(-pc, bk, pd);            // pivot k + 1 after pivot k
      ok = ok && (pd1 > 0.0) && isfinite(pd1);
      const double id = rcp64(pd1);
      const double sa = fma(-pc, ra, Rk1) * id, sb = fma(-pc, rb, Ik1) * id;   // row k + 1 after both
      const double ra2 = fma(-bk, sa, ra), rb2 = fma(-bk, sb, rb);             // row k after both
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + g;
        const double fk1p = fma(-fk[i], bk, fk1[i]);   // column k + 1 after pivot k
        const double w1 = fma(-fk[i], ra, W[P][i]), v1 = fma(-fk[i], rb, inv_t[i]);
        W[P][i] = row == k ? ra2 : (row == k + 1 ? sa : fma(-fk1p, sa, w1));
        inv_t[i] = row == k ? rb2 : (row == k + 1 ? sb : fma(-fk1p, sb, v1));
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
    for (int ct = P + 1; ct < NT; ++ct) {
      d4 r = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) r = mfma64(a[kk], W[ct][kk], r);
      W[ct] = r;
#pragma unroll
      for (int i = 0; i < 4; ++i) sR[(4 * i + g) * kRP + 16 * ct + col] = r[i];
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
    for (int ct = P + 1; ct < NT; ++ct)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) W[ct] = mfma64(a[kk], sR[(4 * kk + g) * kRP + 16 * ct + col], W[ct]);
  }
  __syncthreads();   // sR and sI are rewritten by the next panel
}

__global__ void __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(2)))
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
  gj_panel<8, 0>(W, w, g, col, sR, sI, ok);
  gj_panel<8, 1>(W, w, g, col, sR, sI, ok);
  gj_panel<8, 2>(W, w, g, col, sR, sI, ok);
  gj_panel<8, 3>(W, w, g, col, sR, sI, ok);
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

// ---- d = 128 ---------------------------------------------------------------
// Gram matrices (bf16 storage): wave w accumulates the 32 x 32 tiles of row
// block w, all four column blocks.  The rows of u pass through LDS transposed
// (ut[column][row]), 64 rows at a time, so each operand is one 16-byte read
// of eight consecutive rows of one column; the next 64 rows are loaded while
// the current ones are multiplied.
constexpr int kG128Rows = 64;
constexpr int kG128Ld = kG128Rows + 8;   // bf16 per LDS row: 144 bytes

__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_gram128_kernel(const uint16_t* __restrict__ u, float* __restrict__ G, int T, int r, int L, int nchunks) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint16_t ut[2][D * kG128Ld];
  const int64_t chain = blockIdx.x / nchunks;
  const int c = blockIdx.x % nchunks;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
  const int t_lo = c * L, t_hi = min(T, t_lo + L);
  const int nrows = (t_hi - t_lo) * r;
  const uint16_t* U = u + (chain * T + t_lo) * static_cast<int64_t>(r) * D;
  // Thread (row lr of the group, 16-byte pieces lp .. lp + 3 of that row);
  // loads run two groups ahead of the products (two register sets).
  const int lr = tid & 63, lp = (tid >> 6) * 4;
  uint4 reg[2][4];
  auto load = [&](int k0, uint4 (&rg)[4]) {
    const int k = k0 + lr;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rg[j] = k < nrows ? *reinterpret_cast<const uint4*>(U + static_cast<int64_t>(k) * D + 8 * (lp + j))
                        : make_uint4(0, 0, 0, 0);
  };
  auto store = [&](uint16_t* dst, const uint4 (&rg)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wv[4] = {rg[j].x, rg[j].y, rg[j].z, rg[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dst[(8 * (lp + j) + e) * kG128Ld + lr] = static_cast<uint16_t>(e & 1 ? wv[e >> 1] >> 16 : wv[e >> 1]);
    }
  };
  f32x16 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
    acc[jb] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int ngroups = (nrows + kG128Rows - 1) / kG128Rows;
  if (ngroups > 0) {
    load(0, reg[0]);
    if (ngroups > 1) load(kG128Rows, reg[1]);
    store(ut[0], reg[0]);
  }
  __syncthreads();
  auto group = [&](int gi, const uint4 (&nxt)[4], uint4 (&fut)[4]) {
    // Group gi + 1's rows are in nxt; group gi + 2's go into fut, the set
    // gi's rows came from (stored to LDS in the previous step).
    if (gi + 2 < ngroups) load((gi + 2) * kG128Rows, fut);
    const uint16_t* cur = ut[gi & 1];
#pragma unroll
    for (int kk = 0; kk < kG128Rows / 16; ++kk) {
      const int off = 16 * kk + 8 * h;
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(cur + (32 * w + c32) * kG128Ld + off));
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const bf16x8 b =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(cur + (32 * jb + c32) * kG128Ld + off));
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[jb], 0, 0, 0);
      }
    }
    if (gi + 1 < ngroups) store(ut[(gi + 1) & 1], nxt);
    __syncthreads();
  };
  for (int gi = 0; gi < ngroups; gi += 2) {
    group(gi, reg[1], reg[0]);
    if (gi + 1 < ngroups) group(gi + 1, reg[0], reg[1]);
  }
  float* gout = G + (chain * nchunks + c) * D * D;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int sl = 0; sl < 16; ++sl) {
      const int row = 32 * w + 8 * (sl / 4) + 4 * h + (sl % 4);
      gout[row * D + 32 * jb + c32] = acc[jb][sl];
    }
}

// (N, D) chain on the fp64 matrix cores.  One workgroup (four waves) per
// chain and block of 32 columns; wave w owns rows 32 w .. 32 w + 31 of the
// block's N and D as 16 x 16 tiles [row tile a][column tile b], slot i of
// lane (g, col) at row 32 w + 16 a + 4 i + g, column c0 + 16 b + col.  Per
// period D += Gtot_p N: the A operand Gtot[i][m] is read as Gtot[m][i]
// (symmetric: rows of 16 consecutive doubles) from global memory, where the
// chain's four workgroups share it through L2; the B operand N comes from
// LDS, whose two buffers alternate between periods (one barrier a period).
constexpr int kNd128Cols = 32;
constexpr int kNd128Ld = kNd128Cols + 2;

__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_chain128_kernel(const double* __restrict__ Gtot, const float* __restrict__ A0, double* __restrict__ ND,
                          int nperiods, double eps) {
  constexpr int D = 128;
  __shared__ double sN[2][D * kNd128Ld];
  const int64_t chain = blockIdx.x / (D / kNd128Cols);
  const int c0 = (blockIdx.x % (D / kNd128Cols)) * kNd128Cols;
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  d4 N[2][2], Dm[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 16 * a + 4 * i + g, cc = c0 + 16 * b + col;
        N[a][b][i] = static_cast<double>(A0[(chain * D + row) * D + cc]);
        Dm[a][b][i] = row == cc ? 1.0 : 0.0;
      }
  auto store_nd = [&](int p) {
    double* nd = ND + (chain * nperiods + p) * 2 * D * D;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = (32 * w + 16 * a + 4 * i + g) * D + c0 + 16 * b + col;
          nd[e] = N[a][b][i];
          nd[D * D + e] = Dm[a][b][i];
        }
  };
  auto put_n = [&](double* buf) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[(32 * w + 16 * a + 4 * i + g) * kNd128Ld + 16 * b + col] = N[a][b][i];
  };
  store_nd(0);
  put_n(sN[0]);
  __syncthreads();
  for (int p = 0; p + 1 < nperiods; ++p) {
    const double* gt = Gtot + (chain * nperiods + p) * D * D;
    const double* Ns = sN[p & 1];
#pragma unroll 8
    for (int kk = 0; kk < D / 4; ++kk) {
      const double* grow = gt + (4 * kk + g) * D + 32 * w + col;
      const double ga0 = grow[0], ga1 = grow[16];
      const double nb0 = Ns[(4 * kk + g) * kNd128Ld + col], nb1 = Ns[(4 * kk + g) * kNd128Ld + 16 + col];
      Dm[0][0] = mfma64(ga0, nb0, Dm[0][0]);
      Dm[0][1] = mfma64(ga0, nb1, Dm[0][1]);
      Dm[1][0] = mfma64(ga1, nb0, Dm[1][0]);
      Dm[1][1] = mfma64(ga1, nb1, Dm[1][1]);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) N[a][b][i] = fma(eps, Dm[a][b][i], N[a][b][i]);
    store_nd(p + 1);
    // Buffer (p + 1) & 1 was last read in period p - 1, before the previous barrier.
    put_n(sN[(p + 1) & 1]);
    __syncthreads();
  }
}

// Chunk-start inverses: eight waves per (chain, chunk); wave w holds rows
// 16 w .. 16 w + 15 of W = [ D_c^T | N_p^T ] (128 x 256) as sixteen 16 x 16
// tiles, read from global memory; D_c^T = D_p^T + N_p^T Gpre_c (Gpre_c
// symmetric) on the fp64 matrix cores, then the elimination of the d = 64
// kernel with eight panels.  LDS: the panel rows R (16 x 257) and each wave's
// staging tile (16 x 17), and afterwards the result block in fp32 (128 x 129)
// over them.
constexpr int kStart128Threads = 512;
constexpr int kStart128Lds = 128 * 129 * 4 > (16 * rpad<16>() + 8 * 16 * 17) * 8 ? 128 * 129 * 4
                                                                                 : (16 * rpad<16>() + 8 * 16 * 17) * 8;

__global__ void __launch_bounds__(kStart128Threads)
vla_chunk_start128_kernel(const double* __restrict__ Gpre, const double* __restrict__ ND, float* __restrict__ Ac,
                          int32_t* __restrict__ chain_info, int nchunks, int nperiods, int o, int q, int c_lo,
                          int c_cnt, int c_step) {
  constexpr int D = 128, NT = 16;
  __shared__ double smem[kStart128Lds / 8];
  const int64_t chain = blockIdx.x / c_cnt;
  const int c = (c_lo + static_cast<int>(blockIdx.x % c_cnt)) * c_step;
  const int p = period_of(c, o, q);
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, col = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const double* Np = ND + (chain * nperiods + p) * 2 * D * D;
  const double* Dp = Np + D * D;
  const double* gp = Gpre + (chain * nchunks + c) * D * D;
  const bool has_pre = c > 0 && (q == 0 || (o + c) % q != 0);

  // W[ct] slot i: row 16 w + 4 i + g, column 16 ct + col; the transposes
  // are read directly (left: D_p[col'][row'], right: N_p[col'][row']).
  d4 W[NT];
#pragma unroll
  for (int ct = 0; ct < NT / 2; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (16 * ct + col) * D + 16 * w + 4 * i + g;
      W[ct][i] = Dp[e];
      W[NT / 2 + ct][i] = Np[e];
    }
  if (has_pre) {
#pragma unroll 2
    for (int kk = 0; kk < D / 4; ++kk) {
      const double a = Np[(4 * kk + g) * D + 16 * w + col];
      const double* grow = gp + (4 * kk + g) * D + col;
#pragma unroll
      for (int ct = 0; ct < NT / 2; ++ct) W[ct] = mfma64(a, grow[16 * ct], W[ct]);
    }
  }

  bool ok = true;
  double* sR = smem;
  double* sI = smem + 16 * rpad<NT>() + w * 16 * 17;
  gj_panel<NT, 0>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 1>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 2>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 3>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 4>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 5>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 6>(W, w, g, col, sR, sI, ok);
  gj_panel<NT, 7>(W, w, g, col, sR, sI, ok);
  if (!ok && lane == 0) atomicOr(chain_info + chain * 4 + kInfoFallback, 1);

  // The result block (A_c^T, equal to A_c in exact arithmetic), symmetrised
  // in fp32 (the last panel's barrier freed the LDS).
  float* sF = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int qb = 0; qb < NT / 2; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) sF[(16 * w + 4 * i + g) * (D + 1) + 16 * qb + col] = static_cast<float>(W[NT / 2 + qb][i]);
  __syncthreads();
  float* ac = Ac + (chain * nchunks + c) * D * D;
  for (int e = t; e < D * D; e += kStart128Threads) {
    const int i = e / D, j = e % D;
    ac[e] = 0.5f * (sF[i * (D + 1) + j] + sF[j * (D + 1) + i]);
  }
}

}  // namespace

hipError_t launch_chunk_prologue(const ChunkPlan& pl, const float* A0, const float* S0, const float* n0,
                                 const void* u, bool bf16, hipStream_t stream) {
  if (pl.d != kD && !(pl.d == 128 && bf16)) return hipErrorInvalidValue;
  const int64_t mat = static_cast<int64_t>(pl.chains) * pl.d * pl.d;
  const int64_t want = (mat + 255) / 256;
  const unsigned sgrid = static_cast<unsigned>(want < 4096 ? want : 4096);
  if (pl.d == 128)
    hipLaunchKernelGGL(snapshot_kernel<128>, dim3(sgrid), dim3(256), 0, stream, A0, S0, n0, pl.A_init, pl.S_init,
                       pl.n_init, pl.chain_info, static_cast<int64_t>(pl.chains));
  else
    hipLaunchKernelGGL(snapshot_kernel<kD>, dim3(sgrid), dim3(256), 0, stream, A0, S0, n0, pl.A_init, pl.S_init,
                       pl.n_init, pl.chain_info, static_cast<int64_t>(pl.chains));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned units = static_cast<unsigned>(pl.chains * pl.nchunks);
  if (pl.d == 128) {
    hipLaunchKernelGGL(vla_chunk_gram128_kernel, dim3(units), dim3(kChunkThreads), 0, stream,
                       static_cast<const uint16_t*>(u), pl.G, pl.T, pl.r, pl.L, pl.nchunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(vla_chunk_scan_kernel<128>, dim3(static_cast<unsigned>(pl.chains * pl.nperiods), 128 * 128 / 1024),
                       dim3(256), 0, stream, pl.G, pl.Gpre, pl.Gtot, pl.nchunks, pl.nperiods, pl.o, pl.q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(vla_chunk_chain128_kernel, dim3(pl.chains * (128 / kNd128Cols)), dim3(kChunkThreads), 0, stream,
                       pl.Gtot, pl.A_init, pl.ND, pl.nperiods, static_cast<double>(pl.eps));
    return hipGetLastError();
  }
  if (bf16)
    hipLaunchKernelGGL(vla_chunk_gram_kernel<uint16_t>, dim3(units), dim3(kChunkThreads), 0, stream,
                       static_cast<const uint16_t*>(u), pl.G, pl.T, pl.r, pl.L, pl.nchunks);
  else
    hipLaunchKernelGGL(vla_chunk_gram_kernel<float>, dim3(units), dim3(kChunkThreads), 0, stream,
                       static_cast<const float*>(u), pl.G, pl.T, pl.r, pl.L, pl.nchunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    hipLaunchKernelGGL(vla_chunk_scan_kernel<kD>, dim3(static_cast<unsigned>(pl.chains * pl.nperiods), kD * kD / 1024),
                       dim3(256), 0, stream, pl.G, pl.Gpre, pl.Gtot, pl.nchunks, pl.nperiods, pl.o, pl.q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(vla_chunk_chain_kernel, dim3(pl.chains * kNdSplit), dim3(kChunkThreads), 0, stream, pl.Gtot,
                     pl.A_init, pl.ND, pl.nperiods, static_cast<double>(pl.eps));
  return hipGetLastError();
}

hipError_t launch_chunk_start128(const ChunkPlan& pl, int c_lo, int c_cnt, int c_step, hipStream_t stream) {
  if (c_cnt <= 0) return hipSuccess;
  if (pl.d != 128 || c_step < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vla_chunk_start128_kernel, dim3(static_cast<unsigned>(pl.chains * c_cnt)), dim3(kStart128Threads),
                     0, stream, pl.Gpre, pl.ND, pl.Ac, pl.chain_info, pl.nchunks, pl.nperiods, pl.o, pl.q, c_lo, c_cnt,
                     c_step);
  return hipGetLastError();
}

hipError_t launch_chunk_start(const ChunkPlan& pl, int c_lo, int c_cnt, hipStream_t stream) {
  if (c_cnt <= 0) return hipSuccess;
  if (pl.d == 128) return launch_chunk_start128(pl, c_lo, c_cnt, 1, stream);
  hipLaunchKernelGGL(vla_chunk_start_kernel, dim3(static_cast<unsigned>(pl.chains * c_cnt)), dim3(kChunkThreads), 0,
                     stream, pl.Gpre, pl.ND, pl.Ac, pl.chain_info, pl.nchunks, pl.nperiods, pl.o, pl.q, c_lo, c_cnt);
  return hipGetLastError();
}

}  // namespace vla
