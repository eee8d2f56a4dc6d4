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
//   vla_chunk_start_kernel  per chunk, fp64: A_c by Gauss-Jordan elimination
//                           of [ D_c^T | N_p^T ]; a non-positive pivot flags
//                           the chain for the sequential fallback
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
// owns (N, D), adds them.  The period's Gram total is staged in LDS
// (transposed) and the next one is loaded while the current product runs.
constexpr int kNdSplit = 16;
constexpr int kNdCols = kD / kNdSplit;   // 4
// fp64 LDS rows padded to 65 doubles: a column of a row-major 64x64 block
// then spreads over the banks instead of landing on one (transposed stores,
// column reads).
constexpr int kPad = kD + 1;

__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_chain_kernel(const double* __restrict__ Gtot, const float* __restrict__ A0, double* __restrict__ ND,
                       int nperiods, double eps) {
  __shared__ double sG[kD * kPad];          // sG[m*kPad + i] = Gtot[i][m]
  __shared__ double sN[kD * kNdCols];       // sN[m*kNdCols + c] = N[m][c0 + c]
  __shared__ double sP[4][kD * kNdCols];    // partial products of each wave
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
    __syncthreads();   // the previous step is done with sG, sN and sP
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sG[(4 * sc + j) * kPad + 4 * sr + i] = g[4 * i + j];
    if (owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sN[(4 * rb + i) * kNdCols + cc] = N[i];
    }
    __syncthreads();
    load_g(g, p + 2);
    double part[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int m = 16 * q; m < 16 * q + 16; ++m) {
      const double nm = sN[m * kNdCols + cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) part[i] = fma(sG[m * kPad + 4 * rb + i], nm, part[i]);
    }
    if (!owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sP[q][(4 * rb + i) * kNdCols + cc] = part[i];
    }
    __syncthreads();
    if (owner) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (4 * rb + i) * kNdCols + cc;
        Dm[i] += (part[i] + sP[1][e]) + (sP[2][e] + sP[3][e]);
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
// One workgroup per (chain, chunk).  D_c = D_p + Gpre_c N_p, then Gauss-Jordan
// elimination without pivoting turns [ D_c^T | N_p^T ] (64 x 128, thread t
// owning rows 4*(t/16).. and columns 8*(t%16)..) into [ I | A_c^T ].
__global__ void __launch_bounds__(kChunkThreads)
vla_chunk_start_kernel(const double* __restrict__ Gpre, const double* __restrict__ ND, float* __restrict__ Ac,
                       int32_t* __restrict__ chain_info, int nchunks, int nperiods, int o, int q, int c_lo, int c_cnt) {
  // 65 KiB of LDS: Gpre^T and N_p for the product; afterwards the pivot row
  // and column buffers reuse the N_p half, and the result block the first half.
  __shared__ double smem[2 * kD * kPad];
  double* sA = smem;                 // rows of kPad doubles
  double* sB = smem + kD * kPad;
  // Pivot rows at padded positions rbx(j) = j + 2 (j / 32): the 16 threads
  // reading 8-double runs 8 cb + jj at once hit distinct banks.
  double (*rowbuf)[2 * kD + 8] = reinterpret_cast<double (*)[2 * kD + 8]>(sB);
  double (*colbuf)[kD] = reinterpret_cast<double (*)[kD]>(sB + 2 * (2 * kD + 8));
  auto rbx = [](int j) { return j + 2 * (j >> 5); };
  const int64_t chain = blockIdx.x / c_cnt;
  const int c = c_lo + static_cast<int>(blockIdx.x % c_cnt);
  const int p = period_of(c, o, q);
  const int t = threadIdx.x, rb = t >> 4, cb = t & 15;
  const double* Np = ND + (chain * nperiods + p) * 2 * kD * kD;
  const double* Dp = Np + kD * kD;
  const double* gp = Gpre + (chain * nchunks + c) * kD * kD;
  // The first chunk of a period has no Gram prefix: D_c = D_p.
  const bool has_pre = c > 0 && (q == 0 || (o + c) % q != 0);

  for (int e = t; e < kD * kD; e += kChunkThreads) {
    const int i = e / kD, j = e % kD;
    if (has_pre) sA[j * kPad + i] = gp[e];
    sB[i * kPad + j] = Np[e];
  }
  __syncthreads();

  // W[i][j] for i in 4rb..4rb+3, j in 8cb..8cb+7.
  double W[4][8];
  if (cb < 8) {
    // Left block: W[i][j] = D_c[j][i] = D_p[j][i] + sum_m Gpre[j][m] N_p[m][i].
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) W[ii][jj] = Dp[(8 * cb + jj) * kD + 4 * rb + ii];
    for (int m = 0; has_pre && m < kD; ++m) {
      double gv[8], nv[4];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) gv[jj] = sA[m * kPad + 8 * cb + jj];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) nv[ii] = sB[m * kPad + 4 * rb + ii];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) W[ii][jj] = fma(gv[jj], nv[ii], W[ii][jj]);
    }
  } else {
    // Right block: W[i][64 + j] = N_p[j][i].
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) W[ii][jj] = sB[(8 * (cb - 8) + jj) * kPad + 4 * rb + ii];
  }

  __syncthreads();   // every thread is done reading sB before it holds pivots
  // Pivot k = 8 k8 + kk: unrolled over kk, so the pivot row's place in the
  // owner's block (kk % 4) and the pivot column's (kk) are compile-time.
  bool ok = true;
  for (int k8 = 0; k8 < kD / 8; ++k8) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = 8 * k8 + kk;
      const int par = kk & 1;
      const bool row_owner = rb == 2 * k8 + (kk >> 2);
      if (row_owner) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) rowbuf[par][rbx(8 * cb + jj)] = W[kk & 3][jj];
      }
      if (cb == k8) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) colbuf[par][4 * rb + ii] = W[ii][kk];
      }
      __syncthreads();
      const double piv = rowbuf[par][rbx(k)];
      ok = ok && (piv > 0.0) && isfinite(piv);
      // 1/piv: the hardware reciprocal refined by one Newton step.
      double inv = __builtin_amdgcn_rcp(piv);
      inv = fma(inv, fma(-piv, inv, 1.0), inv);
      double rv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) rv[jj] = rowbuf[par][rbx(8 * cb + jj)] * inv;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (row_owner && ii == (kk & 3)) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) W[ii][jj] = rv[jj];
        } else {
          const double f = colbuf[par][4 * rb + ii];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) W[ii][jj] = fma(-f, rv[jj], W[ii][jj]);
        }
      }
    }
  }
  if (!ok && t == 0) atomicOr(chain_info + chain * 4 + kInfoFallback, 1);

  // Symmetrise the result block (A_c^T, equal to A_c in exact arithmetic).
  __syncthreads();
  if (cb >= 8) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) sA[(4 * rb + ii) * kPad + 8 * (cb - 8) + jj] = W[ii][jj];
  }
  __syncthreads();
  float* ac = Ac + (chain * nchunks + c) * kD * kD;
  for (int e = t; e < kD * kD; e += kChunkThreads) {
    const int i = e / kD, j = e % kD;
    ac[e] = static_cast<float>(0.5 * (sA[i * kPad + j] + sA[j * kPad + i]));
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
