// Time-parallel state pass of the residual (delta-rule) update, d = 64.
//
// Method: "Variational Linear Attention: Stable Associative Memory for
// Long-Context Transformers", technical summary 2.3 (recursive update rule):
// S_t = S_{t-1} + e_t alpha_t^T with the prediction error e_t = v_t - S_{t-1} k_hat_t,
// k_hat_t = k_t / |k_t| and the unit gate alpha_t = A_t k_hat_t / |A_t k_hat_t|.
// The gates depend only on the inverse recurrence, so the time-parallel
// inverse pass writes them for every token before this pass runs.
//
// Blocked form over blocks of 64 tokens starting from S_b, the state before
// the block: inside the block S_{t-1} = S_b + sum_{s<t} e_s alpha_s^T, hence
//   e_t + sum_{s<t} (k_hat_t . alpha_s) e_s = v_t - S_b k_hat_t,
// i.e. (I + L) E = V - K_hat S_b^T with L_ts = k_hat_t . alpha_s for s < t
// (strictly lower triangular).  With W = (I + L)^{-1} K_hat and
// U = (I + L)^{-1} V, E = U - W S_b^T and the block's end state is
//   S_{b+1} = S_b + E^T A = S_b (I + N) + Q,   N = -W^T A,  Q = U^T A,
// an affine map of S_b whose coefficients need no state.
//
// Kernels:
//  * vla_res_prep_kernel, parallel over blocks: k_hat, L, W and U by forward
//    substitution (one thread per column), N and Q.  Stores W and U for the
//    readout, N^T as pre-split bf16 matrix-core operands and Q^T in
//    accumulator order for the chain kernel, and the block's key sum.
//  * vla_res_chain_kernel, one workgroup per chain, sequential over blocks:
//    Y_{b+1} = Y_b + N^T Y_b + Q^T for Y = S^T, one 64x64x64 product per
//    block on the bf16 matrix cores with three-term splits of the fp32
//    operands (four waves, one 32x32 tile of Y each; the two waves of a
//    column block swap tiles through LDS).  Stores S_b and the block-start
//    normaliser for the readout.
//  * vla_res_readout_kernel, parallel over blocks: E = U - W S_b^T, then the
//    block's tokens in order, S_t = S_{t-1} + e_t alpha_t^T,
//    o_t = S_t q_t / (n_t . q_t + den_eps) and, with the cap on, |S_t|_F:
//    a token over the cap flags the chain, and the sequential fallback then
//    recomputes it with the cap applied.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_mfma.h"
#include "vla_seq.h"

namespace vla {
namespace {

constexpr int kD = 64;        // head dimension
constexpr int kB = 64;        // tokens per block
constexpr int kP = 68;        // padded LDS row (16-byte aligned rows)
constexpr int kMat = kB * kP; // floats per padded LDS matrix

// ---------------------------------------------------------------------------
// Prep: one workgroup of 256 threads per (chain, block).
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ void __launch_bounds__(256) vla_res_prep_kernel(ResPlan pl, int chains) {
  extern __shared__ float4 smem4[];
  float* sK = reinterpret_cast<float*>(smem4);   // k, then k_hat, then W, then Q
  float* sV = sK + kMat;                         // v, then U
  float* sA = sV + kMat;                         // alpha
  float* sL = sA + kMat;                         // L, then N
  __shared__ float sKinv[kB];

  const int nblk = pl.nblk;
  const int64_t chain = blockIdx.x / nblk;
  const int b = static_cast<int>(blockIdx.x % nblk);
  if (chain >= chains) return;
  const int tid = threadIdx.x;
  const int t0 = b * kB;
  const int nvalid = min(kB, pl.T - t0);
  const int64_t blk = chain * nblk + b;

  const TIn* kg = static_cast<const TIn*>(pl.k) + (chain * pl.T + t0) * kD;
  const TIn* vg = static_cast<const TIn*>(pl.v) + (chain * pl.T + t0) * kD;
  const float* ag = pl.alpha + (chain * pl.T + t0) * kD;
  for (int e = tid; e < kB * kD; e += 256) {
    const int t = e >> 6, j = e & 63;
    float kv = 0.f, vv = 0.f, av = 0.f;
    if (t < nvalid) {
      kv = Elem<TIn>::load(kg + e);
      vv = Elem<TIn>::load(vg + e);
      av = ag[e];
    }
    sK[t * kP + j] = kv;
    sV[t * kP + j] = vv;
    sA[t * kP + j] = av;
  }
  __syncthreads();

  // Key sum (raw features, for the normaliser) and 1 / max(|k_t|, 1e-12).
  if (tid < kD) {
    float s = 0.f;
    for (int t = 0; t < kB; ++t) s += sK[t * kP + tid];
    pl.ksum[blk * kD + tid] = s;
  } else if (tid < kD + kB) {
    const int t = tid - kD;
    float s = 0.f;
    for (int j = 0; j < kD; ++j) s = fmaf(sK[t * kP + j], sK[t * kP + j], s);
    sKinv[t] = 1.f / fmaxf(sqrtf(s), 1e-12f);
  }
  __syncthreads();
  for (int e = tid; e < kB * kD; e += 256) {
    const int t = e >> 6, j = e & 63;
    sK[t * kP + j] *= sKinv[t];
  }
  __syncthreads();

  // L_ts = k_hat_t . alpha_s for s < t, 0 elsewhere.
  {
    const int t = tid >> 2;
#pragma unroll 4
    for (int m = 0; m < 16; ++m) {
      const int s = (tid & 3) + 4 * m;
      float acc = 0.f;
      if (s < t) {
        for (int j = 0; j < kD; ++j) acc = fmaf(sK[t * kP + j], sA[s * kP + j], acc);
      }
      sL[t * kP + s] = acc;
    }
  }
  __syncthreads();

  // (I + L) X = [K_hat | V] by forward substitution, one column per thread.
  if (tid < 2 * kD) {
    float* col = tid < kD ? sK + tid : sV + (tid - kD);
    float x[kB];
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      float acc = col[t * kP];
#pragma unroll
      for (int s = 0; s < t; ++s) acc = fmaf(-sL[t * kP + s], x[s], acc);
      x[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < kB; ++t) col[t * kP] = x[t];
  }
  __syncthreads();

  // W and U to HBM; N = -W^T A and Q = U^T A (rows m, columns (tid & 3) + 4 q).
  for (int e = tid; e < kB * kD; e += 256) {
    const int t = e >> 6, j = e & 63;
    pl.W[blk * kB * kD + e] = sK[t * kP + j];
    pl.U[blk * kB * kD + e] = sV[t * kP + j];
  }
  float nacc[16], qacc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) nacc[q] = qacc[q] = 0.f;
  {
    const int m = tid >> 2;
    for (int t = 0; t < kB; ++t) {
      const float wv = sK[t * kP + m], uv = sV[t * kP + m];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float av = sA[t * kP + (tid & 3) + 4 * q];
        nacc[q] = fmaf(-wv, av, nacc[q]);
        qacc[q] = fmaf(uv, av, qacc[q]);
      }
    }
  }
  __syncthreads();
  {
    const int m = tid >> 2;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      sL[m * kP + (tid & 3) + 4 * q] = nacc[q];
      sK[m * kP + (tid & 3) + 4 * q] = qacc[q];
    }
  }
  __syncthreads();

  // N^T as A operands: fragment (jb, mb, g) of lane l = (h, i) holds
  // N^T[32 jb + i][32 mb + 16 g + 8 (e >> 2) + 4 h + (e & 3)], e = 0..7, the
  // contraction order in which an accumulator tile of Y serves as the B
  // operand (see vla_mfma.h), split into three bf16 terms.
  for (int f = tid; f < 512; f += 256) {
    const int lane = f & 63, g = (f >> 6) & 1, mb = (f >> 7) & 1, jb = (f >> 8) & 1;
    const int h = lane >> 5, i = lane & 31;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int mrow = 32 * mb + 16 * g + 8 * (e >> 2) + 4 * h + (e & 3);
      x[e] = sL[mrow * kP + 32 * jb + i];
    }
    const Split3 sp = split3(x);
    uint4* dst = reinterpret_cast<uint4*>(pl.NTF) + ((((blk * 2 + jb) * 2 + mb) * 2 + g) * 3) * 64 + lane;
    dst[0] = __builtin_bit_cast(uint4, sp.t1);
    dst[64] = __builtin_bit_cast(uint4, sp.t2);
    dst[128] = __builtin_bit_cast(uint4, sp.t3);
  }
  // Q^T in accumulator order: tile w = jb + 2 c, lane l = (h, i), slot s holds
  // Q^T[32 jb + acc_row(s, h)][32 c + i] = Q[32 c + i][32 jb + acc_row(s, h)].
  {
    const int w = tid >> 6, lane = tid & 63, h = lane >> 5, i = lane & 31;
    const int jb = w & 1, c = w >> 1;
    float4* dst = reinterpret_cast<float4*>(pl.QT + ((blk * 4 + w) * 64 + lane) * 16);
    const float* src = sK + (32 * c + i) * kP + 32 * jb + 4 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = *reinterpret_cast<const float4*>(src + 8 * q);
  }
}

// ---------------------------------------------------------------------------
// Chain: one workgroup of four waves per chain.  Wave w owns tile
// (jb, c) = (w & 1, w >> 1) of Y = S^T in accumulator layout: lane l = (h, i),
// slot s holds Y[32 jb + acc_row(s, h)][32 c + i] = S[32 c + i][32 jb + acc_row(s, h)].
// ---------------------------------------------------------------------------
struct ChainOperands {
  uint4 n[2][2][3];   // N^T fragments [mb][g][term]
  float4 q[4];        // Q^T tile
};

__device__ __forceinline__ void load_operands(ChainOperands& op, const ResPlan& pl, int64_t blk, int w, int jb,
                                              int lane) {
  const uint4* nf = reinterpret_cast<const uint4*>(pl.NTF);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int term = 0; term < 3; ++term)
        op.n[mb][g][term] = nf[(((((blk * 2 + jb) * 2 + mb) * 2 + g) * 3 + term) * 64) + lane];
  const float4* qt = reinterpret_cast<const float4*>(pl.QT + ((blk * 4 + w) * 64 + lane) * 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) op.q[q] = qt[q];
}

__global__ void __launch_bounds__(256) vla_res_chain_kernel(ResPlan pl, const float* __restrict__ S_in,
                                                            const float* __restrict__ n_in, float* __restrict__ S_T,
                                                            float* __restrict__ n_T, int32_t* __restrict__ stats,
                                                            const int32_t* __restrict__ chain_info) {
  __shared__ float xbuf[2][4][16][64];   // each wave's Y tile, double-buffered, [slot][lane]
  const int64_t chain = blockIdx.x;
  const int nblk = pl.nblk;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, i = lane & 31;
  const int jb = w & 1, c = w >> 1;
  const int64_t soff = (32 * c + i) * kD + 32 * jb + 4 * h;   // this lane's S entries: soff + 8 q + 0..3

  f32x16 Y;
  {
    const float* src = S_in + chain * kD * kD + soff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(src + 8 * q);
      Y[4 * q] = x.x; Y[4 * q + 1] = x.y; Y[4 * q + 2] = x.z; Y[4 * q + 3] = x.w;
    }
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) xbuf[0][w][s][lane] = Y[s];
  float nval = w == 0 ? n_in[chain * kD + lane] : 0.f;
  ChainOperands cur, nxt;
  if (nblk > 0) load_operands(cur, pl, chain * nblk, w, jb, lane);
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int p = b & 1;
    const int64_t blk = chain * nblk + b;
    f32x16 Yp;
#pragma unroll
    for (int s = 0; s < 16; ++s) Yp[s] = xbuf[p][w ^ 1][s][lane];
    if (b + 1 < nblk) load_operands(nxt, pl, blk + 1, w, jb, lane);
    // The block-start state for the readout.
    {
      float* dst = pl.Ssnap + blk * kD * kD + soff;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 8 * q) = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
    }
    if (w == 0) {
      pl.nblock[blk * kD + lane] = nval;
      nval += pl.ksum[blk * kD + lane];
    }
    // Y + Q^T + N^T Y: contraction block mb uses Y's tile (mb, c), which is
    // this wave's own for mb = jb and its partner's otherwise.
    f32x16 acc0 = Y, acc1 = zero16();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc0[4 * q] += cur.q[q].x; acc0[4 * q + 1] += cur.q[q].y;
      acc0[4 * q + 2] += cur.q[q].z; acc0[4 * q + 3] += cur.q[q].w;
    }
    const f32x16 B0 = jb == 0 ? Y : Yp;
    const f32x16 B1 = jb == 0 ? Yp : Y;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const Split3 b0 = split_slots(B0, g), b1 = split_slots(B1, g);
      Split3 a0, a1;
      a0.t1 = __builtin_bit_cast(bf16x8, cur.n[0][g][0]);
      a0.t2 = __builtin_bit_cast(bf16x8, cur.n[0][g][1]);
      a0.t3 = __builtin_bit_cast(bf16x8, cur.n[0][g][2]);
      a1.t1 = __builtin_bit_cast(bf16x8, cur.n[1][g][0]);
      a1.t2 = __builtin_bit_cast(bf16x8, cur.n[1][g][1]);
      a1.t3 = __builtin_bit_cast(bf16x8, cur.n[1][g][2]);
      acc0 = mma_split(a0, b0, acc0);
      acc1 = mma_split(a1, b1, acc1);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) Y[s] = acc0[s] + acc1[s];
#pragma unroll
    for (int s = 0; s < 16; ++s) xbuf[p ^ 1][w][s][lane] = Y[s];
    if (b + 1 < nblk) cur = nxt;
    __syncthreads();
  }

  bool bad = false;
  {
    float* dst = S_T + chain * kD * kD + soff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
      bad |= !(isfinite(x.x) && isfinite(x.y) && isfinite(x.z) && isfinite(x.w));
      *reinterpret_cast<float4*>(dst + 8 * q) = x;
    }
  }
  if (w == 0) {
    n_T[chain * kD + lane] = nval;
    bad |= !isfinite(nval);
  }
  const bool wave_bad = __any(bad);
  __syncthreads();
  __shared__ int sbad[4];
  if (lane == 0) sbad[w] = wave_bad ? 1 : 0;
  __syncthreads();
  if (tid == 0 && stats) {
    int32_t* s = stats + chain * 4;
    s[0] = chain_info[chain * 4 + kInfoGuard];
    s[1] = 0;
    s[2] = (sbad[0] | sbad[1] | sbad[2] | sbad[3] | chain_info[chain * 4 + kInfoNonfinite]) ? 1 : 0;
    s[3] = -1;
  }
}

// ---------------------------------------------------------------------------
// Readout: one workgroup of 512 threads per (chain, block).  Thread tid owns
// row i = tid >> 3 of S and the columns (tid & 7) + 8 m, m = 0..7.
// ---------------------------------------------------------------------------
template <typename TIn, bool CAP>
__global__ void __launch_bounds__(512) vla_res_readout_kernel(ResPlan pl, float den_eps, float cap2, int chains,
                                                              int32_t* __restrict__ chain_info) {
  extern __shared__ float4 smem4[];
  float* sS = reinterpret_cast<float*>(smem4);   // S_b
  float* sE = sS + kMat;                          // U, then E
  float* sX = sE + kMat;                          // W, then k, then n_t, then o
  float* sA = sX + kMat;                          // alpha
  float* sQ = sA + kMat;                          // q
  __shared__ float sDen[kB];
  __shared__ float sNorm[kB][32];                 // per-token partial |S_t|^2 of each 16-lane row
  __shared__ float sNb[kD];

  const int nblk = pl.nblk;
  const int64_t chain = blockIdx.x / nblk;
  const int b = static_cast<int>(blockIdx.x % nblk);
  if (chain >= chains) return;
  const int tid = threadIdx.x;
  const int t0 = b * kB;
  const int nvalid = min(kB, pl.T - t0);
  const int64_t blk = chain * nblk + b;
  const int64_t tok0 = chain * pl.T + t0;

  // Phase 1: E = U - W S_b^T.
  for (int e = tid; e < kB * kD; e += 512) {
    const int t = e >> 6, j = e & 63;
    sS[t * kP + j] = pl.Ssnap[blk * kD * kD + e];
    sE[t * kP + j] = pl.U[blk * kB * kD + e];
    sX[t * kP + j] = pl.W[blk * kB * kD + e];
  }
  if (tid < kD) sNb[tid] = pl.nblock[blk * kD + tid];
  __syncthreads();
  {
    const int t = tid >> 3;
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = sE[t * kP + (tid & 7) + 8 * m];
    for (int j = 0; j < kD; ++j) {
      const float wv = sX[t * kP + j];
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(-wv, sS[((tid & 7) + 8 * m) * kP + j], acc[m]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) sE[t * kP + (tid & 7) + 8 * m] = acc[m];
  }
  __syncthreads();

  // Phase 2: alpha, q, k; the normalisers n_t = n_b + sum_{s<=t} k_s and the
  // denominators n_t . q_t + den_eps.
  const TIn* qg = static_cast<const TIn*>(pl.q) + tok0 * kD;
  const TIn* kg = static_cast<const TIn*>(pl.k) + tok0 * kD;
  for (int e = tid; e < kB * kD; e += 512) {
    const int t = e >> 6, j = e & 63;
    float qv = 0.f, kv = 0.f, av = 0.f;
    if (t < nvalid) {
      qv = Elem<TIn>::load(qg + e);
      kv = Elem<TIn>::load(kg + e);
      av = pl.alpha[tok0 * kD + e];
    }
    sQ[t * kP + j] = qv;
    sX[t * kP + j] = kv;
    sA[t * kP + j] = av;
  }
  __syncthreads();
  if (tid < kD) {
    float nv = sNb[tid];
    for (int t = 0; t < kB; ++t) {
      nv += sX[t * kP + tid];
      sX[t * kP + tid] = nv;
    }
  }
  __syncthreads();
  {
    const int t = tid >> 3;
    float d = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) d = fmaf(sX[t * kP + (tid & 7) + 8 * m], sQ[t * kP + (tid & 7) + 8 * m], d);
    d = group_sum<8>(d);
    if ((tid & 7) == 0) sDen[t] = d + den_eps;
  }
  __syncthreads();

  // Phase 3: the block's tokens in order.
  const int i = tid >> 3, jc = tid & 7;
  float S[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) S[m] = sS[i * kP + jc + 8 * m];
  bool bad = false;
  for (int t = 0; t < nvalid; ++t) {
    const float ev = sE[t * kP + i];
    float po = 0.f, ns = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      S[m] = fmaf(ev, sA[t * kP + jc + 8 * m], S[m]);
      po = fmaf(S[m], sQ[t * kP + jc + 8 * m], po);
      if constexpr (CAP) ns = fmaf(S[m], S[m], ns);
    }
    po = group_sum<8>(po);
    if (jc == 0) {
      const float ov = po / sDen[t];
      bad |= !isfinite(ov);
      sX[t * kP + i] = ov;
    }
    if constexpr (CAP) {
      ns = group_sum<16>(ns);
      if ((tid & 15) == 0) sNorm[t][tid >> 4] = ns;
    }
  }
  __syncthreads();

  // Outputs, and the cap test on every token's |S_t|_F.
  TIn* og = static_cast<TIn*>(pl.o) + tok0 * kD;
  for (int e = tid; e < nvalid * kD; e += 512) Elem<TIn>::store(og + e, sX[(e >> 6) * kP + (e & 63)]);
  bool over = false;
  if constexpr (CAP) {
    if (tid < nvalid) {
      float ns = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) ns += sNorm[tid][r];
      over = ns > cap2;
    }
  }
  const bool any_over = __any(over), any_bad = __any(bad);
  if ((tid & 63) == 0) {
    if (any_over) atomicOr(chain_info + chain * 4 + kInfoFallback, 1);
    if (any_bad) atomicOr(chain_info + chain * 4 + kInfoNonfinite, 1);
  }
}

template <typename K>
void allow_lds(K kernel, size_t bytes) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes));
}

}  // namespace

hipError_t launch_res_prep(const ResPlan& pl, int chains, hipStream_t stream) {
  const size_t lds = 4 * kMat * sizeof(float);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(chains) * pl.nblk));
  if (pl.bf16) {
    allow_lds(vla_res_prep_kernel<uint16_t>, lds);
    hipLaunchKernelGGL(vla_res_prep_kernel<uint16_t>, grid, dim3(256), lds, stream, pl, chains);
  } else {
    allow_lds(vla_res_prep_kernel<float>, lds);
    hipLaunchKernelGGL(vla_res_prep_kernel<float>, grid, dim3(256), lds, stream, pl, chains);
  }
  return hipGetLastError();
}

hipError_t launch_res_chain(const ResPlan& pl, const float* S_in, const float* n_in, float* S_T, float* n_T,
                            int32_t* stats, const int32_t* chain_info, int chains, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  hipError_t e = hipSuccess;
  if (ev_start && (e = hipEventRecord(ev_start, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(vla_res_chain_kernel, dim3(static_cast<unsigned>(chains)), dim3(256), 0, stream, pl, S_in, n_in,
                     S_T, n_T, stats, chain_info);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_stop) e = hipEventRecord(ev_stop, stream);
  return e;
}

hipError_t launch_res_readout(const ResPlan& pl, float den_eps, float cap, int cap_on, int chains,
                              int32_t* chain_info, hipStream_t stream) {
  const size_t lds = 5 * kMat * sizeof(float);
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(chains) * pl.nblk));
  const float cap2 = cap * cap;
#define VLA_RES_READOUT(T, C)                                                                             \
  do {                                                                                                    \
    allow_lds(vla_res_readout_kernel<T, C>, lds);                                                         \
    hipLaunchKernelGGL((vla_res_readout_kernel<T, C>), grid, dim3(512), lds, stream, pl, den_eps, cap2, chains, \
                       chain_info);                                                                       \
  } while (0)
  if (pl.bf16) {
    if (cap_on) VLA_RES_READOUT(uint16_t, true); else VLA_RES_READOUT(uint16_t, false);
  } else {
    if (cap_on) VLA_RES_READOUT(float, true); else VLA_RES_READOUT(float, false);
  }
#undef VLA_RES_READOUT
  return hipGetLastError();
}

}  // namespace vla
