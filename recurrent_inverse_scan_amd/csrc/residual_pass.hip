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
//  * vla_res_prep_kernel, parallel over blocks: k_hat, L (matrix cores), W
//    and U by forward substitution (one thread per column), N and Q (matrix
//    cores).  Stores W and U for the readout, N^T as pre-split bf16
//    matrix-core operands and Q^T in accumulator order for the chain kernel,
//    and the block's key sum.
//  * vla_res_chain_kernel, one workgroup per chain, sequential over blocks:
//    Y_{b+1} = Y_b + N^T Y_b + Q^T for Y = S^T, one 64x64x64 product per
//    block on the bf16 matrix cores with three-term splits of the fp32
//    operands (four waves, one 32x32 tile of Y each; the two waves of a
//    column block swap tiles through LDS).  Stores S_b for the readout; a
//    small kernel beside it sums the key sums into block-start normalisers.
//  * vla_res_readout_kernel, parallel over blocks: E = U - W S_b^T, then the
//    block's tokens in order, S_t = S_{t-1} + e_t alpha_t^T,
//    o_t = S_t q_t / (n_t . q_t + den_eps) and, with the cap on, |S_t|_F:
//    a token over the cap flags the chain, and the sequential fallback then
//    recomputes it with the cap applied, from the start of the chunk that
//    holds the chain's first such token (the state there is exact: no token
//    before it was over the cap).
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_residual.h"
#include "vla_mfma.h"
#include "vla_seq.h"

namespace vla {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 64;        // head dimension
constexpr int kB = 64;        // tokens per block
constexpr int kP = 68;        // padded LDS row (16-byte aligned rows)
constexpr int kMat = kB * kP; // floats per padded LDS matrix

// 8 consecutive floats of a padded LDS row as a three-term split, and 8
// entries of a column (rows r0 .. r0 + 7, column c), optionally negated.
__device__ __forceinline__ Split3 row_frag(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return split3(x);
}
__device__ __forceinline__ Split3 col_frag(const float* m, int r0, int c, float sign) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = sign * m[(r0 + e) * kP + c];
  return split3(x);
}

// ---------------------------------------------------------------------------
// Prep: one workgroup of 256 threads per (chain, block).
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ void __launch_bounds__(256) vla_res_prep_kernel(ResPlan pl, int chains, int b_lo, int nb) {
  extern __shared__ float4 smem4[];
  float* sK = reinterpret_cast<float*>(smem4);   // k, then k_hat, then W, then Q
  float* sV = sK + kMat;                         // v, then U
  float* sA = sV + kMat;                         // alpha
  float* sL = sA + kMat;                         // L, then N
  __shared__ float sKinv[kB];

  const int nblk = pl.nblk;
  // Blocks [b_lo, b_lo + nb) of every chain, grid-stride.
  for (int64_t x = blockIdx.x; x < static_cast<int64_t>(chains) * nb; x += gridDim.x) {
  const int64_t chain = x / nb;
  const int b = b_lo + static_cast<int>(x % nb);
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

  // L_ts = k_hat_t . alpha_s for s < t (the strictly lower tiles (tb, sb) =
  // (0, 0), (1, 0), (1, 1), one per wave, on the matrix cores).
  const int wv = tid >> 6, ln = tid & 63, lh = ln >> 5, li = ln & 31;
  if (wv < 3) {
    const int tb = wv == 0 ? 0 : 1, sb = wv == 2 ? 1 : 0;
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const Split3 a = row_frag(sK + (32 * tb + li) * kP + 16 * ks + 8 * lh);
      const Split3 bb = row_frag(sA + (32 * sb + li) * kP + 16 * ks + 8 * lh);
      acc = mma_split(a, bb, acc);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int t = 32 * tb + acc_row(s, lh), sc = 32 * sb + li;
      sL[t * kP + sc] = t > sc ? acc[s] : 0.f;
    }
  }
  __syncthreads();

  // (I + L) X = [K_hat | V] by forward substitution, one column per thread.
  if (tid < 2 * kD) {
    float* col = tid < kD ? sK + tid : sV + (tid - kD);
    float x[kB];
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      // Four interleaved partial sums keep the FMAs independent.
      float acc[4] = {col[t * kP], 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < t; ++s) acc[s & 3] = fmaf(-sL[t * kP + s], x[s], acc[s & 3]);
      x[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
#pragma unroll
    for (int t = 0; t < kB; ++t) col[t * kP] = x[t];
  }
  __syncthreads();

  // W and U to HBM for the readout.
  for (int e = tid; e < kB * kD; e += 256) {
    const int t = e >> 6, j = e & 63;
    pl.W[blk * kB * kD + e] = sK[t * kP + j];
    pl.U[blk * kB * kD + e] = sV[t * kP + j];
  }
  // N = -W^T A (tile (mb, jb) = (wv >> 1, wv & 1)) and Q^T = A^T U (tile
  // (jb, c) = (wv & 1, wv >> 1)) on the matrix cores, contracting over the
  // block's tokens.  A lane's column fragment of A serves as the B operand of
  // the first and the A operand of the second.  In accumulator layout N's
  // tile is already N^T's A-operand fragments for the chain kernel (slots
  // 8 g .. 8 g + 7 are contraction step g) and Q^T's tile is its
  // accumulator tile: both go to HBM from registers.
  {
    const int mb = wv >> 1, jb = wv & 1;
    f32x16 aN = zero16(), aQ = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r0 = 16 * ks + 8 * lh;
      const Split3 fw = col_frag(sK, r0, 32 * mb + li, -1.f);
      const Split3 fu = col_frag(sV, r0, 32 * mb + li, 1.f);
      const Split3 fa = col_frag(sA, r0, 32 * jb + li, 1.f);
      aN = mma_split(fw, fa, aN);
      aQ = mma_split(fa, fu, aQ);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const Split3 sp = split_slots(aN, g);
      uint4* dst = reinterpret_cast<uint4*>(pl.NTF) + ((((blk * 2 + jb) * 2 + mb) * 2 + g) * 3) * 64 + ln;
      dst[0] = __builtin_bit_cast(uint4, sp.t1);
      dst[64] = __builtin_bit_cast(uint4, sp.t2);
      dst[128] = __builtin_bit_cast(uint4, sp.t3);
    }
    float4* qdst = reinterpret_cast<float4*>(pl.QT + blk * kD * kD) + wv * 256 + ln;
#pragma unroll
    for (int q = 0; q < 4; ++q) qdst[64 * q] = make_float4(aQ[4 * q], aQ[4 * q + 1], aQ[4 * q + 2], aQ[4 * q + 3]);
  }
  __syncthreads();   // the next block overwrites the LDS this one read last
  }
}

// ---------------------------------------------------------------------------
// Chain: one workgroup of four waves per chain.  Wave w owns tile
// (jb, c) = (w & 1, w >> 1) of Y = S^T in accumulator layout: lane l = (h, i),
// slot s holds Y[32 jb + acc_row(s, h)][32 c + i] = S[32 c + i][32 jb + acc_row(s, h)].
//
// A block's operands (N^T fragments of both row blocks, 24 KiB, and Q^T,
// 16 KiB) travel by buffer-to-LDS copies into a three-slot ring, issued two
// blocks ahead, ten 1 KiB pieces per wave.  Each wave waits for its own copies
// of the next block with a counted s_waitcnt before the block's closing
// barrier (a bare s_barrier: __syncthreads would also drain the copies
// issued for the block after); per block a wave issues exactly ten copies and
// four stores, so the copies for block b + 1, issued during block b - 1, are
// complete once at most 14 of its memory operations are outstanding at the
// end of block b.
// ---------------------------------------------------------------------------
constexpr int kRing = 3;
constexpr int kSlotBytes = 40 * 1024;       // N^T fragments (24 KiB), then Q^T (16 KiB)
constexpr int kSlotVecs = kSlotBytes / 16;
constexpr int kXFloats = 4 * 16 * 64;       // each wave's Y tile, [wave][slot][lane]

__device__ __forceinline__ void ring_copy(const ResPlan& pl, uint4 (&slot)[kSlotVecs], int64_t blk, int w, int lane) {
  const auto rn = make_rsrc(pl.NTF + blk * 3 * kD * kD, 24 * 1024);
  const auto rq = make_rsrc(pl.QT + blk * kD * kD, 16 * 1024);
  char* base = reinterpret_cast<char*>(slot);
#pragma unroll
  for (int k = 0; k < 10; ++k) {
    const int p = 10 * w + k;
    if (p < 24) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rn, (lds_void*)(base + 1024 * p), 16, 16 * lane, 1024 * p, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(base + 1024 * p), 16, 16 * lane, 1024 * (p - 24), 0,
                                               0);
    }
  }
}

struct ChainLane {
  int64_t chain, soff;
  int nblk, nb, b_lo, w, lane, jb;   // nb blocks from b_lo in this segment
};

// Block lb of the segment (block b_lo + lb): copies for block lb + 2 into
// `ahead`, operands from `cur`, the partner's tile from `xr`, this wave's new
// tile to `xw`.  Distinct LDS objects let the compiler see that reading `cur`
// does not wait for the copies into `ahead`.
__device__ __forceinline__ void chain_block(const ResPlan& pl, const ChainLane& cl, int lb, f32x16& Y,
                                            uint4 (&cur)[kSlotVecs], uint4 (&ahead)[kSlotVecs],
                                            const float (&xr)[kXFloats], float (&xw)[kXFloats]) {
  const int w = cl.w, lane = cl.lane, jb = cl.jb, nb = cl.nb;
  const int64_t blk = cl.chain * cl.nblk + cl.b_lo + lb;
  if (lb + 2 < nb) ring_copy(pl, ahead, blk + 2, w, lane);
  f32x16 Yp;
#pragma unroll
  for (int s = 0; s < 16; ++s) Yp[s] = xr[((w ^ 1) * 16 + s) * 64 + lane];
  // The block-start state for the readout.
  {
    float* dst = pl.Ssnap + blk * kD * kD + cl.soff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + 8 * q) = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
  }
  // Y + Q^T + N^T Y: contraction block mb = jb pairs with this wave's own
  // tile, mb = 1 - jb with its partner's.
  const float4* qt = reinterpret_cast<const float4*>(cur + 24 * 64) + w * 256 + lane;
  f32x16 acc0 = Y, acc1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = qt[64 * q];
    acc1[4 * q] = x.x; acc1[4 * q + 1] = x.y; acc1[4 * q + 2] = x.z; acc1[4 * q + 3] = x.w;
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const Split3 b0 = split_slots(Y, g), b1 = split_slots(Yp, g);
    Split3 a0, a1;
    const int f0 = ((jb * 2 + jb) * 2 + g) * 3, f1 = ((jb * 2 + (1 - jb)) * 2 + g) * 3;
    a0.t1 = __builtin_bit_cast(bf16x8, cur[(f0 + 0) * 64 + lane]);
    a0.t2 = __builtin_bit_cast(bf16x8, cur[(f0 + 1) * 64 + lane]);
    a0.t3 = __builtin_bit_cast(bf16x8, cur[(f0 + 2) * 64 + lane]);
    a1.t1 = __builtin_bit_cast(bf16x8, cur[(f1 + 0) * 64 + lane]);
    a1.t2 = __builtin_bit_cast(bf16x8, cur[(f1 + 1) * 64 + lane]);
    a1.t3 = __builtin_bit_cast(bf16x8, cur[(f1 + 2) * 64 + lane]);
    acc0 = mma_split(a0, b0, acc0);
    acc1 = mma_split(a1, b1, acc1);
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) Y[s] = acc0[s] + acc1[s];
#pragma unroll
  for (int s = 0; s < 16; ++s) xw[(w * 16 + s) * 64 + lane] = Y[s];
  // The next block's operands (copied during block b - 1) have landed once
  // at most this block's ten copies and four stores are outstanding, in
  // whichever order the two were issued.
  if (lb >= 1 && lb + 2 < nb)
    asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Segment [b_lo, b_hi) from S_in (chain c at S_in + c * S_in_stride).  The
// last segment writes S_T and stats; the others leave S at b_hi in the
// snapshot of block b_hi, where the next segment starts.
__global__ void __launch_bounds__(256) vla_res_chain_kernel(ResPlan pl, int b_lo, int b_hi,
                                                            const float* __restrict__ S_in, int64_t S_in_stride,
                                                            float* __restrict__ S_T, int32_t* __restrict__ stats,
                                                            const int32_t* __restrict__ chain_info, int last) {
  __shared__ uint4 sR0[kSlotVecs], sR1[kSlotVecs], sR2[kSlotVecs];   // operand ring
  static_assert(kRing == 3, "the ring is sR0, sR1, sR2");
  __shared__ float sX0[kXFloats], sX1[kXFloats];                     // tile exchange, by block parity
  __shared__ int sbad[4];
  ChainLane cl;
  cl.chain = blockIdx.x;
  cl.nblk = pl.nblk;
  cl.b_lo = b_lo;
  cl.nb = b_hi - b_lo;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, i = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar copy offsets
  const int jb = w & 1, c = w >> 1;
  cl.w = w;
  cl.lane = lane;
  cl.jb = jb;
  cl.soff = (32 * c + i) * kD + 32 * jb + 4 * h;   // this lane's S entries: soff + 8 q + 0..3
  const int64_t chain = cl.chain;
  const int nblk = cl.nblk, nb = cl.nb;

  f32x16 Y;
  {
    const float* src = S_in + chain * S_in_stride + cl.soff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(src + 8 * q);
      Y[4 * q] = x.x; Y[4 * q + 1] = x.y; Y[4 * q + 2] = x.z; Y[4 * q + 3] = x.w;
    }
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) sX0[(w * 16 + s) * 64 + lane] = Y[s];
  const int64_t blk0 = chain * nblk + b_lo;
  if (nb > 0) ring_copy(pl, sR0, blk0, w, lane);
  if (nb > 1) ring_copy(pl, sR1, blk0 + 1, w, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Block lb of the segment reads ring slot lb % 3 and exchange buffer lb % 2.
  for (int lb = 0; lb < nb; lb += 6) {
    chain_block(pl, cl, lb, Y, sR0, sR2, sX0, sX1);
    if (lb + 1 < nb) chain_block(pl, cl, lb + 1, Y, sR1, sR0, sX1, sX0);
    if (lb + 2 < nb) chain_block(pl, cl, lb + 2, Y, sR2, sR1, sX0, sX1);
    if (lb + 3 < nb) chain_block(pl, cl, lb + 3, Y, sR0, sR2, sX1, sX0);
    if (lb + 4 < nb) chain_block(pl, cl, lb + 4, Y, sR1, sR0, sX0, sX1);
    if (lb + 5 < nb) chain_block(pl, cl, lb + 5, Y, sR2, sR1, sX1, sX0);
  }

  if (!last) {
    float* dst = pl.Ssnap + (chain * nblk + b_hi) * kD * kD + cl.soff;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(dst + 8 * q) = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
    return;
  }
  bool bad = false;
  {
    float* dst = S_T + chain * kD * kD + cl.soff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
      bad |= !(isfinite(x.x) && isfinite(x.y) && isfinite(x.z) && isfinite(x.w));
      *reinterpret_cast<float4*>(dst + 8 * q) = x;
    }
  }
  const bool wave_bad = __any(bad);
  if (lane == 0) sbad[w] = wave_bad ? 1 : 0;
  __syncthreads();
  if (tid == 0 && stats) {
    int32_t* st = stats + chain * 4;
    st[0] = chain_info[chain * 4 + kInfoGuard];
    st[1] = 0;
    st[2] = (sbad[0] | sbad[1] | sbad[2] | sbad[3] | chain_info[chain * 4 + kInfoNonfinite]) ? 1 : 0;
    st[3] = -1;
  }
}

// Normalisers at the starts of blocks [b_lo, b_hi), n_b = n_{b_lo} + the key
// sums of the blocks before b, from n_in (n at b_lo, [chains][64]); writes n
// at b_hi to n_out.  One workgroup of 1024 threads per chain, thread (g, f) =
// (tid >> 6, tid & 63) takes feature f over segment g of 16.
__global__ void __launch_bounds__(1024) vla_res_nprefix_kernel(ResPlan pl, int b_lo, int b_hi,
                                                               const float* __restrict__ n_in,
                                                               float* __restrict__ n_out) {
  __shared__ float part[16][kD];
  const int64_t chain = blockIdx.x;
  const int nblk = pl.nblk;
  const int f = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int nb = b_hi - b_lo;
  const int per = (nb + 15) / 16;
  const int lo = b_lo + min(nb, g * per), hi = b_lo + min(nb, g * per + per);
  const float* ks = pl.ksum + chain * nblk * kD + f;
  float sum = 0.f;
  for (int b = lo; b < hi; ++b) sum += ks[b * kD];
  part[g][f] = sum;
  __syncthreads();
  const float n0 = n_in[chain * kD + f];
  float n = n0;
  for (int x = 0; x < g; ++x) n += part[x][f];
  float* nbk = pl.nblock + chain * nblk * kD + f;
  for (int b = lo; b < hi; ++b) {
    nbk[b * kD] = n;
    n += ks[b * kD];
  }
  if (g == 15) {
    float t = n0;
    for (int x = 0; x < 16; ++x) t += part[x][f];
    n_out[chain * kD + f] = t;
  }
}

// ---------------------------------------------------------------------------
// Readout: one workgroup of 512 threads per (chain, block).  In the token
// loop thread tid owns row i = tid >> 3 of S and the eight consecutive
// columns 8 (tid & 7) .. 8 (tid & 7) + 7.
// ---------------------------------------------------------------------------
// 16 bytes of a [64][64] row-major block (index v of 1024 float4 / 512
// 8-value bf16 chunks) into a padded LDS matrix as fp32.
__device__ __forceinline__ void put4(float* m, int v, float4 x) {
  *reinterpret_cast<float4*>(m + (v >> 4) * kP + 4 * (v & 15)) = x;
}
__device__ __forceinline__ void put8(float* m, int v, uint4 x) {
  float* dst = m + (v >> 3) * kP + 8 * (v & 7);
  *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                                                __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
  *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(x.z << 16), __uint_as_float(x.z & 0xffff0000u),
                                                    __uint_as_float(x.w << 16), __uint_as_float(x.w & 0xffff0000u));
}

// Rows [0, nvalid) of a [64][64] block of token vectors in the storage dtype,
// as fp32 into a padded LDS matrix; rows past nvalid read as zero.
template <typename TIn>
struct TokRows {
  static constexpr int kVecs = sizeof(TIn) == 4 ? 2 : 1;   // 16-byte vectors per thread
  uint4 r[kVecs];
  __device__ __forceinline__ void load(const TIn* g, int nvalid, int tid) {
    constexpr int kPerVec = 16 / sizeof(TIn);
#pragma unroll
    for (int x = 0; x < kVecs; ++x) {
      const int v = tid + 512 * x;
      r[x] = (v * kPerVec) / kD < nvalid ? reinterpret_cast<const uint4*>(g)[v] : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void put(float* m, int tid) const {
#pragma unroll
    for (int x = 0; x < kVecs; ++x) {
      const int v = tid + 512 * x;
      if constexpr (sizeof(TIn) == 4) {
        put4(m, v, make_float4(__uint_as_float(r[x].x), __uint_as_float(r[x].y), __uint_as_float(r[x].z),
                               __uint_as_float(r[x].w)));
      } else {
        put8(m, v, r[x]);
      }
    }
  }
};

template <typename TIn, bool CAP>
__global__ void __launch_bounds__(512) vla_res_readout_kernel(ResPlan pl, float den_eps, float cap2, int chains, int b_lo, int nb,
                                                              int32_t* __restrict__ chain_info,
                                                              const int32_t* __restrict__ only_flagged) {
  extern __shared__ float4 smem4[];
  float* R0 = reinterpret_cast<float*>(smem4);   // S_b, then q
  float* R1 = R0 + kMat;                          // W, then k, then o
  float* R2 = R1 + kMat;                          // U, then E
  float* R3 = R2 + kMat;                          // alpha
  __shared__ float sDen[kB];
  __shared__ float sNorm[kB][32];                 // per-token partial |S_t|^2 of each 16-lane group
  __shared__ float sNb[kD];
  __shared__ float sEn[kB];      // |e_t|^2
  __shared__ float sSp[32];      // partial |S_b|^2 of each 16-lane group
  __shared__ int sExact;         // the block needs the exact per-token norms

  const int nblk = pl.nblk;
  // Blocks [b_lo, b_lo + nb) of every chain, grid-stride.
  for (int64_t x = blockIdx.x; x < static_cast<int64_t>(chains) * nb; x += gridDim.x) {
  const int64_t chain = x / nb;
  const int b = b_lo + static_cast<int>(x % nb);
  const int tid = threadIdx.x;
  const int t0 = b * kB;
  const int nvalid = min(kB, pl.T - t0);
  const int64_t blk = chain * nblk + b;
  const int64_t tok0 = chain * pl.T + t0;
  if (only_flagged && only_flagged[blk] == 0) continue;   // uniform per workgroup

  // Every global load up front: S_b, W, U, alpha (fp32) and q, k.
  float4 gS[2], gW[2], gU[2], gA[2];
  {
    const float4* s4 = reinterpret_cast<const float4*>(pl.Ssnap + blk * kD * kD);
    const float4* w4 = reinterpret_cast<const float4*>(pl.W + blk * kB * kD);
    const float4* u4 = reinterpret_cast<const float4*>(pl.U + blk * kB * kD);
    const float4* a4 = reinterpret_cast<const float4*>(pl.alpha + tok0 * kD);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int v = tid + 512 * x;
      gS[x] = s4[v];
      gW[x] = w4[v];
      gU[x] = u4[v];
      gA[x] = (v >> 4) < nvalid ? a4[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  TokRows<TIn> gq, gk;
  gq.load(static_cast<const TIn*>(pl.q) + tok0 * kD, nvalid, tid);
  gk.load(static_cast<const TIn*>(pl.k) + tok0 * kD, nvalid, tid);
  if (tid < kD) sNb[tid] = pl.nblock[blk * kD + tid];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    put4(R0, tid + 512 * x, gS[x]);
    put4(R1, tid + 512 * x, gW[x]);
    put4(R2, tid + 512 * x, gU[x]);
    put4(R3, tid + 512 * x, gA[x]);
  }
  __syncthreads();

  // E = U - W S_b^T: thread (t, jc) computes E[t][jc + 8 m], m = 0..7.
  const int i = tid >> 3, jc = tid & 7;
  {
    const int t = i;
    float acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = R2[t * kP + jc + 8 * m];
#pragma unroll 4
    for (int j = 0; j < kD; j += 4) {
      const float4 wv = *reinterpret_cast<const float4*>(R1 + t * kP + j);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float4 sv = *reinterpret_cast<const float4*>(R0 + (jc + 8 * m) * kP + j);
        acc[m] = fmaf(-wv.x, sv.x, acc[m]);
        acc[m] = fmaf(-wv.y, sv.y, acc[m]);
        acc[m] = fmaf(-wv.z, sv.z, acc[m]);
        acc[m] = fmaf(-wv.w, sv.w, acc[m]);
      }
    }
    __syncthreads();   // every thread has read its U entries before E overwrites them
    float e2 = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      R2[t * kP + jc + 8 * m] = acc[m];
      e2 = fmaf(acc[m], acc[m], e2);
    }
    if constexpr (CAP) {
      e2 = group_sum<8>(e2);
      if (jc == 0) sEn[t] = e2;
    }
  }
  // This thread's row of S_b for the token loop.
  float S[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(R0 + i * kP + 8 * jc);
    const float4 c = *reinterpret_cast<const float4*>(R0 + i * kP + 8 * jc + 4);
    S[0] = a.x; S[1] = a.y; S[2] = a.z; S[3] = a.w; S[4] = c.x; S[5] = c.y; S[6] = c.z; S[7] = c.w;
  }
  if constexpr (CAP) {
    float s2 = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) s2 = fmaf(S[m], S[m], s2);
    s2 = group_sum<16>(s2);
    if ((tid & 15) == 0) sSp[tid >> 4] = s2;
  }
  __syncthreads();
  gq.put(R0, tid);
  gk.put(R1, tid);
  __syncthreads();

  // Denominators n_t . q_t + den_eps, n_t = n_b + sum_{s<=t} k_s: thread
  // (t, jc) takes n_b's features 8 jc .. 8 jc + 7 and the keys s = jc + 8 m <= t.
  {
    const int t = i;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf(sNb[8 * jc + e], R0[t * kP + 8 * jc + e], d);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int s = jc + 8 * m;
      if (s <= t) {
#pragma unroll 4
        for (int j = 0; j < kD; j += 4) {
          const float4 qv = *reinterpret_cast<const float4*>(R0 + t * kP + j);
          const float4 kv = *reinterpret_cast<const float4*>(R1 + s * kP + j);
          d = fmaf(qv.x, kv.x, d);
          d = fmaf(qv.y, kv.y, d);
          d = fmaf(qv.z, kv.z, d);
          d = fmaf(qv.w, kv.w, d);
        }
      }
    }
    d = group_sum<8>(d);
    if (jc == 0) sDen[t] = d + den_eps;
  }
  if constexpr (CAP) {
    // |S_t|_F <= |S_b|_F + sum_{s<=t} |e_s| |alpha_s| and |alpha_s| <= 1: when
    // that bound stays under the cap for the whole block, no token can fire.
    if (tid < 64) {
      const float ssq = wave_sum(tid < 32 ? sSp[tid] : 0.f);
      const float esum = wave_sum(sqrtf(sEn[tid]));
      if (tid == 0) sExact = (sqrtf(ssq) + esum) * (1.f + 1e-5f) > sqrtf(cap2) ? 1 : 0;
    }
  }
  __syncthreads();
  const bool exact = CAP && sExact != 0;

  // The block's tokens in order: S_t = S_{t-1} + e_t alpha_t^T, o_t, |S_t|^2.
  bool bad = false;
  for (int t = 0; t < nvalid; ++t) {
    const float ev = R2[t * kP + i];
    const float4 a0 = *reinterpret_cast<const float4*>(R3 + t * kP + 8 * jc);
    const float4 a1 = *reinterpret_cast<const float4*>(R3 + t * kP + 8 * jc + 4);
    const float4 q0 = *reinterpret_cast<const float4*>(R0 + t * kP + 8 * jc);
    const float4 q1 = *reinterpret_cast<const float4*>(R0 + t * kP + 8 * jc + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float po = 0.f, ns = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      S[m] = fmaf(ev, av[m], S[m]);
      po = fmaf(S[m], qv[m], po);
      if (exact) ns = fmaf(S[m], S[m], ns);
    }
    po = group_sum<8>(po);
    if (jc == 0) {
      const float ov = po / sDen[t];
      bad |= !isfinite(ov);
      R1[t * kP + i] = ov;
    }
    if (exact) {
      ns = group_sum<16>(ns);
      if ((tid & 15) == 0) sNorm[t][tid >> 4] = ns;
    }
  }
  __syncthreads();

  // Outputs, and the cap test on every token's |S_t|_F.
  {
    TIn* og = static_cast<TIn*>(pl.o) + tok0 * kD;
    const int t = tid >> 3, c8 = 8 * (tid & 7);
    if (t < nvalid) {
      const float4 x0 = *reinterpret_cast<const float4*>(R1 + t * kP + c8);
      const float4 x1 = *reinterpret_cast<const float4*>(R1 + t * kP + c8 + 4);
      if constexpr (sizeof(TIn) == 4) {
        *reinterpret_cast<float4*>(og + t * kD + c8) = x0;
        *reinterpret_cast<float4*>(og + t * kD + c8 + 4) = x1;
      } else {
        const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wv[e] = static_cast<uint32_t>(f32_to_bf16(f[2 * e])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * e + 1])) << 16);
        *reinterpret_cast<uint4*>(og + t * kD + c8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  }
  bool over = false;
  if (exact) {
    if (tid < nvalid) {
      float ns = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) ns += sNorm[tid][r];
      over = ns > cap2;
    }
  }
  const bool any_over = __any(over), any_bad = __any(bad);
  if ((tid & 63) == 0) {
    if (any_over) atomicMax(chain_info + chain * 4 + kInfoRestart, nblk - b);
    if (any_bad) atomicOr(chain_info + chain * 4 + kInfoNonfinite, 1);
  }
  __syncthreads();   // the next block overwrites the LDS this one read last
  }
}

// ---------------------------------------------------------------------------
// Readout on the matrix cores: one workgroup of four waves per (chain, block);
// wave w computes output tile (tb, ib) = (w >> 1, w & 1) (tokens x values):
//   E = U - W S_b^T,   O = Q S_b^T + (M o (A_hat Q^T))^T E,
//   den_t = n_b . q_t + sum_{s <= t} k_s . q_t + den_eps,
// with M the causal mask s <= t.  A_hat Q^T is computed as its transpose
// tile CT[s][t] (rows s in accumulator slots, columns t in lanes), which read
// as the A operand is the (t, s) operand of the product with E.  q and k
// enter as matrix-core operands loaded straight from HBM (bf16 storage
// exactly, fp32 as three-term splits).  The per-token norms of the cap test
// are not formed here: a block whose bound |S_b|_F + sum_s |e_s| exceeds the
// cap is flagged, and the per-token readout above recomputes it exactly.
// ---------------------------------------------------------------------------
template <typename TIn> struct QFrag;
template <> struct QFrag<uint16_t> {
  bf16x8 f;
  __device__ __forceinline__ void load(const uint16_t* p, bool ok) {
    f = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0));
  }
  __device__ __forceinline__ const bf16x8& op() const { return f; }
};
template <> struct QFrag<float> {
  Split3 f;
  __device__ __forceinline__ void load(const float* p, bool ok) {
    float x[8];
    const float4 a = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 b = ok ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    f = split3(x);
  }
  __device__ __forceinline__ const Split3& op() const { return f; }
};
__device__ __forceinline__ float frag_dot(const bf16x8& f, const float* nb) {
  const uint4 u = __builtin_bit_cast(uint4, f);
  const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    d = fmaf(__uint_as_float(w4[e] << 16), nb[2 * e], d);
    d = fmaf(__uint_as_float(w4[e] & 0xffff0000u), nb[2 * e + 1], d);
  }
  return d;
}
__device__ __forceinline__ float frag_dot(const Split3& f, const float* nb) {
  // t1 + t2 + t3 is the fp32 value exactly.
  return frag_dot(f.t1, nb) + (frag_dot(f.t2, nb) + frag_dot(f.t3, nb));
}

template <typename TIn, bool CAP>
__global__ void __launch_bounds__(256) vla_res_readout_mma_kernel(ResPlan pl, float den_eps, float cap2, int chains,
                                                                  int b_lo, int nb, int32_t* __restrict__ chain_info,
                                                                  int32_t* __restrict__ exact_flags) {
  extern __shared__ float4 smem4[];
  float* R0 = reinterpret_cast<float*>(smem4);   // S_b
  float* R1 = R0 + kMat;                          // W, then o
  float* R2 = R1 + kMat;                          // U, then E
  float* R3 = R2 + kMat;                          // alpha
  __shared__ float sNb[kD];
  __shared__ float sDen[kB];
  __shared__ float sEn[kB];
  __shared__ float sSp[4];
  __shared__ int sFlag;

  const int nblk = pl.nblk;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, lh = lane >> 5;
  const int w = tid >> 6, tb = w >> 1, ib = w & 1;
  for (int64_t x = blockIdx.x; x < static_cast<int64_t>(chains) * nb; x += gridDim.x) {
  const int64_t chain = x / nb;
  const int b = b_lo + static_cast<int>(x % nb);
  const int t0 = b * kB;
  const int nvalid = min(kB, pl.T - t0);
  const int64_t blk = chain * nblk + b;
  const int64_t tok0 = chain * pl.T + t0;

  // HBM: S_b, W, U, alpha into LDS; q rows of token block tb and k rows of
  // blocks sb <= tb as operand fragments.
  {
    const float4* s4 = reinterpret_cast<const float4*>(pl.Ssnap + blk * kD * kD);
    const float4* w4 = reinterpret_cast<const float4*>(pl.W + blk * kB * kD);
    const float4* u4 = reinterpret_cast<const float4*>(pl.U + blk * kB * kD);
    const float4* a4 = reinterpret_cast<const float4*>(pl.alpha + tok0 * kD);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int v = tid + 256 * r;
      put4(R0, v, s4[v]);
      put4(R1, v, w4[v]);
      put4(R2, v, u4[v]);
      put4(R3, v, (v >> 4) < nvalid ? a4[v] : make_float4(0.f, 0.f, 0.f, 0.f));
    }
  }
  if (tid < kD) sNb[tid] = pl.nblock[blk * kD + tid];
  const TIn* qg = static_cast<const TIn*>(pl.q) + tok0 * kD;
  const TIn* kg = static_cast<const TIn*>(pl.k) + tok0 * kD;
  QFrag<TIn> qf[4], kf[2][4];
  {
    const int tq = 32 * tb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks].load(qg + tq * kD + 16 * ks + 8 * lh, tq < nvalid);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int ts = 32 * sb + li;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[sb][ks].load(kg + ts * kD + 16 * ks + 8 * lh, sb <= tb && ts < nvalid);
    }
  }
  __syncthreads();

  // E tile (tb, ib) = U - W S_b^T, and Q S_b^T into the output accumulator.
  f32x16 E, O = zero16();
#pragma unroll
  for (int s = 0; s < 16; ++s) E[s] = R2[(32 * tb + acc_row(s, lh)) * kP + 32 * ib + li];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const Split3 bs = row_frag(R0 + (32 * ib + li) * kP + 16 * ks + 8 * lh);
    float wv[8];
    {
      const float* p = R1 + (32 * tb + li) * kP + 16 * ks + 8 * lh;
      const float4 a = *reinterpret_cast<const float4*>(p), c = *reinterpret_cast<const float4*>(p + 4);
      wv[0] = -a.x; wv[1] = -a.y; wv[2] = -a.z; wv[3] = -a.w; wv[4] = -c.x; wv[5] = -c.y; wv[6] = -c.z; wv[7] = -c.w;
    }
    E = mma_split(split3(wv), bs, E);
    O = mma_split(qf[ks].op(), bs, O);
  }
  __syncthreads();   // every wave has read its U tile and the W rows
#pragma unroll
  for (int s = 0; s < 16; ++s) R2[(32 * tb + acc_row(s, lh)) * kP + 32 * ib + li] = E[s];
  __syncthreads();

  // (M o (A_hat Q^T))^T E, and the denominators from (M o (K Q^T)).
  float kq = 0.f;   // sum_{s <= t} k_s . q_t for t = 32 tb + li (this lane's half of s)
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    if (sb > tb) continue;
    f32x16 CT = zero16(), KQ = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const Split3 af = row_frag(R3 + (32 * sb + li) * kP + 16 * ks + 8 * lh);
      CT = mma_split(af, qf[ks].op(), CT);
      KQ = mma_split(kf[sb][ks].op(), qf[ks].op(), KQ);
    }
    const int tg = 32 * tb + li;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const bool keep = 32 * sb + acc_row(s, lh) <= tg;
      CT[s] = keep ? CT[s] : 0.f;
      kq += keep ? KQ[s] : 0.f;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float ev[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ev[e] = R2[(32 * sb + acc_row(8 * g + e, lh)) * kP + 32 * ib + li];
      O = mma_split(split_slots(CT, g), split3(ev), O);
    }
  }
  if (ib == 0) {
    float nq = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) nq += frag_dot(qf[ks].op(), sNb + 16 * ks + 8 * lh);
    float d = kq + nq;
    d += __shfl_xor(d, 32);
    if (lh == 0) sDen[32 * tb + li] = d + den_eps;
  }
  // Norm bound: |S_b|^2 and |e_t|^2 (thread t = tid >> 2 takes 16 columns).
  if constexpr (CAP) {
    const int t = tid >> 2, c16 = 16 * (tid & 3);
    float e2 = 0.f, s2 = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float ev = R2[t * kP + c16 + c], sv = R0[t * kP + c16 + c];
      e2 = fmaf(ev, ev, e2);
      s2 = fmaf(sv, sv, s2);
    }
    e2 = group_sum<4>(e2);
    if ((tid & 3) == 0) sEn[t] = e2;
    s2 = wave_sum(s2);
    if (lane == 0) sSp[w] = s2;
  }
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int t = 32 * tb + acc_row(s, lh);
    const float ov = O[s] / sDen[t];
    bad |= t < nvalid && !isfinite(ov);
    R1[t * kP + 32 * ib + li] = ov;
  }
  if constexpr (CAP) {
    if (tid < 64) {
      const float esum = wave_sum(sqrtf(sEn[tid]));
      const float ssq = (sSp[0] + sSp[1]) + (sSp[2] + sSp[3]);
      if (tid == 0) sFlag = (sqrtf(ssq) + esum) * (1.f + 1e-5f) > sqrtf(cap2) ? 1 : 0;
    }
  }
  __syncthreads();
  if (tid == 0) exact_flags[blk] = CAP ? sFlag : 0;
  {
    TIn* og = static_cast<TIn*>(pl.o) + tok0 * kD;
    const int t = tid >> 2, c16 = 16 * (tid & 3);
    if (t < nvalid) {
      const float* src = R1 + t * kP + c16;
      if constexpr (sizeof(TIn) == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(og + t * kD + c16 + 4 * q) = *reinterpret_cast<const float4*>(src + 4 * q);
      } else {
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wv[e] = static_cast<uint32_t>(f32_to_bf16(src[8 * h8 + 2 * e])) |
                    (static_cast<uint32_t>(f32_to_bf16(src[8 * h8 + 2 * e + 1])) << 16);
          *reinterpret_cast<uint4*>(og + t * kD + c16 + 8 * h8) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      }
    }
  }
  if (__any(bad) && lane == 0) atomicOr(chain_info + chain * 4 + kInfoNonfinite, 1);
  __syncthreads();   // the next block overwrites the LDS this one read last
  }
}

template <typename K>
void allow_lds(K kernel, size_t bytes) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes));
}

}  // namespace

static unsigned side_grid(int64_t units, int max_wg) {
  if (max_wg > 0 && units > max_wg) units = max_wg;
  return static_cast<unsigned>(units);
}

hipError_t launch_res_prep(const ResPlan& pl, int chains, int b_lo, int nb, int max_wg, hipStream_t stream) {
  if (nb <= 0) return hipSuccess;
  const size_t lds = 4 * kMat * sizeof(float);
  const dim3 grid(side_grid(static_cast<int64_t>(chains) * nb, max_wg));
  if (pl.bf16) {
    allow_lds(vla_res_prep_kernel<uint16_t>, lds);
    hipLaunchKernelGGL(vla_res_prep_kernel<uint16_t>, grid, dim3(256), lds, stream, pl, chains, b_lo, nb);
  } else {
    allow_lds(vla_res_prep_kernel<float>, lds);
    hipLaunchKernelGGL(vla_res_prep_kernel<float>, grid, dim3(256), lds, stream, pl, chains, b_lo, nb);
  }
  return hipGetLastError();
}

hipError_t launch_res_nprefix(const ResPlan& pl, int b_lo, int b_hi, const float* n_in, float* n_out, int chains,
                              hipStream_t stream) {
  hipLaunchKernelGGL(vla_res_nprefix_kernel, dim3(static_cast<unsigned>(chains)), dim3(1024), 0, stream, pl, b_lo,
                     b_hi, n_in, n_out);
  return hipGetLastError();
}

hipError_t launch_res_chain(const ResPlan& pl, int b_lo, int b_hi, const float* S_in, int64_t S_in_stride,
                            float* S_T, int32_t* stats, const int32_t* chain_info, int last, int chains,
                            hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  hipError_t e = hipSuccess;
  if (ev_start && (e = hipEventRecord(ev_start, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(vla_res_chain_kernel, dim3(static_cast<unsigned>(chains)), dim3(256), 0, stream, pl, b_lo, b_hi,
                     S_in, S_in_stride, S_T, stats, chain_info, last);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_stop) e = hipEventRecord(ev_stop, stream);
  return e;
}

hipError_t launch_res_readout(const ResPlan& pl, float den_eps, float cap, int cap_on, int chains, int b_lo, int nb,
                              int max_wg, int32_t* chain_info, hipStream_t stream) {
  if (nb <= 0) return hipSuccess;
  const dim3 grid(side_grid(static_cast<int64_t>(chains) * nb, max_wg));
  const float cap2 = cap * cap;
  const size_t lds_mma = 4 * kMat * sizeof(float);
#define VLA_RES_READOUT_MMA(T, C)                                                                               \
  do {                                                                                                          \
    allow_lds(vla_res_readout_mma_kernel<T, C>, lds_mma);                                                       \
    hipLaunchKernelGGL((vla_res_readout_mma_kernel<T, C>), grid, dim3(256), lds_mma, stream, pl, den_eps, cap2, \
                       chains, b_lo, nb, chain_info, pl.exact);                                                 \
  } while (0)
  if (pl.bf16) {
    if (cap_on) VLA_RES_READOUT_MMA(uint16_t, true); else VLA_RES_READOUT_MMA(uint16_t, false);
  } else {
    if (cap_on) VLA_RES_READOUT_MMA(float, true); else VLA_RES_READOUT_MMA(float, false);
  }
#undef VLA_RES_READOUT_MMA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !cap_on) return e;
  // Blocks whose norm bound exceeds the cap: the per-token readout, with the
  // exact cap test (the others return at once).
  const size_t lds = 4 * kMat * sizeof(float);
  if (pl.bf16) {
    allow_lds(vla_res_readout_kernel<uint16_t, true>, lds);
    hipLaunchKernelGGL((vla_res_readout_kernel<uint16_t, true>), grid, dim3(512), lds, stream, pl, den_eps, cap2,
                       chains, b_lo, nb, chain_info, pl.exact);
  } else {
    allow_lds(vla_res_readout_kernel<float, true>, lds);
    hipLaunchKernelGGL((vla_res_readout_kernel<float, true>), grid, dim3(512), lds, stream, pl, den_eps, cap2,
                       chains, b_lo, nb, chain_info, pl.exact);
  }
  return hipGetLastError();
}


// Restart set-up for the sequential fallback of the residual update: a chain
// with a token over the cap, and no other reason to rerun, restarts at the
// start of the chunk holding its first such block, from the chunk-start
// inverse and the exact state snapshot and normaliser there, written over
// its initial-state snapshot (which nothing reads after this).  Its start
// token goes to kInfoRestart and it is flagged for the fallback.  Chains
// flagged otherwise (a guard fire or a failed chunk-start inverse) rerun from
// token 0.
__global__ void __launch_bounds__(256) vla_res_restart_kernel(ResPlan pl, ResRestart rs) {
  const int64_t chain = blockIdx.x;
  int32_t* info = rs.chain_info + chain * 4;
  const int first = info[kInfoRestart];
  const int other = info[kInfoFallback];
  const int b = first > 0 ? pl.nblk - first : 0;
  const int t_r = (first > 0 && !other) ? (b * kB / rs.chunk_len) * rs.chunk_len : 0;
  if (t_r > 0) {
    const int chunk = t_r / rs.chunk_len, blk = t_r / kB;
    const float4* a = reinterpret_cast<const float4*>(rs.Ac + (chain * rs.nchunks + chunk) * kD * kD);
    const float4* sn = reinterpret_cast<const float4*>(pl.Ssnap + (chain * pl.nblk + blk) * kD * kD);
    float4* ad = reinterpret_cast<float4*>(rs.A_init + chain * kD * kD);
    float4* sd = reinterpret_cast<float4*>(rs.S_init + chain * kD * kD);
    for (int i = threadIdx.x; i < kD * kD / 4; i += blockDim.x) {
      ad[i] = a[i];
      sd[i] = sn[i];
    }
    if (threadIdx.x < kD) rs.n_init[chain * kD + threadIdx.x] = pl.nblock[(chain * pl.nblk + blk) * kD + threadIdx.x];
  }
  __syncthreads();   // every thread has read info
  if (threadIdx.x == 0) {
    info[kInfoRestart] = t_r;
    if (first > 0) info[kInfoFallback] = 1;
  }
}

hipError_t launch_res_restart(const ResPlan& pl, const ResRestart& rs, int chains, hipStream_t stream) {
  if (chains <= 0) return hipSuccess;
  hipLaunchKernelGGL(vla_res_restart_kernel, dim3(chains), dim3(256), 0, stream, pl, rs);
  return hipGetLastError();
}

}  // namespace vla
