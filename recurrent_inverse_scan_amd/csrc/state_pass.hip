// Blocked state pass of the chunked schedule (d = 64): the S/n recurrence, the
// Frobenius cap and the readout, given alpha_hat from the inverse pass.
//
// Per token ("Mathematical Primitives", section 5; README v3 notes item 5):
//     S <- S + v alpha_hat^T;  if |S|_F > cap: S <- S cap/|S|_F
//     n <- n + k;              o = S q / (n.q + den_eps)
// The cap makes this a nonlinear recurrence, but only through one scalar per
// token: S_t = c_t (S_{t-1} + v_t alpha_t^T) with c_t <= 1 decided by
// |S_{t-1} + v_t alpha_t^T|^2 = |S_{t-1}|^2 + 2 g_t + e_t,
//     g_t = v_t^T S_{t-1} alpha_t,   e_t = |v_t|^2 |alpha_t|^2.
// Over a block of 64 tokens starting from S_b, with sigma_t = prod_{r<=t} c_r
// (block-local):
//     S_t = sigma_t S_b + sum_{s<=t} (sigma_t / sigma_{s-1}) v_s alpha_s^T,
// so g_t = sigma_{t-1} v_t^T S_b alpha_t + sum_{s<t} (sigma_{t-1}/sigma_{s-1}) K(t,s)
// with K(t,s) = (v_t.v_s)(alpha_t.alpha_s).  The first term of every token is
// one matrix product with S_b, K does not depend on the cap and is computed
// for all blocks in parallel, and the recursion keeps one accumulator per
// token (lane) that gains K(t,s) after token s and is multiplied by c_s when
// the cap fires: only this 64-step scalar recursion is sequential.  Every
// weight is a ratio sigma_t/sigma_{s-1} <= 1, carried as block-local log
// scales L_t = log2 sigma_t, so nothing overflows however often the cap fires.
// S then advances by sigma_end S_b + V^T diag(sigma_end/sigma_{s-1}) A_hat and
// |S|^2 is recomputed exactly at each block boundary.  The outputs are a
// causal linear-attention form per block,
//     o_t = (sigma_t S_b q_t + sum_{s<=t} (sigma_t/sigma_{s-1}) (alpha_s.q_t) v_s) / den_t,
// computed in parallel once the per-token log scales and every block-start
// S_b are known.
//
// Kernels: vla_state_prep_kernel (parallel over blocks), vla_state_chain_kernel
// (one workgroup per chain, sequential over blocks), vla_state_readout_kernel
// (parallel over blocks).  Matrix products use 32x32x2 fp32 MFMA tiles: every
// wave owns one 32x32 tile of a 64x64 result.
#include <type_traits>

#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_mfma.h"
#include "vla_seq.h"

namespace vla {

namespace {

constexpr int kD = 64;     // head dimension
constexpr int kLb = 64;    // tokens per block
constexpr int kLd = 68;    // LDS row stride in floats (rows of 16 lanes hit distinct banks)
constexpr int kThreads = 256;
// Per-block pack the recursion wave consumes: the lower triangle of the
// exclusive row prefix sums of K, row t's entries j = 0..t at t(t+1)/2 + j
// (the sum over s < j of K(t,s); j = t is the sum before the diagonal), then
// 64 values each of K(t,t), the row totals and the block's key sum; padded to
// whole KiB.  Triangular numbers are distinct modulo 64, so lanes reading row
// t's entry t(t+1)/2 + j for one j hit distinct LDS banks.
constexpr int kTriN = kLb * (kLb + 1) / 2;
constexpr int kPackE = kTriN, kPackTot = kTriN + kLb, kPackKs = kTriN + 2 * kLb;
constexpr int kPackFloats = 2304;
constexpr int kPackPieces = kPackFloats / 256;   // 1 KiB pieces
static_assert(kPackKs + kLb <= kPackFloats, "pack layout");

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads and stores (a __syncthreads fence
// would also drain the global loads still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// acc[m][n] += sum_k A[m][k] B[n][k]; A and B point at the tile's first row in
// LDS (row stride kLd), K = 64.  Lane half h covers k = 32h .. 32h+31.
__device__ __forceinline__ void mma_rr(f32x16& acc, const float* A, const float* B, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const float* a = A + r * kLd + 32 * h;
  const float* b = B + r * kLd + 32 * h;
#pragma unroll
  for (int kb = 0; kb < 32; kb += 4) {
    const float4 av = *reinterpret_cast<const float4*>(a + kb);
    const float4 bv = *reinterpret_cast<const float4*>(b + kb);
    acc = mfma(av.x, bv.x, acc);
    acc = mfma(av.y, bv.y, acc);
    acc = mfma(av.z, bv.z, acc);
    acc = mfma(av.w, bv.w, acc);
  }
}

// acc[m][n] += sum_k A[m][k] w[k] B[n][k] (rows as in mma_rr, w indexed by k).
__device__ __forceinline__ void mma_rr_w(f32x16& acc, const float* A, const float* B, const float* w, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const float* a = A + r * kLd + 32 * h;
  const float* b = B + r * kLd + 32 * h;
  const float* ww = w + 32 * h;
#pragma unroll
  for (int kb = 0; kb < 32; kb += 4) {
    const float4 av = *reinterpret_cast<const float4*>(a + kb);
    const float4 bv = *reinterpret_cast<const float4*>(b + kb);
    const float4 wv = *reinterpret_cast<const float4*>(ww + kb);
    acc = mfma(av.x * wv.x, bv.x, acc);
    acc = mfma(av.y * wv.y, bv.y, acc);
    acc = mfma(av.z * wv.z, bv.z, acc);
    acc = mfma(av.w * wv.w, bv.w, acc);
  }
}

// acc[m][n] += sum_k A[m][k] B[k][n]; A at the tile's first row, B at its first column.
__device__ __forceinline__ void mma_rc(f32x16& acc, const float* A, const float* B, int lane) {
  const int c = lane & 31, h = lane >> 5;
  const float* a = A + c * kLd + 32 * h;
#pragma unroll
  for (int kb = 0; kb < 32; kb += 4) {
    const float4 av = *reinterpret_cast<const float4*>(a + kb);
    const int k = 32 * h + kb;
    acc = mfma(av.x, B[(k + 0) * kLd + c], acc);
    acc = mfma(av.y, B[(k + 1) * kLd + c], acc);
    acc = mfma(av.z, B[(k + 2) * kLd + c], acc);
    acc = mfma(av.w, B[(k + 3) * kLd + c], acc);
  }
}

// ---- bf16 operands and buffer-to-LDS copies ----------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// Operand of 8 consecutive values at p: exact bf16 for bf16 storage, a
// three-term split for fp32.
__device__ __forceinline__ bf16x8 operand8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ Split3 operand8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return split3(x);
}

// Copies rows [0, nvalid) of a [64][64] block (global, contiguous rows of 64)
// into LDS as float32 with stride kLd; rows past nvalid become zero.
template <typename T>
__device__ __forceinline__ void stage_block(float* lds, const T* g, int nvalid, int tid) {
  constexpr int EPV = Elem<T>::kPer16B;
  for (int e = tid; e < kLb * kD / EPV; e += kThreads) {
    const int row = e / (kD / EPV), c = (e % (kD / EPV)) * EPV;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (row < nvalid) x = *reinterpret_cast<const uint4*>(g + row * kD + c);
    float* dst = lds + row * kLd + c;
    if constexpr (EPV == 4) {
      *reinterpret_cast<uint4*>(dst) = x;
    } else {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        dst[2 * h] = __uint_as_float(w[h] << 16);
        dst[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
      }
    }
  }
}

// ---- prep: kernel matrices, local normaliser terms, block key sums ---------
// Per block b of 64 tokens:
//   pack      = CK[t][j] = sum_{s<j} K(t,s) for j <= t, K(t,s) =
//               (v_t.v_s)(alpha_t.alpha_s) (exclusive row prefix, lower
//               triangle), then K(t,t), sum_s K(t,s) and sum_t k_t
//   Kx[t][s]  = (v_t.v_s)(alpha_t.alpha_s) with s in block b-1 (b >= 1)
//   ld[t]     = sum_{s<=t in block} k_s.q_t
//   VT, AT    = (fp32 storage only) v and alpha_hat of the block regrouped as
//               the chain kernel's matrix-core operands of its rank-64 update:
//               fragment (c, kb, lane) holds tokens 16 kb + 8 (lane / 32) + e,
//               e < 8, of feature 32 c + lane % 32.
// The Gram products run on the bf16 matrix cores: v.v and q.k exactly when
// stored as bf16, alpha.alpha (and fp32-stored inputs) through three-term splits.
template <typename TIn>
struct PrepLds {
  static constexpr int kRd = sizeof(TIn) == 2 ? 72 : 68;   // row stride of storage-dtype rows (16-byte aligned)
  static constexpr size_t kBytes = 4 * kLb * kRd * sizeof(TIn) + 2 * kLb * kLd * sizeof(float);
};

// Copies rows [0, nvalid) of a [64][64] block in its own dtype into LDS rows
// of the given stride; rows past nvalid become zero.
template <typename T>
__device__ __forceinline__ void stage_rows(T* lds, const T* g, int nvalid, int tid, int stride) {
  constexpr int EPV = 16 / static_cast<int>(sizeof(T));
  for (int e = tid; e < kLb * kD / EPV; e += kThreads) {
    const int row = e / (kD / EPV), c = (e % (kD / EPV)) * EPV;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (row < nvalid) x = *reinterpret_cast<const uint4*>(g + row * kD + c);
    *reinterpret_cast<uint4*>(lds + row * stride + c) = x;
  }
}

// A [64][64] tile in 16-byte pieces held in registers: thread tid holds
// pieces tid + 256 j.  Loading every tile a block needs before storing any of
// them to LDS puts all their global-memory latencies in one round.
template <typename T>
struct TileRegs {
  static constexpr int EPV = 16 / static_cast<int>(sizeof(T));   // elements per piece
  static constexpr int PPR = kD / EPV;                           // pieces per row
  static constexpr int N = kLb * PPR / kThreads;                 // pieces per thread
  uint4 r[N];
  // Rows [0, nvalid) of the tile at g (rows of 64); later rows read as zero.
  __device__ __forceinline__ void load(const T* g, int nvalid, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int e = tid + j * kThreads, row = e / PPR, c = (e % PPR) * EPV;
      r[j] = row < nvalid ? *reinterpret_cast<const uint4*>(g + row * kD + c) : make_uint4(0, 0, 0, 0);
    }
  }
  // As stored, rows of the given stride (elements of T).
  __device__ __forceinline__ void store_rows(T* lds, int stride, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int e = tid + j * kThreads, row = e / PPR, c = (e % PPR) * EPV;
      *reinterpret_cast<uint4*>(lds + row * stride + c) = r[j];
    }
  }
  // Widened to float32 rows of stride kLd.
  __device__ __forceinline__ void store_f32(float* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int e = tid + j * kThreads, row = e / PPR, c = (e % PPR) * EPV;
      float* dst = lds + row * kLd + c;
      if constexpr (EPV == 4) {
        *reinterpret_cast<uint4*>(dst) = r[j];
      } else {
        const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
        *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                                      __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
        *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                                          __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
      }
    }
  }
};

template <typename TIn>
__device__ __forceinline__ void prep_block(const StatePlan& pl, const TIn* __restrict__ q, const TIn* __restrict__ k,
                                           const TIn* __restrict__ v, int b_lo, int nb, int64_t item) {
  constexpr int kRd = PrepLds<TIn>::kRd;
  extern __shared__ float4 smem4[];
  TIn* Vb = reinterpret_cast<TIn*>(smem4);    // [64][kRd] v rows of the block
  TIn* Qb = Vb + kLb * kRd;                   // q rows
  TIn* Kb = Qb + kLb * kRd;                   // k rows
  TIn* Vp = Kb + kLb * kRd;                   // v rows of the previous block
  float* Af = reinterpret_cast<float*>(Vp + kLb * kRd);   // [64][kLd] alpha_hat rows, later K
  float* Ap = Af + kLb * kLd;                 // previous block's alpha_hat rows, later masked q.k
  const int64_t chain = item / nb;
  const int b = b_lo + static_cast<int>(item % nb);
  const int64_t blk = chain * pl.nblk + b;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
  const int64_t row0 = chain * pl.T + tb;
  {
    TileRegs<TIn> rv, rq, rk, rvp;
    TileRegs<float> ra, rap;
    rv.load(v + row0 * kD, tcount, tid);
    rq.load(q + row0 * kD, tcount, tid);
    rk.load(k + row0 * kD, tcount, tid);
    ra.load(pl.alpha + row0 * kD, tcount, tid);
    if (b > 0) {   // uniform; the previous block is always full
      rvp.load(v + (row0 - kLb) * kD, kLb, tid);
      rap.load(pl.alpha + (row0 - kLb) * kD, kLb, tid);
    }
    rv.store_rows(Vb, kRd, tid);
    rq.store_rows(Qb, kRd, tid);
    rk.store_rows(Kb, kRd, tid);
    ra.store_f32(Af, tid);
    if (b > 0) {
      rvp.store_rows(Vp, kRd, tid);
      rap.store_f32(Ap, tid);
    }
  }
  lds_barrier();

  const int ti = w >> 1, tj = w & 1, rl = lane & 31;
  f32x16 gv = zero16(), ga = zero16(), pk = zero16(), xv = zero16(), xa = zero16();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int c0 = 16 * kb + 8 * h;
    const auto va = operand8(Vb + (ti * 32 + rl) * kRd + c0);
    gv = mma_split(va, operand8(Vb + (tj * 32 + rl) * kRd + c0), gv);
    const Split3 aa = operand8(Af + (ti * 32 + rl) * kLd + c0);
    ga = mma_split(aa, operand8(Af + (tj * 32 + rl) * kLd + c0), ga);
    pk = mma_split(operand8(Kb + (ti * 32 + rl) * kRd + c0), operand8(Qb + (tj * 32 + rl) * kRd + c0), pk);   // k_s . q_t
    if (b > 0) {
      xv = mma_split(va, operand8(Vp + (tj * 32 + rl) * kRd + c0), xv);
      xa = mma_split(aa, operand8(Ap + (tj * 32 + rl) * kLd + c0), xa);
    }
  }
  float* pack = pl.Kmat + blk * kPackFloats;
  __shared__ float ksum_part[4][kLb];   // key sums over 16-token quarters of the block
  {
    const int f = tid & 63, qt = tid >> 6;
    float acc = 0.f;
#pragma unroll
    for (int t = 16 * qt; t < 16 * qt + 16; ++t) acc += Elem<TIn>::load(Kb + t * kRd + f);   // rows >= tcount are 0
    ksum_part[qt][f] = acc;
  }
  if (tid >= kLb && tid < kLb + (kPackFloats - kPackKs - kLb)) pack[kPackKs + tid] = 0.f;   // padding
  // Matrix-core operands of the chain kernel's update for fp32 storage
  // (features of v and alpha_hat are LDS columns here); with bf16 storage the
  // chain kernel reads them from its own LDS rows.
  if constexpr (sizeof(TIn) == 4) {
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int f = tid + 256 * rep, c = f >> 8, kb = (f >> 6) & 3, fl = f & 63;
      const int t0 = 16 * kb + 8 * (fl >> 5), feat = 32 * c + (fl & 31);
      float xa8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xa8[e] = Af[(t0 + e) * kLd + feat];
      float4* ad = reinterpret_cast<float4*>(pl.AT + (blk * 512 + f) * 8);
      ad[0] = make_float4(xa8[0], xa8[1], xa8[2], xa8[3]);
      ad[1] = make_float4(xa8[4], xa8[5], xa8[6], xa8[7]);
      float4* vd = reinterpret_cast<float4*>(static_cast<float*>(pl.VT) + (blk * 512 + f) * 8);
      vd[0] = make_float4(Vb[t0 * kRd + feat], Vb[(t0 + 1) * kRd + feat], Vb[(t0 + 2) * kRd + feat], Vb[(t0 + 3) * kRd + feat]);
      vd[1] = make_float4(Vb[(t0 + 4) * kRd + feat], Vb[(t0 + 5) * kRd + feat], Vb[(t0 + 6) * kRd + feat], Vb[(t0 + 7) * kRd + feat]);
    }
  }
  const int col = tj * 32 + rl;
  if (b > 0) {
    float* Xout = pl.Kcross + blk * kLb * kLb;
#pragma unroll
    for (int s = 0; s < 16; ++s) Xout[(ti * 32 + acc_row(s, h)) * kLb + col] = xv[s] * xa[s];
  }
  // This wave's tile of K = (v.v) o (alpha.alpha): rows s = 32 ti + slot
  // rows, columns 32 tj + lane; K is symmetric, so lane (n, h) holds row
  // t = 32 tj + n of K over s in block ti, down its slots.  The tile of pk
  // is k_s . q_t in the same arrangement.
  float Kt[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) Kt[s2] = gv[s2] * ga[s2];
  __shared__ float sX[16 * 64];       // tile (1, 1)'s prefix over s < 32, [slot][lane]
  __shared__ float sTot[kLb], sLd[kLb];   // row sums over s >= 32
  const int trow = tj * 32 + rl;      // this lane's row t for the row sums
  {
    float tp = 0.f, lp = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      tp += Kt[s2];
      lp += (ti * 32 + acc_row(s2, h) <= trow) ? pk[s2] : 0.f;
    }
    tp += __shfl_xor(tp, 32);
    lp += __shfl_xor(lp, 32);
    if (ti == 1 && h == 0) {
      sTot[trow] = tp;
      sLd[trow] = lp;
    }
    if (ti == tj) {   // the diagonal K(t, t)
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2)
        if (acc_row(s2, h) == rl) pack[kPackE + ti * 32 + rl] = Kt[s2];
    }
    gv = zero16();   // reused below for the prefix tiles
    if (ti == 0) {
      lds_barrier();
      if (h == 0) {
        pack[kPackTot + trow] = tp + (tj == 1 ? sTot[trow] : 0.f);
        if (trow < tcount) pl.ld[row0 + trow] = lp + (tj == 1 ? sLd[trow] : 0.f);
      }
    } else {
      lds_barrier();
    }
  }
  // Exclusive row prefixes CK[t][j] = sum_{s<j} K[t][s] on the matrix cores:
  // the K tile, read as the A operand (slots 8 g .. 8 g + 7 as k step g),
  // gives rows t = 32 tj + lane over s = 32 ti + 16 g + 8 (e / 4) + 4 h +
  // e % 4; the B operand is the 0/1 matrix [s < j] in the same k order.
  // Row block 0 needs s < 32 only (wave (0, 0)); row block 1 takes s < 32
  // from wave (0, 1) and s >= 32 from wave (1, 1).
  auto bmask = [&](int sb, int jb, int g) {   // [s < j], s = 32 sb + k order, j = 32 jb + lane
    uint32_t wd[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t x = 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int e = 2 * e2 + hh;
        const int sx = 32 * sb + 16 * g + 8 * (e >> 2) + 4 * h + (e & 3);
        x |= (sx < 32 * jb + rl) ? (0x3F80u << (16 * hh)) : 0u;
      }
      wd[e2] = x;
    }
    return __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
  };
  const auto rpack = make_rsrc(pack, kPackFloats * 4);
  auto store_tri = [&](const f32x16& D, int rb, int jb) {   // pack row t, column j <= t
    const int j = 32 * jb + rl;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const int t = 32 * rb + acc_row(s2, h);
      if (j <= t) buf_store_f32(rpack, 4 * (t * (t + 1) / 2 + j), D[s2]);
    }
  };
  if (!(ti == 1 && tj == 0)) {
    float k0[8], k1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      k0[e] = Kt[e];
      k1[e] = Kt[8 + e];
    }
    const Split3 A0 = split3(k0), A1 = split3(k1);
    if (ti == 0) {
      f32x16 D = mma_split(A1, bmask(0, 0, 1), mma_split(A0, bmask(0, 0, 0), zero16()));
      store_tri(D, tj, 0);   // tile (tj, 0): complete
      if (tj == 1) {
        const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
        D = mma_split(A1, ones, mma_split(A0, ones, zero16()));
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) sX[s2 * 64 + lane] = D[s2];
      }
    } else {
      gv = mma_split(A1, bmask(1, 1, 1), mma_split(A0, bmask(1, 1, 0), zero16()));
    }
  }
  lds_barrier();
  if (ti == 1 && tj == 1) {
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) gv[s2] += sX[s2 * 64 + lane];
    store_tri(gv, 1, 1);
  }
  if (tid < kLb) pack[kPackKs + tid] = (ksum_part[0][tid] + ksum_part[1][tid]) + (ksum_part[2][tid] + ksum_part[3][tid]);
}

// Blocks [b_lo, b_lo + nb) of every chain; a grid smaller than chains * nb
// strides over them.
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
vla_state_prep_kernel(StatePlan pl, const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v, int b_lo, int nb, int64_t items) {
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    prep_block<TIn>(pl, q, k, v, b_lo, nb, item);
    lds_barrier();   // LDS is restaged by the next item
  }
}

// ---- chain: the sequential part, one workgroup per chain ---------------------
// Five waves.  Wave 0 (the recursion wave) runs the cap recursion of block b.
// Waves 1-4 (the product waves) each own a 32x32 tile of S and, during the
// same time, apply block b-1's rank-64 update (S_b from S_{b-1}) and compute
// the next block's bilinear terms v_t^T S_b alpha_t, one block behind; the
// recursion wave repairs the lag exactly with the cross-block kernel:
//     v_t^T S_{b+1} alpha_t = sigma_end(b) v_t^T S_b alpha_t
//                            + sum_{s in b} (sigma_end(b)/sigma_{s-1}) Kx(t,s).
//
// Both products run on the bf16 matrix cores at fp32-grade accuracy: an fp32
// operand x is split into three bf16 terms x = x1 + x2 + x3 (each the
// round-to-nearest bf16 of what remains; the residuals are exact in fp32, so
// the split is exact to about 2^-27 |x|), bf16 v is exact as it stands, and
// the partial products (all pairs of terms whose orders add up to at most 2)
// accumulate in fp32.
//
// Staging is register-free: v and alpha_hat rows (for the bilinear terms) and
// the prefix-summed K and Kx (for the recursion) go from memory straight into
// LDS with buffer-to-LDS loads, two generations deep, in 16-byte chunks whose
// position within a row is XOR-swizzled by the row index (conflict-free
// row-per-lane reads).  The update's operands come from the prep kernel's
// regrouped copies into registers, one block ahead.  One barrier per block.
constexpr int kChainThreads = 320;

__device__ __forceinline__ void to_floats(uint4 x, float (&f)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(w[e] << 16);
    f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// Swizzled LDS image of a [64][64] fp32 matrix: chunk c (floats 4c..4c+3) of
// row r sits at chunk position c ^ (r & 15).
__device__ __forceinline__ int swz32(int r, int x) { return r * 64 + (((x >> 2) ^ (r & 15)) << 2) + (x & 3); }
// The same for bf16 rows (8 values per chunk, 8 chunks per row): index in bf16 units.
__device__ __forceinline__ int swz16(int r, int x) { return r * 64 + (((x >> 3) ^ (r & 7)) << 3) + (x & 7); }

// Buffer-to-LDS copy of 1 KiB piece p of a matrix: lane l's 16 bytes land at
// lds + 1024 p + 16 l; vo is the lane's source offset within the piece.
__device__ __forceinline__ void dma_piece(__amdgpu_buffer_rsrc_t r, char* lds, int p, int vo) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + 1024 * p), 16, vo, 1024 * p, 0, 0);
}

// The update's operands of one product wave for one block (fp32 storage):
// slot (kb, e) of lane l holds token 16 kb + 8 (l / 32) + e of feature
// 32 ti + l % 32 (v) and of feature 32 tj + l % 32 (alpha_hat).
template <typename TIn>
struct UpdFrags {
  static constexpr int kV = sizeof(TIn) / 2;   // uint4 per 8 values of v
  uint4 v[4][kV];
  uint4 a[4][2];
  // From the prep kernel's regrouped copies (fp32 storage).
  __device__ __forceinline__ void load(const StatePlan& pl, int64_t blk, int ti, int tj, int lane) {
    const auto rv = make_rsrc(static_cast<const TIn*>(pl.VT) + blk * 512 * 8, 512 * 8 * static_cast<int>(sizeof(TIn)));
    const auto ra = make_rsrc(pl.AT + blk * 512 * 8, 512 * 8 * 4);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int fv = (ti * 4 + kb) * 64 + lane, fa = (tj * 4 + kb) * 64 + lane;
#pragma unroll
      for (int j = 0; j < kV; ++j) v[kb][j] = buf_load16(rv, (fv * 8 * static_cast<int>(sizeof(TIn))) + 16 * j);
      a[kb][0] = buf_load16(ra, fa * 32);
      a[kb][1] = buf_load16(ra, fa * 32 + 16);
    }
  }
};

// X <- se X + sum over the block of (v_t)_i w_t (alpha_t)_j on this wave's tile.
template <typename TIn>
__device__ __forceinline__ void rank_update(f32x16& X, const UpdFrags<TIn>& fr, const float* wp, float se, int h) {
#pragma unroll
  for (int s = 0; s < 16; ++s) X[s] *= se;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float4 w0 = *reinterpret_cast<const float4*>(wp + 16 * kb + 8 * h);
    const float4 w1 = *reinterpret_cast<const float4*>(wp + 16 * kb + 8 * h + 4);
    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint32_t aw[8] = {fr.a[kb][0].x, fr.a[kb][0].y, fr.a[kb][0].z, fr.a[kb][0].w,
                            fr.a[kb][1].x, fr.a[kb][1].y, fr.a[kb][1].z, fr.a[kb][1].w};
    float bx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bx[e] = __uint_as_float(aw[e]) * ww[e];
    const Split3 B = split3(bx);
    if constexpr (sizeof(TIn) == 2) {
      X = mma_split(__builtin_bit_cast(bf16x8, fr.v[kb][0]), B, X);
    } else {
      const uint32_t vw[8] = {fr.v[kb][0].x, fr.v[kb][0].y, fr.v[kb][0].z, fr.v[kb][0].w,
                              fr.v[kb][1].x, fr.v[kb][1].y, fr.v[kb][1].z, fr.v[kb][1].w};
      float vx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vx[e] = __uint_as_float(vw[e]);
      X = mma_split(split3(vx), B, X);
    }
  }
}

// The same update with bf16 storage, its operands read from the block's
// swizzled LDS rows (column reads: slot (kb, e) of lane l is token
// 16 kb + 8 (l / 32) + e).  The lane's byte offsets of rows 8 (l / 32) + e
// come precomputed (UpdOffsets); rows 16 kb further are constant offsets.
struct UpdOffsets {
  int v[8], a[8];
  __device__ __forceinline__ void init(int ti, int tj, int lane) {
    const int h = lane >> 5, fv = ti * 32 + (lane & 31), fa = tj * 32 + (lane & 31);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = 2 * swz16(8 * h + e, fv);   // bf16 rows
      a[e] = 4 * swz32(8 * h + e, fa);   // fp32 rows
    }
  }
};
__device__ __forceinline__ void rank_update_lds(f32x16& X, const char* VR, const char* AR, const UpdOffsets& off,
                                                const float* wp, float se, int h) {
  uint32_t vr[4][8];
  float ar[4][8];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vr[kb][e] = *reinterpret_cast<const uint16_t*>(VR + off.v[e] + 2 * swz16(16 * kb, 0));
      ar[kb][e] = *reinterpret_cast<const float*>(AR + off.a[e] + 4 * swz32(16 * kb, 0));
    }
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) X[s] *= se;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const float4 w0 = *reinterpret_cast<const float4*>(wp + 16 * kb + 8 * h);
    const float4 w1 = *reinterpret_cast<const float4*>(wp + 16 * kb + 8 * h + 4);
    const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float bx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bx[e] = ar[kb][e] * ww[e];
    const uint4 va = make_uint4(vr[kb][0] | (vr[kb][1] << 16), vr[kb][2] | (vr[kb][3] << 16),
                                vr[kb][4] | (vr[kb][5] << 16), vr[kb][6] | (vr[kb][7] << 16));
    X = mma_split(__builtin_bit_cast(bf16x8, va), split3(bx), X);
  }
}

// Partial v_t^T S alpha_t of one block over this wave's tile of S (rows
// 32 ti.., columns 32 tj..), from the LDS rows of the block; lanes of the
// lower half write hr[t].  All LDS operands are read before the products.
template <typename TIn>
__device__ __forceinline__ void bilinear_terms(const f32x16& X, const char* VR, const float* AR, float* hr, int ti,
                                               int tj, int lane) {
  const int h = lane >> 5;
  constexpr int kVW = sizeof(TIn) == 2 ? 2 : 4;   // 32-bit words per 4 features of v
  uint32_t vp[2][2][2][kVW];                       // [tt][kb2][piece][word]
  float4 ar[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = tt * 32 + (lane & 31);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int f0 = ti * 32 + 16 * kb2 + 4 * h;   // features f0..f0+3 and f0+8..f0+11
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        if constexpr (sizeof(TIn) == 2) {
          const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(VR) + swz16(t, f0 + 8 * pc));
          vp[tt][kb2][pc][0] = x.x;
          vp[tt][kb2][pc][1] = x.y;
        } else {
          const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(VR) + swz32(t, f0 + 8 * pc));
          vp[tt][kb2][pc][0] = x.x;
          vp[tt][kb2][pc][1] = x.y;
          vp[tt][kb2][pc][2] = x.z;
          vp[tt][kb2][pc][3] = x.w;
        }
      }
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) ar[tt][q4] = *reinterpret_cast<const float4*>(AR + swz32(t, tj * 32 + 8 * q4 + 4 * h));
  }
  // S^T as the A operand: slots 8 kb2 + e of this lane are rows
  // 16 kb2 + 8 (e / 4) + 4 h + e % 4 of the tile, column = lane % 32.
  Split3 SA[2];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    float xs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[e] = X[8 * kb2 + e];
    SA[kb2] = split3(xs);
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    f32x16 Z = zero16();
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      if constexpr (sizeof(TIn) == 2) {
        Z = mma_split(SA[kb2], __builtin_bit_cast(bf16x8, make_uint4(vp[tt][kb2][0][0], vp[tt][kb2][0][1],
                                                                    vp[tt][kb2][1][0], vp[tt][kb2][1][1])), Z);
      } else {
        float vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vx[e] = __uint_as_float(vp[tt][kb2][0][e]);
          vx[4 + e] = __uint_as_float(vp[tt][kb2][1][e]);
        }
        Z = mma_split(SA[kb2], split3(vx), Z);
      }
    }
    // Z[j][t] = sum_i S_ij v_ti over the tile; contract with alpha_t over j.
    float p = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 a = ar[tt][q4];
      p = fmaf(a.x, Z[4 * q4], fmaf(a.y, Z[4 * q4 + 1], fmaf(a.z, Z[4 * q4 + 2], fmaf(a.w, Z[4 * q4 + 3], p))));
    }
    p += __shfl_xor(p, 32, 64);
    if (h == 0) hr[tt * 32 + (lane & 31)] = p;
  }
}

template <typename TIn>
__global__ void __launch_bounds__(kChainThreads)
vla_state_chain_kernel(StatePlan pl, ChainSeg sg, float* __restrict__ S_T, float* __restrict__ n_T,
                       int32_t* __restrict__ stats, const int32_t* __restrict__ chain_info, float cap, int cap_on) {
  // Buffers that buffer-to-LDS loads fill have one LDS object per
  // generation, every one selected at compile time: the compiler then sees
  // that reading one does not depend on loads still in flight into another.
  // A block's copies are issued when it starts, into buffers whose last
  // reader passed the previous barrier.  Each product wave waits for its own
  // copies before the block's closing barrier (the barrier alone does not
  // wait for them), so what one wave copies is complete for every wave after
  // that barrier.  The recursion wave copies the pack and Kx, which only it
  // reads, one block ahead and waits for them itself.
  // The v and alpha_hat rows of block j arrive during block j-2, give the
  // bilinear terms in block j-1 and, with bf16 storage, the update's
  // operands in block j+1: four generations.  With fp32 storage the update's
  // operands come from the prep kernel's regrouped copies instead, and two
  // generations (twice the bytes each) suffice.
  constexpr bool kBf = sizeof(TIn) == 2;
  constexpr int kRowGens = kBf ? 4 : 2;
  constexpr int kVR4 = kLb * kD * static_cast<int>(sizeof(TIn)) / 16;   // float4s per v-row block
  constexpr int kAR4x = kBf ? kLb * kD / 4 : 1, kVR4x = kBf ? kVR4 : 1;  // generations 2 and 3
  __shared__ float4 sCK0[kPackFloats / 4], sCK1[kPackFloats / 4];   // the pack
  __shared__ float4 sKX0[kLb * kLb / 4], sKX1[kLb * kLb / 4];   // Kx, swizzled
  __shared__ float4 sAR0[kLb * kD / 4], sAR1[kLb * kD / 4], sAR2[kAR4x], sAR3[kAR4x];   // alpha_hat rows, swizzled
  __shared__ float4 sVR0[kVR4], sVR1[kVR4], sVR2[kVR4x], sVR3[kVR4x];                   // v rows, swizzled
  __shared__ float sH[2][4 * kLb];                              // partial v^T S alpha per product wave
  __shared__ float sW[2][kLb];                                  // update weights sigma_end/sigma_{s-1}
  __shared__ float sSig[2];                                     // sigma_end
  __shared__ float sNrm[2][4];                                  // |S_b|^2 per product wave
  __shared__ float sRed[8];
  auto rows_ar = [&](int r) -> float4* { return r == 0 ? sAR0 : (r == 1 ? sAR1 : (r == 2 ? sAR2 : sAR3)); };
  auto rows_vr = [&](int r) -> float4* { return r == 0 ? sVR0 : (r == 1 ? sVR1 : (r == 2 ? sVR2 : sVR3)); };

  // Parallel-in-time mode: this workgroup's chain and segment.
  const int nchains = sg.pr ? static_cast<int>(gridDim.x) / sg.nseg : static_cast<int>(gridDim.x);
  const int seg = sg.pr ? static_cast<int>(blockIdx.x) / nchains : 0;
  const int64_t chain = sg.pr ? static_cast<int64_t>(blockIdx.x) % nchains : static_cast<int64_t>(blockIdx.x);
  if (sg.pr && sg.conv && sg.conv[chain]) return;   // uniform: its segment starts have converged
  const int64_t pidx = chain * sg.nseg + seg;        // (chain, segment) record index
  if (sg.pr && sg.active && !sg.active[pidx]) return;   // uniform: this segment's start has not moved
  // The wave index is uniform; saying so keeps LDS destinations and buffer
  // descriptors derived from it in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool rwave = w == 0;
  const int m = (w + 3) & 3;                           // product wave index (waves 1..4 -> 0..3)
  const int ti = m >> 1, tj = m & 1;                   // product wave's S tile
  const int col = tj * 32 + (lane & 31);
  const float cap2 = cap * cap;
  const int nblk = pl.nblk;
  const int64_t blk0 = chain * nblk;
  const int b_lo = sg.pr ? sg.bnd[seg] : sg.b_lo, b_hi = sg.pr ? sg.bnd[seg + 1] : sg.b_hi;

  // Buffer-to-LDS copies: this wave takes pieces m, m+4, ...; vo32 / vo16
  // are a lane's source offsets within a piece (fp32 / bf16 rows).
  auto dma_mat = [&](const float* g, int bytes, float4* dst, int vo32) {
    const auto r = make_rsrc(g, bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_piece(r, reinterpret_cast<char*>(dst), m + 4 * i, vo32);
  };
  auto dma_rows = [&](int j, float4* ar, float4* vr, int lane) {
    const int vo32 = (lane >> 4) * 256 + (((lane & 15) ^ (4 * m + (lane >> 4))) << 4);
    const int vo16 = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
    const int tcount = min(kLb, pl.T - j * kLb);
    const int64_t row0 = chain * pl.T + j * kLb;
    dma_mat(pl.alpha + row0 * kD, tcount * kD * 4, ar, vo32);
    const auto r = make_rsrc(static_cast<const TIn*>(pl.v) + row0 * kD, tcount * kD * static_cast<int>(sizeof(TIn)));
    if constexpr (kBf) {
      dma_piece(r, reinterpret_cast<char*>(vr), m, vo16);
      dma_piece(r, reinterpret_cast<char*>(vr), m + 4, vo16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma_piece(r, reinterpret_cast<char*>(vr), m + 4 * i, vo32);
    }
  };
  // The pack and Kx of block j: pieces m, m+4, ... when a product wave calls
  // it (m = 0..3, the prologue), every piece when the recursion wave does
  // (all = true).
  auto dma_kernels = [&](int j, float4* ck, float4* kx, int lane, auto all) {
    constexpr bool kAll = decltype(all)::value;
    const int p0 = kAll ? 0 : m, dp = kAll ? 1 : 4;
    const auto r = make_rsrc(pl.Kmat + (blk0 + j) * kPackFloats, kPackFloats * 4);
#pragma unroll
    for (int p = p0; p < kPackPieces; p += dp) dma_piece(r, reinterpret_cast<char*>(ck), p, 16 * lane);
    if (j > b_lo) {
      const auto rx = make_rsrc(pl.Kcross + (blk0 + j) * kLb * kLb, kLb * kLb * 4);
#pragma unroll
      for (int p = p0; p < 16; p += dp)
        dma_piece(rx, reinterpret_cast<char*>(kx), p,
                  (lane >> 4) * 256 + (((lane & 15) ^ ((4 * p + (lane >> 4)) & 15)) << 4));
    }
  };

  f32x16 X = zero16();
  UpdFrags<TIn> fr;
  UpdOffsets uoff;   // loop-invariant LDS offsets of the update's column reads
  uoff.init(ti, tj, lane);
  float nvec = 0.f, N = 0.f, Nstart = 0.f, lsum = 0.f;
  int fires = 0, first = -1;
  bool bad = false;

  // ---- prologue: continue from S and n at block b_lo -------------------------
  if (rwave) {
    nvec = sg.pr ? sg.n_in[pidx * kD + lane] : sg.n_in[chain * sg.n_in_stride + lane];
    if (b_lo > 0 && !sg.pr) {
      fires = sg.counters[chain * 2];
      first = sg.counters[chain * 2 + 1];
    }
  } else {
    const float* s0 = sg.pr ? sg.S_in + pidx * kD * kD : sg.S_in + chain * sg.S_in_stride;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      X[s] = s0[(ti * 32 + acc_row(s, h)) * kD + col];
      part = fmaf(X[s], X[s], part);
    }
    part = wave_sum(part);
    if (lane == 0) sRed[m] = part;
    dma_kernels(b_lo, sCK0, sKX0, lane, std::false_type{});
    dma_rows(b_lo, sAR0, sVR0, lane);
    if (b_lo + 1 < b_hi) dma_rows(b_lo + 1, sAR1, sVR1, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (!rwave)
    bilinear_terms<TIn>(X, reinterpret_cast<const char*>(sVR0), reinterpret_cast<const float*>(sAR0), sH[0] + m * kLb,
                        ti, tj, lane);
  __syncthreads();
  N = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);

  // ---- one block; RG (compile time) is the row generation of block b, and
  // its parity the generation of the pack and of the per-block LDS outputs.
  auto step = [&](auto rgc, int b) {
    constexpr int RG = decltype(rgc)::value;
    constexpr int RGp1 = (RG + 1) % kRowGens, RGp2 = (RG + 2) % kRowGens;
    constexpr int RGm1 = (RG + kRowGens - 1) % kRowGens;
    constexpr int g = RG & 1;   // = (b - b_lo) & 1: parity relative to the segment start
    const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
    // A fresh copy of the lane index per block keeps the many lane-dependent
    // LDS addresses from being hoisted out of the loop (and spilled).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (rwave) {
      const int t = ln;
      // The product waves carry the longer share of a block, so this wave
      // also copies the next block's pack and Kx (only it reads them) and
      // stores its own per-block outputs.  Its copies for this block were
      // issued one block ago; wait for them before issuing the next ones.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (b + 1 < b_hi) dma_kernels(b + 1, g ? sCK0 : sCK1, g ? sKX0 : sKX1, ln, std::true_type{});
      const float* CK = reinterpret_cast<const float*>(g ? sCK1 : sCK0);
      const int tri = t * (t + 1) / 2;   // row t of the pack's triangle
      const float e_t = CK[kPackE + t], ks = CK[kPackKs + t];
      const float* hr = sH[g];
      // v_t^T S_b alpha_t, the one-block lag repaired with the cross kernel.
      float acc = (hr[t] + hr[kLb + t]) + (hr[2 * kLb + t] + hr[3 * kLb + t]);
      if (b > b_lo) {
        const float se = sSig[g ^ 1];
        // |S|^2 is carried through the recursion; re-anchor it on the exact
        // norm of S_{b-1} as the product waves hold it (the carried value
        // depends on the block-start norm linearly, with factor sigma_end^2).
        const float* np = sNrm[g ^ 1];
        N = fmaf(se * se, ((np[0] + np[1]) + (np[2] + np[3])) - Nstart, N);
        const float* KX = reinterpret_cast<const float*>(g ? sKX1 : sKX0);
        const float* wprev = sW[g ^ 1];
        float cx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float4 xv[8], wv[8];   // all reads of a half before its sums
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            xv[c] = *reinterpret_cast<const float4*>(KX + swz32(t, 32 * half + 4 * c));
            wv[c] = *reinterpret_cast<const float4*>(wprev + 32 * half + 4 * c);
          }
#pragma unroll
          for (int c = 0; c < 8; ++c)
            cx[c & 3] = fmaf(xv[c].x, wv[c].x, fmaf(xv[c].y, wv[c].y, fmaf(xv[c].z, wv[c].z, fmaf(xv[c].w, wv[c].w, cx[c & 3]))));
        }
        acc = fmaf(se, acc, (cx[0] + cx[1]) + (cx[2] + cx[3]));
      }
      Nstart = N;
      const float nstart = nvec;   // n at the block start
      const float own = CK[tri + t];   // sum_{s<t} K(t,s)
      // Cap recursion by rounds: each round assumes no fire for the rest of
      // the block, and the first token whose norm would exceed the cap ends it.
      const uint64_t valid = tcount >= 64 ? ~0ull : ((1ull << tcount) - 1ull);
      float base = 0.f, lprev_t = 0.f, l_t = 0.f, L = 0.f;
      int s0 = 0;
      while (s0 < tcount) {
        const bool act = t >= s0 && t < tcount;
        const float gg = acc + (own - base);
        const float npre = N + wave_incl_scan(act ? fmaf(2.f, gg, e_t) : 0.f, t);
        const uint64_t over = cap_on ? (__ballot(npre > cap2) & valid & (~0ull << s0)) : 0ull;
        if (over == 0) {
          N = readlane_f(npre, tcount - 1);
          break;
        }
        const int f = __ffsll(static_cast<long long>(over)) - 1;
        const float nf = readlane_f(npre, f);
        const float c = cap * __builtin_amdgcn_rsqf(nf);
        const float lg = __builtin_amdgcn_logf(c);   // log2
        // sum_{s<=f} K(t,s), needed on lanes t > f only (others read their own entry)
        const float cf = CK[tri + min(f + 1, t)];
        acc = (t > f) ? c * (acc + (cf - base)) : acc;
        lprev_t += (t > f) ? lg : 0.f;
        l_t += (t >= f) ? lg : 0.f;
        L += lg;
        N = c * c * nf;
        base = cf;
        if (first < 0) first = tb + f;
        ++fires;
        s0 = f + 1;
      }
      lsum += L;
      sW[g][t] = (t < tcount) ? exp2f(L - lprev_t) : 0.f;
      if (t == 0) sSig[g] = exp2f(L);
      {
        const int64_t r0 = chain * pl.T + tb;
        const auto rw = make_rsrc(pl.wsig + 2 * r0, 2 * tcount * 4);
        buf_store_f32(rw, 8 * t, lprev_t);
        buf_store_f32(rw, 8 * t + 4, l_t);
        pl.nblock[(blk0 + b) * kD + t] = nstart;
      }
      nvec += ks;
    } else {
      // Rows of block b+2 into the generation whose last reader was the
      // previous block.
      if (b + 2 < b_hi) dma_rows(b + 2, rows_ar(RGp2), rows_vr(RGp2), ln);
      if (b > b_lo) {
        // S_b = sigma_end(b-1) S_{b-1} + V^T diag(w) A_hat over block b-1.
        if constexpr (kBf)
          rank_update_lds(X, reinterpret_cast<const char*>(rows_vr(RGm1)), reinterpret_cast<const char*>(rows_ar(RGm1)),
                          uoff, sW[g ^ 1], sSig[g ^ 1], ln >> 5);
        else
          rank_update<TIn>(X, fr, sW[g ^ 1], sSig[g ^ 1], ln >> 5);
      }
      {
        const int xs_off = ((ti * 32 + 4 * (ln >> 5)) * kD + tj * 32 + (ln & 31)) * 4;
        const auto rs = make_rsrc(pl.Xsnap + (blk0 + b) * kD * kD, kD * kD * 4);
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          buf_store_f32(rs, xs_off + acc_row(s, 0) * kD * 4, X[s]);
          part = fmaf(X[s], X[s], part);
        }
        part = wave_sum(part);
        if (ln == 0) sNrm[g][m] = part;
      }
      if (b + 1 < b_hi)
        bilinear_terms<TIn>(X, reinterpret_cast<const char*>(rows_vr(RGp1)), reinterpret_cast<const float*>(rows_ar(RGp1)),
                            sH[g ^ 1] + m * kLb, ti, tj, ln);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies have landed
      // fp32 storage: block b's update operands, for the next block's update,
      // loaded only now so that they are not live through the bilinear terms
      // (they land while the recursion wave runs the next block).
      if constexpr (!kBf) fr.load(pl, blk0 + b, ti, tj, ln);
    }
    // The block's closing barrier, without the fence of __syncthreads: that
    // fence would also hold the recursion wave until its Kx copies land.
    // LDS writes are complete first; the asm is a compiler memory barrier.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  for (int b = b_lo; b < b_hi; b += kRowGens) {   // block b_lo has relative parity 0
    step(std::integral_constant<int, 0>{}, b);
    if (b + 1 < b_hi) step(std::integral_constant<int, 1>{}, b + 1);
    if constexpr (kRowGens == 4) {
      if (b + 2 < b_hi) step(std::integral_constant<int, 2>{}, b + 2);
      if (b + 3 < b_hi) step(std::integral_constant<int, 3>{}, b + 3);
    }
  }

  // ---- epilogue: the segment's last block update ----------------------------
  if (!rwave) {
    // The last block's LDS outputs sit in the buffer of its parity relative
    // to b_lo, which may be odd (a remainder shared between two segments).
    const int g = (b_hi - 1 - b_lo) & 1;
    if constexpr (kBf) {
      const int r = (b_hi - 1 - b_lo) % kRowGens;
      rank_update_lds(X, reinterpret_cast<const char*>(rows_vr(r)), reinterpret_cast<const char*>(rows_ar(r)), uoff,
                      sW[g], sSig[g], h);
    } else {
      rank_update<TIn>(X, fr, sW[g], sSig[g], h);
    }
    if (sg.pr) {
      // S at the segment's end, for the sweep; the last segment's is S_T.
      float* fo = sg.F + pidx * kD * kD;
#pragma unroll
      for (int s = 0; s < 16; ++s) fo[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
      if (seg + 1 == sg.nseg) {
        float* st = S_T + chain * kD * kD;
#pragma unroll
        for (int s = 0; s < 16; ++s) st[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
      }
    } else if (sg.last) {
      float* st = S_T + chain * kD * kD;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        st[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
        bad |= !isfinite(X[s]);
      }
    } else {
      // S at the next segment's first block (also that block's readout input).
      float* st = pl.Xsnap + (blk0 + b_hi) * kD * kD;
#pragma unroll
      for (int s = 0; s < 16; ++s) st[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
    }
  } else if (sg.pr) {
    if (seg + 1 == sg.nseg) n_T[chain * kD + lane] = nvec;
    if (lane == 0) {
      float* rc = sg.rec + pidx * 4;
      rc[0] = lsum;
      rc[1] = static_cast<float>(fires);
      rc[2] = static_cast<float>(first);
      rc[3] = 0.f;
    }
  } else if (sg.last) {
    n_T[chain * kD + lane] = nvec;
    bad |= !isfinite(nvec);
  } else {
    sg.n_carry[chain * kD + lane] = nvec;
    if (lane == 0) {
      sg.counters[chain * 2] = fires;
      sg.counters[chain * 2 + 1] = first;
    }
  }
  if (!sg.last || sg.pr) return;   // uniform
  const bool wave_bad = __any(bad);
  if (lane == 0) sRed[w] = wave_bad ? 1.f : 0.f;
  __syncthreads();
  if (tid == 0 && stats) {
    bool any_bad = chain_info[chain * 4 + kInfoNonfinite] != 0;
    for (int ww = 0; ww < 5; ++ww) any_bad |= sRed[ww] != 0.f;
    int32_t* s = stats + chain * 4;
    s[0] = chain_info[chain * 4 + kInfoGuard];
    s[1] = fires;
    s[2] = any_bad ? 1 : 0;
    s[3] = first;
  }
}

// ---- readout: o for every block in parallel --------------------------------
// Per block, with tiles tt (tokens) x ti (features) of 32 x 32, one per wave:
//   o_t = (sigma_t (S_b q_t) + sum_{s<=t} P'[t][s] v_s) / den_t,
//   P'[t][s] = (alpha_s . q_t) sigma_t / sigma_{s-1},  den_t = q_t . n_b + ld_t + den_eps.
// The three products run on the bf16 matrix cores with three-term splits of
// their fp32 operands (q and v are exact when stored as bf16).  Wave (tt, ts)
// with ts <= tt computes the P' tile (tt, ts); the tile above the diagonal
// is zero.  LDS rows are padded so row-per-lane 16-byte reads do not collide.
template <typename TIn>
struct ReadoutLds {
  static constexpr int kQd = sizeof(TIn) == 2 ? 72 : 68;   // row stride (elements) of q and v^T rows
  // q rows and v^T, then two swizzled [64][64] fp32 matrices (S_b rows, which
  // later stage the outputs; alpha_hat rows, which later hold P'), then four
  // vectors: 51.4 KiB with bf16 storage, three workgroups per compute unit.
  static constexpr size_t kBytes = 2 * kLb * kQd * sizeof(TIn) + 2 * kLb * kD * sizeof(float) + 4 * kLb * sizeof(float);
};

// Eight consecutive values (columns c0 .. c0 + 7, c0 a multiple of 8) of row r
// of a swizzled [64][64] fp32 LDS matrix, as a three-term split.
__device__ __forceinline__ Split3 swz_operand8(const float* m, int r, int c0) {
  const float4 a = *reinterpret_cast<const float4*>(m + swz32(r, c0));
  const float4 b = *reinterpret_cast<const float4*>(m + swz32(r, c0 + 4));
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return split3(x);
}

template <typename TIn>
__device__ __forceinline__ void readout_block(const StatePlan& pl, const TIn* __restrict__ q, TIn* __restrict__ o,
                                              float den_eps, int32_t* __restrict__ chain_info, int b_lo, int nb,
                                              int64_t item) {
  constexpr int kQd = ReadoutLds<TIn>::kQd;
  extern __shared__ float4 smem4[];
  TIn* Qs = reinterpret_cast<TIn*>(smem4);          // [64 t][kQd] q rows
  TIn* Vt = Qs + kLb * kQd;                         // [64 i][kQd] v transposed (rows = features)
  float* Xs = reinterpret_cast<float*>(Vt + kD * kQd);   // swizzled [64 i][64] S_b rows; later the outputs
  float* As = Xs + kD * kD;                         // swizzled [64 s][64] alpha_hat rows; later P'
  float* Ps = As;
  float* wl = As + kLb * kD;                        // [64] log2 sigma_{s-1} (block-local)
  float* sl = wl + kLb;                             // [64] log2 sigma_t
  float* dl = sl + kLb;                             // [64] 1 / den_t
  float* nl = dl + kLb;                             // [64] n at the block start
  const int64_t chain = item / nb;
  const int b = b_lo + static_cast<int>(item % nb);
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
  const int64_t row0 = chain * pl.T + tb;
  const int64_t blk = chain * pl.nblk + b;
  constexpr int EPV = 16 / static_cast<int>(sizeof(TIn));   // elements per 16 bytes
  float ldv = 0.f;
  {
    // Every global load of the block first, then the LDS stores: q rows,
    // v^T (v is read as rows and written transposed), S_b, alpha_hat rows.
    TileRegs<TIn> rq, rv;
    TileRegs<float> rx, ra;
    rq.load(q + row0 * kD, tcount, tid);
    rv.load(static_cast<const TIn*>(pl.v) + row0 * kD, tcount, tid);
    rx.load(pl.Xsnap + blk * kD * kD, kD, tid);
    ra.load(pl.alpha + row0 * kD, tcount, tid);
    float w0 = 0.f, w1 = 0.f, nb0 = 0.f;
    if (tid < kLb) {
      const bool ok = tid < tcount;
      w0 = ok ? pl.wsig[2 * (row0 + tid)] : 0.f;
      w1 = ok ? pl.wsig[2 * (row0 + tid) + 1] : 0.f;
      nb0 = pl.nblock[blk * kD + tid];
      ldv = ok ? pl.ld[row0 + tid] : 0.f;
    }
    rq.store_rows(Qs, kQd, tid);
#pragma unroll
    for (int j = 0; j < TileRegs<TIn>::N; ++j) {
      const int e = tid + j * kThreads, r = e / TileRegs<TIn>::PPR, c = (e % TileRegs<TIn>::PPR) * EPV;
      const TIn* xe = reinterpret_cast<const TIn*>(&rv.r[j]);
#pragma unroll
      for (int k = 0; k < EPV; ++k) Vt[(c + k) * kQd + r] = xe[k];
    }
#pragma unroll
    for (int j = 0; j < TileRegs<float>::N; ++j) {
      const int e = tid + j * kThreads, r = e / TileRegs<float>::PPR, c = (e % TileRegs<float>::PPR) * 4;
      *reinterpret_cast<uint4*>(Xs + swz32(r, c)) = rx.r[j];
      *reinterpret_cast<uint4*>(As + swz32(r, c)) = ra.r[j];
    }
    if (tid < kLb) {
      wl[tid] = w0;
      sl[tid] = w1;
      nl[tid] = nb0;
    }
  }
  lds_barrier();
  if (tid < kLb) {
    float acc = 0.f;
    for (int i = 0; i < kD; ++i) acc = fmaf(Elem<TIn>::load(Qs + tid * kQd + i), nl[i], acc);
    dl[tid] = 1.f / (acc + ldv + den_eps);   // the outputs take 1 / den_t
  }

  const int tt = w >> 1, ti = w & 1;   // this wave's output tile; its P' tile is (tt, ts = ti)
  const int rl = lane & 31;
  // P'(tt, ts) for ts <= tt: A = q rows of tile tt, B[k=j][n=s] = alpha_hat[s][j].
  f32x16 P = zero16();
  if (ti <= tt) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const auto a = operand8(Qs + (tt * 32 + rl) * kQd + 16 * kb + 8 * h);
      P = mma_split(a, swz_operand8(As, ti * 32 + rl, 16 * kb + 8 * h), P);
    }
  }
  // sigma_t S_b q_t: A = q rows, B[k=j][n=i] = S_b[i][j].
  f32x16 Z = zero16();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const auto a = operand8(Qs + (tt * 32 + rl) * kQd + 16 * kb + 8 * h);
    Z = mma_split(a, swz_operand8(Xs, ti * 32 + rl, 16 * kb + 8 * h), Z);
  }
#pragma unroll
  for (int a = 0; a < 16; ++a) Z[a] *= exp2f(sl[tt * 32 + acc_row(a, h)]);
  lds_barrier();   // every wave is done with alpha_hat and S_b; P' takes alpha_hat's place
  if (ti <= tt) {
    const int s = ti * 32 + rl;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int t = tt * 32 + acc_row(a, h);
      Ps[swz32(t, s)] = (s <= t) ? P[a] * exp2f(sl[t] - wl[s]) : 0.f;
    }
  }
  lds_barrier();
  // + sum_s P'[t][s] v_s over the tiles ts <= tt: A = P' rows, B[k=s][n=i] = v^T[i][s].
  for (int ts = 0; ts <= tt; ++ts) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const Split3 a = swz_operand8(Ps, tt * 32 + rl, ts * 32 + 16 * kb + 8 * h);
      const auto bb = operand8(Vt + (ti * 32 + rl) * kQd + ts * 32 + 16 * kb + 8 * h);
      Z = mma_split(a, bb, Z);
    }
  }
  bool bad = false;
  const int fcol = ti * 32 + rl;
  // The outputs are staged in S_b's place (free since the barrier above).
#pragma unroll
  for (int a = 0; a < 16; ++a) {
    const int t = tt * 32 + acc_row(a, h);
    const float ov = Z[a] * dl[t];
    bad |= t < tcount && !isfinite(ov);
    Xs[swz32(t, fcol)] = ov;
  }
  if (__any(bad) && lane == 0) atomicOr(chain_info + chain * 4 + kInfoNonfinite, 1);
  lds_barrier();
  // Whole 16-byte pieces of o rows from the staged block.
  constexpr int PPR = kD / EPV;
#pragma unroll
  for (int e = tid; e < kLb * PPR; e += kThreads) {
    const int t = e / PPR, c = (e % PPR) * EPV;
    if (t >= tcount) continue;
    uint4 wv;
    if constexpr (EPV == 4) {
      wv = *reinterpret_cast<const uint4*>(Xs + swz32(t, c));
    } else {
      const float4 lo = *reinterpret_cast<const float4*>(Xs + swz32(t, c));
      const float4 hi = *reinterpret_cast<const float4*>(Xs + swz32(t, c + 4));
      const float src[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t hw[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2)
        hw[k2] = static_cast<uint32_t>(f32_to_bf16(src[2 * k2])) | (static_cast<uint32_t>(f32_to_bf16(src[2 * k2 + 1])) << 16);
      wv = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
    *reinterpret_cast<uint4*>(o + (row0 + t) * kD + c) = wv;
  }
}

// Three workgroups per compute unit with bf16 storage (51.4 KiB of LDS
// each): the register budget is held to three waves per SIMD.
template <typename TIn>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
vla_state_readout_kernel(StatePlan pl, const TIn* __restrict__ q, TIn* __restrict__ o, float den_eps,
                         int32_t* __restrict__ chain_info, int b_lo, int nb, int64_t items) {
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    readout_block<TIn>(pl, q, o, den_eps, chain_info, b_lo, nb, item);
    lds_barrier();   // LDS is restaged by the next item
  }
}

}  // namespace

// ---- parallel-in-time state pass: initial segment starts, the sweep, stats ----
// The state recurrence over a segment of blocks is a map of its starting S
// (the cap makes it nonlinear, but only through the per-token scales).  All
// segments of all chains run at once from guessed starts (the chain kernel in
// parallel-in-time mode); a sweep per chain then corrects the guesses in
// segment order with a cheap linear model of each segment's map around its
// last pass and the pass's exact end state (a parareal iteration):
//     S'_{j+1} = F_j(S_j) + G_j(S'_j - S_j).
// Once the cap binds, |S| stays at the cap, so a change of the start along S
// is undone by the next fire while a change across it is carried along as
// the state turns; G_j models exactly that: sigma_j (the segment's total cap
// scale) times the rotation taking the start's direction a to the end's b in
// their common plane, after removing the component along a.  Without a fire
// in the segment G_j = identity.  A segment's start is exact once every
// earlier segment's is, so with nseg segments the iteration is exact after
// nseg passes; it stops as soon as no start moves by more than tol (relative).
// The first guesses come from the plain sums of v alpha_hat^T over four
// sub-steps of every segment (a parallel kernel), chained from the true start
// with the cap applied after each sub-step.

// The normaliser at every segment start (n is linear: n0 plus the key sums
// of the blocks before).  One workgroup per chain.
__global__ void __launch_bounds__(1024) vla_para_init_kernel(ParaPlan pp, StatePlan pl, const float* __restrict__ n_init,
                                                             float* __restrict__ n_seg) {
  __shared__ float part[kMaxParaSegs][kD];
  const int64_t c = blockIdx.x;
  const int tid = threadIdx.x, G = pp.nseg;
  if (tid == 0) pp.conv[c] = 0;
  const int sg = tid >> 6, f = tid & 63;
  if (sg < G) {
    // Eight loads in flight at a time, added in block order.
    const float* ks = pl.Kmat + c * pl.nblk * kPackFloats + kPackKs + f;
    const int be = pp.bnd[sg + 1];
    float acc = 0.f;
    int b = pp.bnd[sg];
    for (; b + 8 <= be; b += 8) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = ks[static_cast<int64_t>(b + i) * kPackFloats];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += x[i];
    }
    for (; b < be; ++b) acc += ks[static_cast<int64_t>(b) * kPackFloats];
    part[sg][f] = acc;
  }
  __syncthreads();
  if (sg < G) {
    float n = n_init[c * kD + f];
    for (int j = 0; j < sg; ++j) n += part[j][f];
    n_seg[(c * G + sg) * kD + f] = n;
  }
}

// Plain sums sum_t v_t alpha_hat_t^T over the blocks of one sub-step of one
// segment: workgroup (c, j, sub), four waves each owning a 32 x 32 tile.
// Block rows are staged in LDS (the next block's held in registers while the
// current one is summed); the products contract over tokens, so the operands
// are LDS column reads: v exact in bf16 (three-term splits for fp32 storage),
// alpha_hat through three-term splits.
// (Four waves per SIMD: the 1,024 workgroups of 16 chains x 16 segments x 4
// sub-steps then run in one round on 256 compute units.)
template <typename TIn>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
vla_para_sums_kernel(ParaPlan pp, StatePlan pl) {
  constexpr int kVd = sizeof(TIn) == 2 ? 72 : 68;   // row stride of the v rows (elements)
  __shared__ TIn Vs[kLb * kVd];
  __shared__ float As[kLb * kLd];
  const int G = pp.nseg;
  const int sub = static_cast<int>(blockIdx.x % kParaSub);
  const int j = static_cast<int>((blockIdx.x / kParaSub) % G);
  const int64_t c = blockIdx.x / (kParaSub * G);
  const int blo = pp.bnd[j], len = pp.bnd[j + 1] - blo;
  const int nsub = len < kParaSub ? len : kParaSub;
  if (sub >= nsub) return;   // uniform
  const int b0 = blo + (sub * len) / nsub, b1 = blo + ((sub + 1) * len) / nsub;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, rl = lane & 31;
  const int m = __builtin_amdgcn_readfirstlane(tid >> 6), ti = m >> 1, tj = m & 1;
  const TIn* v = static_cast<const TIn*>(pl.v);
  TileRegs<TIn> rv;
  TileRegs<float> ra;
  auto load = [&](int b) {
    const int tcount = min(kLb, pl.T - b * kLb);
    const int64_t row0 = c * pl.T + static_cast<int64_t>(b) * kLb;
    rv.load(v + row0 * kD, tcount, tid);
    ra.load(pl.alpha + row0 * kD, tcount, tid);
  };
  f32x16 X = zero16();
  load(b0);
  for (int b = b0; b < b1; ++b) {
    rv.store_rows(Vs, kVd, tid);
    ra.store_f32(As, tid);
    lds_barrier();
    if (b + 1 < b1) load(b + 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float ax[8];
      TIn vx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 16 * kb + 8 * h + e;
        vx[e] = Vs[t * kVd + ti * 32 + rl];
        ax[e] = As[t * kLd + tj * 32 + rl];
      }
      const Split3 B = split3(ax);
      if constexpr (sizeof(TIn) == 2) {
        const uint4 pv = make_uint4(vx[0] | (static_cast<uint32_t>(vx[1]) << 16), vx[2] | (static_cast<uint32_t>(vx[3]) << 16),
                                    vx[4] | (static_cast<uint32_t>(vx[5]) << 16), vx[6] | (static_cast<uint32_t>(vx[7]) << 16));
        X = mma_split(__builtin_bit_cast(bf16x8, pv), B, X);
      } else {
        float fx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) fx[e] = vx[e];
        X = mma_split(split3(fx), B, X);
      }
    }
    lds_barrier();
  }
  float* out = pp.P + ((c * G + j) * kParaSub + sub) * kD * kD;
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) out[(ti * 32 + acc_row(s2, h)) * kD + tj * 32 + rl] = X[s2];
}

constexpr int kSweepThreads = 512;                      // 8 waves: two per SIMD
constexpr int kSweepWaves = kSweepThreads / 64;
constexpr int kSweepEpt = kD * kD / kSweepThreads;      // matrix entries per thread

// Sums of the first N of 8 values over the workgroup; red holds
// [2][kSweepWaves][8] (alternating halves, so one barrier per sum suffices).
// The barrier waits for LDS only: the caller's global loads of the next step
// stay in flight.
template <int N>
__device__ __forceinline__ void para_sum8(float (&x)[8], float* red, int buf, int tid) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = wave_sum(x[i]);   // DPP row sums and readlanes, no LDS
  if ((tid & 63) == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) red[(buf * kSweepWaves + (tid >> 6)) * 8 + i] = x[i];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float* r = red + buf * kSweepWaves * 8 + i;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kSweepWaves; ++w) t += r[8 * w];
    x[i] = t;
  }
}

// The sweep over one chain's segments (one workgroup per chain, each thread
// kSweepEpt consecutive entries of every 64 x 64 matrix).  first: the sweep
// before the first pass (plain sums chained with the cap at sub-step ends).
__global__ void __launch_bounds__(kSweepThreads) vla_para_sweep_kernel(ParaPlan pp, int first) {
  constexpr int E = kSweepEpt;
  __shared__ float red[2 * kSweepWaves * 8];
  __shared__ float srec[kMaxParaSegs * 4];   // the segments' records, read once
  const int64_t c = blockIdx.x;
  if (!first && pp.conv[c]) return;   // uniform
  const int tid = threadIdx.x, G = pp.nseg;
  if (!first && tid < G * 4) srec[tid] = pp.rec[c * G * 4 + tid];
  const int64_t base = c * G * kD * kD;
  const int e0 = tid * E;
  float nw[E], od[E], fj[E];
  auto load = [](const float* p, float (&x)[E]) {
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(p)[q];
      x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
    }
  };
  load(pp.S_init + c * kD * kD + e0, nw);
  float maxchg = 0.f;
  // Segment j's start and end are loaded one step ahead (they do not depend
  // on the sweep), so their latency hides behind step j - 1.
  float odn[E], fjn[E];
  if (!first) {
    load(pp.Sit + base + e0, odn);   // segment 0's start (the true one)
    load(pp.F + base + e0, fjn);
  }
  __syncthreads();   // srec
  int nred = 0;      // sums so far: consecutive sums alternate halves of red
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      od[i] = odn[i];
      fj[i] = fjn[i];
    }
    if (!first && j + 1 < G) {   // the first sweep reads neither starts nor ends
      load(pp.Sit + base + (j + 1) * kD * kD + e0, odn);
      load(pp.F + base + (j + 1) * kD * kD + e0, fjn);
    }
    float nx[E];
    float chg_j = 0.f;   // relative move of this segment's start
    if (first) {
      // The segment's plain sums over its sub-steps added to the running
      // state, the cap applied after each (each sub-step's sum is loaded one
      // sub-step ahead).
      const int len = pp.bnd[j + 1] - pp.bnd[j];
      const int nsub = len < kParaSub ? len : kParaSub;
      const float* pj = pp.P + (c * G + j) * kParaSub * kD * kD + e0;
      float cur[E], nxt[E];
#pragma unroll
      for (int i = 0; i < E; ++i) nx[i] = nw[i];
      load(pj, nxt);
      for (int sub = 0; sub < nsub; ++sub) {
#pragma unroll
        for (int i = 0; i < E; ++i) cur[i] = nxt[i];
        if (sub + 1 < nsub) load(pj + (sub + 1) * kD * kD, nxt);
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < E; ++i) {
          nx[i] += cur[i];
          x[0] = fmaf(nx[i], nx[i], x[0]);
        }
        para_sum8<1>(x, red, nred++ & 1, tid);
        const float nrm = sqrtf(x[0]);
        const float sc = (pp.cap_on && nrm > pp.cap) ? pp.cap / nrm : 1.f;
#pragma unroll
        for (int i = 0; i < E; ++i) nx[i] *= sc;
      }
    } else {
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float Ev[E];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        Ev[i] = nw[i] - od[i];
        x[0] = fmaf(Ev[i], od[i], x[0]);   // <E, old>
        x[1] = fmaf(Ev[i], fj[i], x[1]);   // <E, F>
        x[2] = fmaf(Ev[i], Ev[i], x[2]);   // |E|^2
        x[3] = fmaf(nw[i], nw[i], x[3]);   // |new|^2
        x[4] = fmaf(od[i], fj[i], x[4]);   // <old, F>
        x[5] = fmaf(od[i], od[i], x[5]);   // |old|^2
        x[6] = fmaf(fj[i], fj[i], x[6]);   // |F|^2
      }
      para_sum8<7>(x, red, nred++ & 1, tid);
      const float sig = exp2f(srec[4 * j]);   // the segment's total cap scale
      const bool fired = srec[4 * j + 1] > 0.f;
      chg_j = sqrtf(x[2]) / fmaxf(sqrtf(x[3]), 1e-30f);
      chg_j = chg_j == chg_j ? chg_j : 3.0e38f;   // NaN counts as moved
      maxchg = fmaxf(maxchg, chg_j);
      if (fired && x[5] > 0.f && x[6] > 0.f) {
        const float no = sqrtf(x[5]), nf = sqrtf(x[6]);
        const float ia = 1.f / no, ib = 1.f / nf;
        const float cab = x[4] * ia * ib;          // cos of the angle between start and end
        const float ea = x[0] * ia, eb = x[1] * ib;
        if (1.f + cab > 1e-3f) {
          const float g = (ea + eb) / (1.f + cab);
#pragma unroll
          for (int i = 0; i < E; ++i) {
            const float av = od[i] * ia, bv = fj[i] * ib;
            // R E - (E.a) b with R the rotation a -> b: E - g (a + b) + 2 (E.a) b - (E.a) b
            nx[i] = fmaf(sig, fmaf(ea, bv, fmaf(-g, av + bv, Ev[i])), fj[i]);
          }
        } else {   // (start and end nearly opposite: remove the component along the end only)
#pragma unroll
          for (int i = 0; i < E; ++i) nx[i] = fmaf(sig, fmaf(-eb, fj[i] * ib, Ev[i]), fj[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) nx[i] = fmaf(sig, Ev[i], fj[i]);
      }
    }
    // The first pass runs every segment; a later one reruns a segment only
    // if its start moved by more than tol_skip (one left out keeps the start
    // its results came from).  Segment 0 starts at the true S: after the
    // first pass it never reruns.
    const bool run = first || (j > 0 && chg_j > pp.tol_skip);
    if (tid == 0) pp.active[c * G + j] = run ? 1 : 0;
    if (run) {
      float4* dst = reinterpret_cast<float4*>(pp.Sit + base + j * kD * kD + e0);
#pragma unroll
      for (int q = 0; q < E / 4; ++q) dst[q] = make_float4(nw[4 * q], nw[4 * q + 1], nw[4 * q + 2], nw[4 * q + 3]);
    }
#pragma unroll
    for (int i = 0; i < E; ++i) nw[i] = nx[i];
  }
  if (!first && tid == 0) {
    const bool done = maxchg <= pp.tol;
    pp.conv[c] = done ? 1 : 0;
    if (!done && pp.iter_last) pp.chain_info[c * 4 + kInfoFallback] = 1;
  }
}

// Per-chain statistics of the parallel-in-time pass: cap fires summed over
// segments, the first one, non-finite final state or inverse pass.
__global__ void __launch_bounds__(256) vla_para_stats_kernel(ParaPlan pp, const float* __restrict__ S_T,
                                                             const float* __restrict__ n_T, int32_t* __restrict__ stats) {
  __shared__ int bad_any;
  __shared__ int s_fires[kMaxParaSegs], s_first[kMaxParaSegs];
  const int64_t c = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) bad_any = 0;
  if (tid < pp.nseg) {   // the segments' records, read in parallel
    const float* rc = pp.rec + (c * pp.nseg + tid) * 4;
    s_fires[tid] = static_cast<int>(rc[1]);
    s_first[tid] = rc[2] >= 0.f ? static_cast<int>(rc[2]) : -1;
  }
  __syncthreads();
  bool bad = false;
  for (int e = tid; e < kD * kD; e += 256) bad |= !isfinite(S_T[c * kD * kD + e]);
  if (tid < kD) bad |= !isfinite(n_T[c * kD + tid]);
  if (bad) atomicOr(&bad_any, 1);
  __syncthreads();
  if (tid == 0) {
    int fires = 0, first = -1;
    for (int j = 0; j < pp.nseg; ++j) {
      fires += s_fires[j];
      if (first < 0) first = s_first[j];
    }
    int32_t* st = stats + c * 4;
    st[0] = pp.chain_info[c * 4 + kInfoGuard];
    st[1] = fires;
    st[2] = (bad_any || pp.chain_info[c * 4 + kInfoNonfinite]) ? 1 : 0;
    st[3] = first;
  }
}

template <typename TIn>
size_t state_prep_lds_bytes() { return PrepLds<TIn>::kBytes; }

template <typename TIn>
size_t state_readout_lds_bytes() { return ReadoutLds<TIn>::kBytes; }

template <typename K>
static void allow_lds(K kernel, size_t bytes) {
  // Raise the dynamic LDS limit of a kernel above the 64 KiB default once.
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes));
}

static void allow_state_lds() {
  static const bool once = [] {
    allow_lds(vla_state_prep_kernel<uint16_t>, state_prep_lds_bytes<uint16_t>());
    allow_lds(vla_state_prep_kernel<float>, state_prep_lds_bytes<float>());
    allow_lds(vla_state_readout_kernel<uint16_t>, state_readout_lds_bytes<uint16_t>());
    allow_lds(vla_state_readout_kernel<float>, state_readout_lds_bytes<float>());
    return true;
  }();
  (void)once;
}

hipError_t launch_state_prep(const StatePlan& pl, const ScanArgs& a, int chains, int b_lo, int nb, int max_wg,
                             hipStream_t stream) {
  if (nb <= 0) return hipSuccess;
  allow_state_lds();
  const int64_t items = static_cast<int64_t>(chains) * nb;
  const unsigned blocks = static_cast<unsigned>(max_wg > 0 ? std::min<int64_t>(items, max_wg) : items);
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_prep_kernel<uint16_t>, dim3(blocks), dim3(kThreads), state_prep_lds_bytes<uint16_t>(),
                       stream, pl, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), b_lo, nb, items);
  else
    hipLaunchKernelGGL(vla_state_prep_kernel<float>, dim3(blocks), dim3(kThreads), state_prep_lds_bytes<float>(), stream,
                       pl, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v), b_lo, nb, items);
  return hipGetLastError();
}

hipError_t launch_para_sums(const ParaPlan& pp, const StatePlan& pl, hipStream_t stream) {
  if (pp.chains <= 0 || pp.nseg < 1 || pp.nseg > kMaxParaSegs) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(pp.chains * pp.nseg * kParaSub));
  if (pl.bf16)
    hipLaunchKernelGGL(vla_para_sums_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, pp, pl);
  else
    hipLaunchKernelGGL(vla_para_sums_kernel<float>, grid, dim3(kThreads), 0, stream, pp, pl);
  return hipGetLastError();
}

hipError_t launch_para_init(const ParaPlan& pp, const StatePlan& pl, const float* n_init, float* n_seg,
                            hipStream_t stream) {
  if (pp.chains <= 0 || pp.nseg < 1 || pp.nseg > kMaxParaSegs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vla_para_init_kernel, dim3(pp.chains), dim3(1024), 0, stream, pp, pl, n_init, n_seg);
  return hipGetLastError();
}

hipError_t launch_para_sweep(const ParaPlan& pp, int first, hipStream_t stream) {
  hipLaunchKernelGGL(vla_para_sweep_kernel, dim3(pp.chains), dim3(kSweepThreads), 0, stream, pp, first);
  return hipGetLastError();
}

hipError_t launch_para_stats(const ParaPlan& pp, const float* S_T, const float* n_T, int32_t* stats,
                             hipStream_t stream) {
  if (!stats) return hipSuccess;
  hipLaunchKernelGGL(vla_para_stats_kernel, dim3(pp.chains), dim3(256), 0, stream, pp, S_T, n_T, stats);
  return hipGetLastError();
}

hipError_t launch_state_chain(const StatePlan& pl, const ChainSeg& sg, const ScanArgs& a, const int32_t* chain_info,
                              int chains, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  hipError_t e = hipSuccess;
  if (sg.pr && (sg.nseg < 1 || sg.nseg > kMaxParaSegs)) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(sg.pr ? chains * sg.nseg : chains);
  if (ev_start && (e = hipEventRecord(ev_start, stream)) != hipSuccess) return e;
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_chain_kernel<uint16_t>, dim3(grid), dim3(kChainThreads), 0, stream, pl, sg, a.S_T,
                       a.n_T, a.stats, chain_info, a.cap, a.cap_on);
  else
    hipLaunchKernelGGL(vla_state_chain_kernel<float>, dim3(grid), dim3(kChainThreads), 0, stream, pl, sg, a.S_T,
                       a.n_T, a.stats, chain_info, a.cap, a.cap_on);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_stop && (e = hipEventRecord(ev_stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_state_readout(const StatePlan& pl, const ScanArgs& a, int32_t* chain_info, int chains, int b_lo,
                                int nb, int max_wg, hipStream_t stream) {
  if (nb <= 0) return hipSuccess;
  allow_state_lds();
  const int64_t items = static_cast<int64_t>(chains) * nb;
  const unsigned blocks = static_cast<unsigned>(max_wg > 0 ? std::min<int64_t>(items, max_wg) : items);
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_readout_kernel<uint16_t>, dim3(blocks), dim3(kThreads),
                       state_readout_lds_bytes<uint16_t>(), stream, pl, static_cast<const uint16_t*>(a.q),
                       static_cast<uint16_t*>(a.o), a.den_eps, chain_info, b_lo, nb, items);
  else
    hipLaunchKernelGGL(vla_state_readout_kernel<float>, dim3(blocks), dim3(kThreads), state_readout_lds_bytes<float>(),
                       stream, pl, static_cast<const float*>(a.q), static_cast<float*>(a.o), a.den_eps, chain_info,
                       b_lo, nb, items);
  return hipGetLastError();
}

}  // namespace vla
