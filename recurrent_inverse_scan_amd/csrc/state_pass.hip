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
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_seq.h"

namespace vla {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;     // head dimension
constexpr int kLb = 64;    // tokens per block
constexpr int kLd = 68;    // LDS row stride in floats (rows of 16 lanes hit distinct banks)
constexpr int kThreads = 256;

__device__ __forceinline__ f32x16 zero16() {
  return f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (within the tile) held by accumulator slot s of a lane in half h.
__device__ __forceinline__ int acc_row(int s, int h) { return 8 * (s / 4) + 4 * h + (s % 4); }

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

// ---- prep: kernel matrix, local normaliser terms, block key sums -----------
// K[t][s] = (v_t.v_s)(alpha_t.alpha_s); ld[t] = sum_{s<=t} k_s.q_t (block-local);
// ksum = sum_t k_t over the block.
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
vla_state_prep_kernel(StatePlan pl, const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v) {
  extern __shared__ float4 smem4[];
  float* Vl = reinterpret_cast<float*>(smem4);
  float* Al = Vl + kLb * kLd;
  float* Ql = Al + kLb * kLd;
  float* Kl = Ql + kLb * kLd;
  const int64_t chain = blockIdx.x / pl.nblk;
  const int b = blockIdx.x % pl.nblk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
  const int64_t row0 = chain * pl.T + tb;
  stage_block<TIn>(Vl, v + row0 * kD, tcount, tid);
  stage_block<float>(Al, pl.alpha + row0 * kD, tcount, tid);
  stage_block<TIn>(Ql, q + row0 * kD, tcount, tid);
  stage_block<TIn>(Kl, k + row0 * kD, tcount, tid);
  __syncthreads();

  const int ti = w >> 1, tj = w & 1;
  f32x16 gv = zero16(), ga = zero16(), pk = zero16();
  mma_rr(gv, Vl + ti * 32 * kLd, Vl + tj * 32 * kLd, lane);
  mma_rr(ga, Al + ti * 32 * kLd, Al + tj * 32 * kLd, lane);
  mma_rr(pk, Ql + ti * 32 * kLd, Kl + tj * 32 * kLd, lane);   // q_t . k_s
  float* Kout = pl.Kmat + (chain * pl.nblk + b) * kLb * kLb;
  const int col = tj * 32 + (lane & 31);
#pragma unroll
  for (int s = 0; s < 16; ++s) Kout[(ti * 32 + acc_row(s, h)) * kLb + col] = gv[s] * ga[s];
  __syncthreads();   // Vl is free from here on
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int t = ti * 32 + acc_row(s, h);
    Vl[t * kLd + col] = (col <= t) ? pk[s] : 0.f;
  }
  __syncthreads();
  if (tid < kLb) {
    float acc = 0.f;
    for (int s = 0; s < kLb; ++s) acc += Vl[tid * kLd + s];
    if (tid < tcount) pl.ld[row0 + tid] = acc;
  } else if (tid < 2 * kLb) {
    const int c = tid - kLb;
    float acc = 0.f;
    for (int t = 0; t < tcount; ++t) acc += Kl[t * kLd + c];
    pl.ksum[(chain * pl.nblk + b) * kD + c] = acc;
  }
}

// ---- chain: the sequential part, one workgroup per chain ---------------------
// One block's v, alpha_hat and K held in registers, so the next block's loads
// are in flight while the current block computes.
template <typename TIn>
struct BlockRegs {
  static constexpr int kVVec = kLb * kD / Elem<TIn>::kPer16B / kThreads;   // 16-byte vectors per thread
  static constexpr int kFVec = kLb * kD / 4 / kThreads;
  uint4 v[kVVec], a[kFVec], k[kFVec];
  float ks;   // threads 0..63: block sum of k, feature tid

  __device__ __forceinline__ void load(const StatePlan& pl, int64_t chain, int b, int tid) {
    const int tcount = min(kLb, pl.T - b * kLb);
    const int64_t row0 = chain * pl.T + b * kLb;
    constexpr int vpr = kD / Elem<TIn>::kPer16B;
    const TIn* vg = static_cast<const TIn*>(pl.v) + row0 * kD;
#pragma unroll
    for (int j = 0; j < kVVec; ++j) {
      const int e = tid + j * kThreads, row = e / vpr;
      v[j] = row < tcount ? *reinterpret_cast<const uint4*>(vg + row * kD + (e % vpr) * Elem<TIn>::kPer16B)
                          : make_uint4(0, 0, 0, 0);
    }
    const float* ag = pl.alpha + row0 * kD;
    const float* kg = pl.Kmat + (chain * pl.nblk + b) * kLb * kLb;
#pragma unroll
    for (int j = 0; j < kFVec; ++j) {
      const int e = tid + j * kThreads, row = e / 16;
      a[j] = row < tcount ? *reinterpret_cast<const uint4*>(ag + row * kD + (e % 16) * 4) : make_uint4(0, 0, 0, 0);
      k[j] = *reinterpret_cast<const uint4*>(kg + e * 4);
    }
    ks = tid < kD ? pl.ksum[(chain * pl.nblk + b) * kD + tid] : 0.f;
  }

  // Row-major copies of v, alpha_hat and K, plus transposed copies of v and
  // alpha_hat (feature-major) for the state update's matrix product.
  __device__ __forceinline__ void store(float* Vl, float* Al, float* Kl, float* Vt, float* At, int tid) const {
    constexpr int EPV = Elem<TIn>::kPer16B, vpr = kD / EPV;
#pragma unroll
    for (int j = 0; j < kVVec; ++j) {
      const int e = tid + j * kThreads, row = e / vpr, c = (e % vpr) * EPV;
      float f[EPV];
      if constexpr (EPV == 4) {
        f[0] = __uint_as_float(v[j].x); f[1] = __uint_as_float(v[j].y);
        f[2] = __uint_as_float(v[j].z); f[3] = __uint_as_float(v[j].w);
      } else {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[2 * q] = __uint_as_float(w[q] << 16);
          f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int q = 0; q < EPV; q += 4)
        *reinterpret_cast<float4*>(Vl + row * kLd + c + q) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
#pragma unroll
      for (int q = 0; q < EPV; ++q) Vt[(c + q) * kLd + row] = f[q];
    }
#pragma unroll
    for (int j = 0; j < kFVec; ++j) {
      const int e = tid + j * kThreads, row = e / 16, c = (e % 16) * 4;
      *reinterpret_cast<uint4*>(Al + row * kLd + c) = a[j];
      *reinterpret_cast<uint4*>(Kl + row * kLd + c) = k[j];
      At[(c + 0) * kLd + row] = __uint_as_float(a[j].x);
      At[(c + 1) * kLd + row] = __uint_as_float(a[j].y);
      At[(c + 2) * kLd + row] = __uint_as_float(a[j].z);
      At[(c + 3) * kLd + row] = __uint_as_float(a[j].w);
    }
  }
};

template <typename TIn>
__global__ void __launch_bounds__(kThreads)
vla_state_chain_kernel(StatePlan pl, const float* __restrict__ S0, const float* __restrict__ n0,
                       float* __restrict__ S_T, float* __restrict__ n_T, int32_t* __restrict__ stats,
                       const int32_t* __restrict__ chain_info, float cap, int cap_on) {
  extern __shared__ float4 smem4[];
  float* Xl = reinterpret_cast<float*>(smem4);     // [64][kLd] S at the block start
  float* Vl = Xl + kD * kLd;                        // [64][kLd] v of the block
  float* Al = Vl + kLb * kLd;                       // [64][kLd] alpha_hat of the block
  float* Kl = Al + kLb * kLd;                       // [64][kLd] kernel matrix of the block
  float* Vt = Kl + kLb * kLd;                       // [64][kLd] v, feature-major
  float* At = Vt + kD * kLd;                        // [64][kLd] alpha_hat, feature-major
  float* CKl = At + kD * kLd;                       // [64][kLd] row prefix sums of K (65 used)
  float* hpart = CKl + kLb * kLd;                   // [2][64]
  float* wbuf = hpart + 2 * kLb;                    // [64]
  float* sbuf = wbuf + kLb;                         // [64]
  float* red = sbuf + kLb;                          // [8]
  const int64_t chain = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int ti = w >> 1, tj = w & 1;                // this wave's tile of S
  const int col = tj * 32 + (lane & 31);
  const float cap2 = cap * cap;

  // S tile in accumulator layout.
  f32x16 X;
  const float* s0 = S0 + chain * kD * kD;
#pragma unroll
  for (int s = 0; s < 16; ++s) X[s] = s0[(ti * 32 + acc_row(s, h)) * kD + col];
  float nrm = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    nrm = fmaf(X[s], X[s], nrm);
    Xl[(ti * 32 + acc_row(s, h)) * kLd + col] = X[s];
  }
  nrm = wave_sum(nrm);
  if (lane == 0) red[w] = nrm;
  float nvec = (w == 0) ? n0[chain * kD + lane] : 0.f;   // wave 0, lane i: n_i
  int fires = 0, first = -1;
  bool bad = false;
  BlockRegs<TIn> regs;
  regs.load(pl, chain, 0, tid);
  regs.store(Vl, Al, Kl, Vt, At, tid);
  float ks_cur = regs.ks;   // k summed over the current block (threads 0..63)
  __syncthreads();
  float N = (red[0] + red[1]) + (red[2] + red[3]);   // |S|^2, identical on every wave

  for (int b = 0; b < pl.nblk; ++b) {
    const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
    const int64_t row0 = chain * pl.T + tb;
    if (b + 1 < pl.nblk) regs.load(pl, chain, b + 1, tid);   // in flight during this block
    float* Xs = pl.Xsnap + (chain * pl.nblk + b) * kD * kD;
#pragma unroll
    for (int s = 0; s < 16; ++s) Xs[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
    if (w == 0) pl.nblock[(chain * pl.nblk + b) * kD + lane] = nvec;

    // h_t = v_t^T S_b alpha_t: Y = S_b A^T (tile ti x tt, tt = tj), then
    // contract Y's rows with v_t.
    {
      f32x16 Y = zero16();
      mma_rr(Y, Xl + ti * 32 * kLd, Al + tj * 32 * kLd, lane);
      const int t = tj * 32 + (lane & 31);
      float p = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) p = fmaf(Vl[t * kLd + ti * 32 + acc_row(s, h)], Y[s], p);
      p += __shfl_xor(p, 32, 64);
      if (h == 0) hpart[ti * kLb + t] = p;
    }
    __syncthreads();

    // Cap recursion over the block's tokens (wave 0, lane t).  Invariant:
    // acc_t = v_t^T S alpha_t for the state S after the last cap fire, and
    // N = |S|^2.  Cap fires are rare, so each round assumes none for the rest
    // of the block: token t's pre-cap norm is N plus the prefix sum over
    // s0 <= s <= t of 2 g_s + e_s, with g_s = acc_s + sum_{s0<=r<s} K(s,r)
    // taken from row prefix sums of K.  The first token that exceeds the cap
    // ends the round; the accumulators of later tokens then move to the
    // post-fire state, and the next round starts after it.
    if (w == 0) {
      const int t = lane;
      float acc = hpart[t] + hpart[kLb + t];
      const float e_t = Kl[t * kLd + t];
      float own = 0.f;   // sum_{r<t} K(t,r)
      {
        float run = 0.f;
#pragma unroll
        for (int m = 0; m < kLb / 4; ++m) {
          const float4 kv = *reinterpret_cast<const float4*>(Kl + t * kLd + 4 * m);
          float4 o;
          o.x = run; own = (t == 4 * m) ? run : own; run += kv.x;
          o.y = run; own = (t == 4 * m + 1) ? run : own; run += kv.y;
          o.z = run; own = (t == 4 * m + 2) ? run : own; run += kv.z;
          o.w = run; own = (t == 4 * m + 3) ? run : own; run += kv.w;
          *reinterpret_cast<float4*>(CKl + t * kLd + 4 * m) = o;
        }
        CKl[t * kLd + kLb] = run;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float base = 0.f, lprev_t = 0.f, l_t = 0.f, L = 0.f;
      int s0 = 0;
      while (s0 < tcount) {
        const bool act = t >= s0 && t < tcount;
        const float g = acc + (own - base);
        const float npre = N + wave_incl_scan(act ? fmaf(2.f, g, e_t) : 0.f, t);
        const uint64_t over = __ballot(act && cap_on && npre > cap2);
        if (over == 0) {
          N = readlane_f(npre, tcount - 1);
          break;
        }
        const int f = __ffsll(static_cast<long long>(over)) - 1;
        const float nf = readlane_f(npre, f);
        const float c = cap * __builtin_amdgcn_rsqf(nf);
        const float lg = __builtin_amdgcn_logf(c);   // log2
        const float cf = CKl[t * kLd + f + 1];
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
      // GEMM weights sigma_end / sigma_{s-1}; the block's final scale in sbuf[0].
      wbuf[t] = (t < tcount) ? exp2f(L - lprev_t) : 0.f;
      if (t == 0) sbuf[0] = exp2f(L);
      if (t < tcount) {
        pl.wsig[2 * (row0 + t)] = lprev_t;
        pl.wsig[2 * (row0 + t) + 1] = l_t;
      }
      nvec += ks_cur;
    }
    __syncthreads();

    // S <- sigma_end S_b + V^T diag(sigma_end / sigma_{s-1}) A; N <- |S|^2 exactly.
    const float sig_end = sbuf[0];
#pragma unroll
    for (int s = 0; s < 16; ++s) X[s] *= sig_end;
    mma_rr_w(X, Vt + ti * 32 * kLd, At + tj * 32 * kLd, wbuf, lane);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) part = fmaf(X[s], X[s], part);
    part = wave_sum(part);
    if (lane == 0) red[4 + w] = part;
    __syncthreads();
    N = (red[4] + red[5]) + (red[6] + red[7]);
#pragma unroll
    for (int s = 0; s < 16; ++s) Xl[(ti * 32 + acc_row(s, h)) * kLd + col] = X[s];
    if (b + 1 < pl.nblk) {
      regs.store(Vl, Al, Kl, Vt, At, tid);
      ks_cur = regs.ks;
    }
    __syncthreads();
  }

  float* st = S_T + chain * kD * kD;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    st[(ti * 32 + acc_row(s, h)) * kD + col] = X[s];
    bad |= !isfinite(X[s]);
  }
  if (w == 0) {
    n_T[chain * kD + lane] = nvec;
    bad |= !isfinite(nvec);
  }
  const bool wave_bad = __any(bad);
  if (lane == 0) red[w] = wave_bad ? 1.f : 0.f;
  __syncthreads();
  if (tid == 0 && stats) {
    const bool any_bad = red[0] != 0.f || red[1] != 0.f || red[2] != 0.f || red[3] != 0.f ||
                         chain_info[chain * 4 + kInfoNonfinite] != 0;
    int32_t* s = stats + chain * 4;
    s[0] = chain_info[chain * 4 + kInfoGuard];
    s[1] = fires;
    s[2] = any_bad ? 1 : 0;
    s[3] = first;
  }
}

// ---- readout: o for every block in parallel --------------------------------
template <typename TIn>
__global__ void __launch_bounds__(kThreads)
vla_state_readout_kernel(StatePlan pl, const TIn* __restrict__ q, TIn* __restrict__ o, float den_eps,
                         int32_t* __restrict__ stats) {
  extern __shared__ float4 smem4[];
  float* Ql = reinterpret_cast<float*>(smem4);
  float* Xl = Ql + kLb * kLd;
  float* Al = Xl + kD * kLd;
  float* Vl = Al + kLb * kLd;
  float* Pl = Vl + kLb * kLd;
  float* wl = Pl + kLb * kLd;      // [64] log2 sigma_{s-1} (block-local)
  float* sl = wl + kLb;            // [64] log2 sigma_t
  float* dl = sl + kLb;            // [64] den_t
  float* nl = dl + kLb;            // [64] n at the block start
  const int64_t chain = blockIdx.x / pl.nblk;
  const int b = blockIdx.x % pl.nblk;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int tb = b * kLb, tcount = min(kLb, pl.T - tb);
  const int64_t row0 = chain * pl.T + tb;
  stage_block<TIn>(Ql, q + row0 * kD, tcount, tid);
  stage_block<float>(Xl, pl.Xsnap + (chain * pl.nblk + b) * kD * kD, kD, tid);
  stage_block<float>(Al, pl.alpha + row0 * kD, tcount, tid);
  if (pl.bf16)
    stage_block<uint16_t>(Vl, static_cast<const uint16_t*>(pl.v) + row0 * kD, tcount, tid);
  else
    stage_block<float>(Vl, static_cast<const float*>(pl.v) + row0 * kD, tcount, tid);
  if (tid < kLb) {
    const bool ok = tid < tcount;
    wl[tid] = ok ? pl.wsig[2 * (row0 + tid)] : 0.f;
    sl[tid] = ok ? pl.wsig[2 * (row0 + tid) + 1] : 0.f;
    nl[tid] = pl.nblock[(chain * pl.nblk + b) * kD + tid];
  }
  __syncthreads();
  if (tid < kLb) {
    float acc = 0.f;
    for (int i = 0; i < kD; ++i) acc = fmaf(Ql[tid * kLd + i], nl[i], acc);
    dl[tid] = acc + (tid < tcount ? pl.ld[row0 + tid] : 0.f) + den_eps;
  }

  const int tt = w >> 1, ti = w & 1;   // output tile: tokens tt, features ti
  f32x16 Z = zero16();
  mma_rr(Z, Ql + tt * 32 * kLd, Xl + ti * 32 * kLd, lane);   // (X_b q_t)_i
  if (ti == 0) {
    // P'[t][s] = (sigma_t / sigma_{s-1}) (alpha_s . q_t) for s <= t.
    const int scol = lane & 31;
    for (int ts = 0; ts < 2; ++ts) {
      f32x16 P = zero16();
      mma_rr(P, Ql + tt * 32 * kLd, Al + ts * 32 * kLd, lane);
      const int s = ts * 32 + scol;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int t = tt * 32 + acc_row(a, h);
        Pl[t * kLd + s] = (s <= t) ? P[a] * exp2f(sl[t] - wl[s]) : 0.f;
      }
    }
  }
  // sigma_t S_b q_t
#pragma unroll
  for (int a = 0; a < 16; ++a) Z[a] *= exp2f(sl[tt * 32 + acc_row(a, h)]);
  __syncthreads();
  mma_rc(Z, Pl + tt * 32 * kLd, Vl + ti * 32, lane);
  bool bad = false;
  const int fcol = ti * 32 + (lane & 31);
#pragma unroll
  for (int a = 0; a < 16; ++a) {
    const int t = tt * 32 + acc_row(a, h);
    if (t < tcount) {
      const float ov = Z[a] / dl[t];
      bad |= !isfinite(ov);
      Elem<TIn>::store(o + (row0 + t) * kD + fcol, ov);
    }
  }
  // The chain kernel has written this chain's statistics already.
  if (__any(bad) && lane == 0 && stats) atomicOr(stats + chain * 4 + 2, 1);
}

}  // namespace

size_t state_prep_lds_bytes() { return sizeof(float) * 4 * kLb * kLd; }
size_t state_chain_lds_bytes() { return sizeof(float) * (7 * kLb * kLd + 4 * kLb + 8); }
size_t state_readout_lds_bytes() { return sizeof(float) * (5 * kLb * kLd + 4 * kLb); }

template <typename K>
static void allow_lds(K kernel, size_t bytes) {
  // Raise the dynamic LDS limit of a kernel above the 64 KiB default once.
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes));
}

hipError_t launch_state_pass(const StatePlan& pl, const ScanArgs& a, int32_t* chain_info, int chains,
                             hipStream_t stream) {
  static const bool once = [] {
    allow_lds(vla_state_prep_kernel<uint16_t>, state_prep_lds_bytes());
    allow_lds(vla_state_prep_kernel<float>, state_prep_lds_bytes());
    allow_lds(vla_state_chain_kernel<uint16_t>, state_chain_lds_bytes());
    allow_lds(vla_state_chain_kernel<float>, state_chain_lds_bytes());
    allow_lds(vla_state_readout_kernel<uint16_t>, state_readout_lds_bytes());
    allow_lds(vla_state_readout_kernel<float>, state_readout_lds_bytes());
    return true;
  }();
  (void)once;
  const unsigned blocks = static_cast<unsigned>(chains * pl.nblk);
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_prep_kernel<uint16_t>, dim3(blocks), dim3(kThreads), state_prep_lds_bytes(), stream,
                       pl, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v));
  else
    hipLaunchKernelGGL(vla_state_prep_kernel<float>, dim3(blocks), dim3(kThreads), state_prep_lds_bytes(), stream,
                       pl, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                       static_cast<const float*>(a.v));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_chain_kernel<uint16_t>, dim3(chains), dim3(kThreads), state_chain_lds_bytes(), stream,
                       pl, a.S0, a.n0, a.S_T, a.n_T, a.stats, chain_info, a.cap, a.cap_on);
  else
    hipLaunchKernelGGL(vla_state_chain_kernel<float>, dim3(chains), dim3(kThreads), state_chain_lds_bytes(), stream,
                       pl, a.S0, a.n0, a.S_T, a.n_T, a.stats, chain_info, a.cap, a.cap_on);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (pl.bf16)
    hipLaunchKernelGGL(vla_state_readout_kernel<uint16_t>, dim3(blocks), dim3(kThreads), state_readout_lds_bytes(),
                       stream, pl, static_cast<const uint16_t*>(a.q), static_cast<uint16_t*>(a.o), a.den_eps,
                       a.stats);
  else
    hipLaunchKernelGGL(vla_state_readout_kernel<float>, dim3(blocks), dim3(kThreads), state_readout_lds_bytes(),
                       stream, pl, static_cast<const float*>(a.q), static_cast<float*>(a.o), a.den_eps, a.stats);
  return hipGetLastError();
}

}  // namespace vla
