// Backward pass of the VLA scan (additive update, sequential per chain).
//
// The pages ask for "full gradient flow" through the recurrence ("Variational
// Linear Attention (VLA)" README, VLA v3 research implementation notes item
// 2) and state only the forward steps ("Mathematical Primitives" sections 2-5;
// README v3 notes item 5).  The gradient here is the exact derivative of that
// recurrence for L = sum_t <g_o[t], o_t> + <g_A, A_T> + <g_S, S_T> + <g_n, n_T>,
// taken token by token in reverse.  Per token (forward order):
//   for i = 1..r:  z = A u_i, delta = 1 + u_i.z; fire: A += eps I; else A -= z z^T/delta
//   nudge:         A += eps I
//   alpha = A k;   alpha_hat = alpha / max(|alpha|, 1)
//   X = S + v alpha_hat^T;  S = c X with c = min(1, cap/|X|)
//   n += k;        o = S q / (n.q + den_eps)
// Reverse, with gS, gA, gn the adjoints of the state after the token:
//   readout:  gS += g_o q^T/den;  g_q = S^T g_o/den - (g_o.o/den) n;  gn -= (g_o.o/den) q
//   normaliser: g_k = gn (n_{t-1} = n_t - k_t)
//   cap (fired): gX = c (gS - <gS, S> S/|S|^2)   (S/|S| is X/|X|)
//   state:    g_v = gX alpha_hat;  g_alpha_hat = gX^T v;  gS_{t-1} = gX
//   clamp:    |alpha| > 1: g_alpha = (g_ah - (ah.g_ah) ah)/|alpha|, else g_ah
//   alpha:    gA += g_alpha k^T;  g_k += A^T g_alpha
//   rank-1 i (reverse order, not fired), G = gA after it:
//             gdelta = z^T G z / delta^2;  gz = -(G + G^T) z/delta + gdelta u_i
//             gA = G + gz u_i^T;  g_u_i = A_before^T gz + gdelta z
// A_before = A_after + z z^T/delta is rebuilt from the recorded z and delta
// (no division that could amplify rounding); S is recomputed forward inside
// chunks of kChk tokens from checkpoints, since undoing the cap would divide
// by c.
//
// Kernels (one workgroup of 256 threads per chain, matrices in LDS):
//   vla_bwd_tape_kernel     the forward recurrence, recording per token the
//                           z and delta of every rank-1 step, the guard
//                           fires, alpha_hat, |alpha| and c, plus A, S, n at
//                           every chunk start and at the end;
//   vla_bwd_reverse_kernel  the reverse recurrence above, chunk by chunk.
#include "vla_common.h"
#include "vla_kernels.h"

namespace vla {

namespace {

constexpr int kThr = 256;
constexpr int kChk = 32;   // tokens per checkpoint chunk

// Thread layout for a D x D matrix in LDS (row stride D + 4): thread tid owns
// row tid / P, columns [W (tid % P), W (tid % P + 1)), P = 256 / D threads per
// row and W = D / P columns each.  A column operation reads the same thread
// as (column tid / P, rows [W (tid % P), ...)).
template <int D>
struct Lay {
  static constexpr int P = kThr / D;
  static constexpr int W = D / P;
  static constexpr int S = D + 4;
  static_assert(P * D == kThr && W * P == D, "layout");
};

// Sum over the P consecutive lanes that share a row (P a power of two <= 16).
template <int P>
__device__ __forceinline__ float part_sum(float x) {
#pragma unroll
  for (int m = 1; m < P; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// (M x)[row] for this thread's row: the full sum on every lane of the row.
template <int D>
__device__ __forceinline__ float row_op(const float* M, const float* x, int tid) {
  using L = Lay<D>;
  const int i = tid / L::P, c0 = (tid % L::P) * L::W;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < L::W; ++j) acc = fmaf(M[i * L::S + c0 + j], x[c0 + j], acc);
  return part_sum<L::P>(acc);
}

// (M^T x)[col] for the column tid / P: the full sum on every lane of the group.
template <int D>
__device__ __forceinline__ float col_op(const float* M, const float* x, int tid) {
  using L = Lay<D>;
  const int j = tid / L::P, r0 = (tid % L::P) * L::W;
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < L::W; ++r) acc = fmaf(M[(r0 + r) * L::S + j], x[r0 + r], acc);
  return part_sum<L::P>(acc);
}

// Block-wide sum of one value per thread; `red` holds 4 floats.  Ends with
// the total on every thread (two barriers).
__device__ __forceinline__ float block_sum(float x, float* red, int tid) {
  x = part_sum<64>(x);   // xor over the whole wave
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

template <int D>
__device__ __forceinline__ float dot_lds(const float* a, const float* b) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < D; ++j) acc = fmaf(a[j], b[j], acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elem<T>::load(p + i);
}

}  // namespace

// ---- forward with a tape ---------------------------------------------------
template <typename TIn, int D>
__global__ void __launch_bounds__(kThr) vla_bwd_tape_kernel(BwdArgs a) {
  using L = Lay<D>;
  __shared__ float sA[D * L::S], sS[D * L::S];
  __shared__ float vu[4][D], vk[D], vv[D], vz[D], vah[D];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int T = a.T, r = a.r;
  const int64_t nck = (T + kChk - 1) / kChk;
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const TIn* u = static_cast<const TIn*>(a.u);
  (void)q;
  const int i = tid / L::P, c0 = (tid % L::P) * L::W;
  // initial state
#pragma unroll
  for (int j = 0; j < L::W; ++j) {
    const int col = c0 + j;
    sA[i * L::S + col] = a.A0 ? a.A0[(c * D + i) * D + col] : (i == col ? 1.f : 0.f);
    sS[i * L::S + col] = a.S0 ? a.S0[(c * D + i) * D + col] : 0.f;
  }
  float n_own = 0.f;   // n[tid] for tid < D
  if (tid < D) n_own = a.n0 ? a.n0[c * D + tid] : 0.f;
  float* ckA = a.ckA + c * (nck + 1) * D * D;
  float* ckS = a.ckS + c * (nck + 1) * D * D;
  float* ckn = a.ckn + c * (nck + 1) * D;
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int64_t row = c * T + t;
    if (t % kChk == 0) {   // checkpoint at the chunk start (state before token t)
      const int64_t ck = t / kChk;
#pragma unroll
      for (int j = 0; j < L::W; ++j) {
        ckA[(ck * D + i) * D + c0 + j] = sA[i * L::S + c0 + j];
        ckS[(ck * D + i) * D + c0 + j] = sS[i * L::S + c0 + j];
      }
      if (tid < D) ckn[ck * D + tid] = n_own;
    }
    for (int e = tid; e < r * D; e += kThr) vu[e / D][e % D] = ld(u, row * r * D + e);
    if (tid < D) {
      vk[tid] = ld(k, row * D + tid);
      vv[tid] = ld(v, row * D + tid);
    }
    __syncthreads();
    for (int s = 0; s < r; ++s) {
      const float zi = row_op<D>(sA, vu[s], tid);   // z[i] on every lane of row i
      if (tid % L::P == 0) vz[i] = zi;
      __syncthreads();
      const float delta = 1.f + dot_lds<D>(vu[s], vz);
      const bool fire = fabsf(delta) < a.eps;
      if (tid < D) a.tz[(row * r + s) * D + tid] = vz[tid];
      if (tid == 0) {
        a.tdelta[row * r + s] = delta;
        a.tfire[row * r + s] = fire ? 1.f : 0.f;
      }
      const float inv = fire ? 0.f : 1.f / delta;
#pragma unroll
      for (int j = 0; j < L::W; ++j) {
        const int col = c0 + j;
        float x = sA[i * L::S + col];
        x = fire ? (x + (i == col ? a.eps : 0.f)) : fmaf(-zi * inv, vz[col], x);
        sA[i * L::S + col] = x;
      }
      __syncthreads();
    }
    if (a.nudge_period > 0 && (a.nudge_phase0 + t) % a.nudge_period == 0) {
#pragma unroll
      for (int j = 0; j < L::W; ++j)
        if (i == c0 + j) sA[i * L::S + c0 + j] += a.eps;
      __syncthreads();
    }
    const float al = row_op<D>(sA, vk, tid);   // alpha[i]
    if (tid % L::P == 0) vz[i] = al;
    __syncthreads();
    const float an = sqrtf(dot_lds<D>(vz, vz));
    const float m = fmaxf(an, 1.f);
    if (tid < D) {
      vah[tid] = vz[tid] / m;
      a.tah[row * D + tid] = vz[tid] / m;
    }
    if (tid == 0) a.tan_[row] = an;
    __syncthreads();
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < L::W; ++j) {
      const int col = c0 + j;
      const float x = fmaf(vv[i], vah[col], sS[i * L::S + col]);
      sS[i * L::S + col] = x;
      part = fmaf(x, x, part);
    }
    float cscale = 1.f;
    if (a.cap_on) {
      const float fn = sqrtf(block_sum(part, red, tid));
      if (fn > a.cap) {
        cscale = a.cap / fn;
#pragma unroll
        for (int j = 0; j < L::W; ++j) sS[i * L::S + c0 + j] *= cscale;
      }
    }
    if (tid == 0) a.tc[row] = cscale;
    if (tid < D) n_own += vk[tid];
    __syncthreads();
  }
  // final state (checkpoint nck) and A_T, S_T, n_T
#pragma unroll
  for (int j = 0; j < L::W; ++j) {
    ckA[(nck * D + i) * D + c0 + j] = sA[i * L::S + c0 + j];
    ckS[(nck * D + i) * D + c0 + j] = sS[i * L::S + c0 + j];
  }
  if (tid < D) ckn[nck * D + tid] = n_own;
}

// ---- reverse ---------------------------------------------------------------
template <typename TIn, int D>
__global__ void __launch_bounds__(kThr) vla_bwd_reverse_kernel(BwdArgs a) {
  using L = Lay<D>;
  __shared__ float sA[D * L::S], sS[D * L::S], gA[D * L::S], gS[D * L::S];
  __shared__ float vq[D], vk[D], vv[D], vgo[D], vah[D], vn[D], vy[D], vw1[D], vw2[D], vga[D];
  __shared__ float vu[4][D], vz[4][D];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int T = a.T, r = a.r;
  const int64_t nck = (T + kChk - 1) / kChk;
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
  const TIn* v = static_cast<const TIn*>(a.v);
  const TIn* u = static_cast<const TIn*>(a.u);
  const int i = tid / L::P, c0 = (tid % L::P) * L::W;
  const float* ckA = a.ckA + c * (nck + 1) * D * D;
  const float* ckS = a.ckS + c * (nck + 1) * D * D;
  const float* ckn = a.ckn + c * (nck + 1) * D;
  float* sbuf = a.sbuf + c * kChk * D * D;
  // adjoints of the final state
#pragma unroll
  for (int j = 0; j < L::W; ++j) {
    const int col = c0 + j;
    gA[i * L::S + col] = a.gAT ? a.gAT[(c * D + i) * D + col] : 0.f;
    gS[i * L::S + col] = a.gST ? a.gST[(c * D + i) * D + col] : 0.f;
  }
  float gn_own = 0.f;   // gn[tid] for tid < D
  if (tid < D) gn_own = a.gnT ? a.gnT[c * D + tid] : 0.f;

  for (int64_t ck = nck - 1; ck >= 0; --ck) {
    const int t_lo = ck * kChk, t_hi = min(T, t_lo + kChk);
    // S_t for the chunk's tokens, recomputed from the chunk-start checkpoint
    // with the recorded alpha_hat and cap scale (the forward's arithmetic).
    {
      float s_own[L::W];
#pragma unroll
      for (int j = 0; j < L::W; ++j) s_own[j] = ckS[(ck * D + i) * D + c0 + j];
      for (int t = t_lo; t < t_hi; ++t) {
        const int64_t row = c * T + t;
        const float vi = ld(v, row * D + i), cs = a.tc[row];
#pragma unroll
        for (int j = 0; j < L::W; ++j) {
          const float x = fmaf(vi, a.tah[row * D + c0 + j], s_own[j]);
          s_own[j] = cs < 1.f ? x * cs : x;
          sbuf[((t - t_lo) * D + i) * D + c0 + j] = s_own[j];
        }
      }
    }
    // A and n after the chunk's last token
#pragma unroll
    for (int j = 0; j < L::W; ++j) sA[i * L::S + c0 + j] = ckA[((ck + 1) * D + i) * D + c0 + j];
    if (tid < D) vn[tid] = ckn[(ck + 1) * D + tid];
    __syncthreads();   // sbuf writes visible to the workgroup, sA ready

    for (int t = t_hi - 1; t >= t_lo; --t) {
      const int64_t row = c * T + t;
      // token vectors and S_t
      if (tid < D) {
        vq[tid] = ld(q, row * D + tid);
        vk[tid] = ld(k, row * D + tid);
        vv[tid] = ld(v, row * D + tid);
        vgo[tid] = a.go[row * D + tid];
        vah[tid] = a.tah[row * D + tid];
      }
      for (int e = tid; e < r * D; e += kThr) {
        vu[e / D][e % D] = ld(u, row * r * D + e);
        vz[e / D][e % D] = a.tz[row * r * D + e];
      }
#pragma unroll
      for (int j = 0; j < L::W; ++j) sS[i * L::S + c0 + j] = sbuf[((t - t_lo) * D + i) * D + c0 + j];
      __syncthreads();
      // readout: y = S q, den = n.q + den_eps
      const float yi = row_op<D>(sS, vq, tid);
      if (tid % L::P == 0) vy[i] = yi;
      __syncthreads();
      const float den = dot_lds<D>(vn, vq) + a.den_eps;
      const float sdot = dot_lds<D>(vgo, vy) / den;   // g_o . o
      // g_q = S^T g_o / den - (g_o.o / den) n
      const float sg = col_op<D>(sS, vgo, tid);
      const int jc = tid / L::P;   // this thread's column in column operations
      float gq_col = sg / den - (sdot / den) * vn[jc];
      // gS += g_o q^T / den, then the cap's projection needs <gS, S> and |S|^2
      float pgs = 0.f, pss = 0.f;
#pragma unroll
      for (int j = 0; j < L::W; ++j) {
        const int col = c0 + j;
        const float g = fmaf(vgo[i] / den, vq[col], gS[i * L::S + col]);
        gS[i * L::S + col] = g;
        const float s = sS[i * L::S + col];
        pgs = fmaf(g, s, pgs);
        pss = fmaf(s, s, pss);
      }
      const float cs = a.tc[row];
      if (cs < 1.f) {
        const float gss = block_sum(pgs, red, tid);
        const float ss = block_sum(pss, red, tid);
        const float f = gss / ss;
#pragma unroll
        for (int j = 0; j < L::W; ++j) {
          const int col = c0 + j;
          gS[i * L::S + col] = cs * fmaf(-f, sS[i * L::S + col], gS[i * L::S + col]);
        }
      }
      // normaliser: gn -= (g_o.o/den) q; g_k = gn
      float gk_col = 0.f;
      if (tid < D) {
        gn_own = fmaf(-sdot / den, vq[tid], gn_own);
        vw1[tid] = gn_own;   // staged for the column-owner threads
      }
      __syncthreads();
      gk_col = vw1[jc];
      // state update: g_v = gX alpha_hat, g_alpha_hat = gX^T v
      const float gvi = row_op<D>(gS, vah, tid);
      const float gah = col_op<D>(gS, vv, tid);
      if (tid % L::P == 0) vga[jc] = gah;
      __syncthreads();
      // clamp
      const float an = a.tan_[row];
      const float adot = dot_lds<D>(vah, vga);
      // alpha = A k: gA += g_alpha k^T, g_k += A^T g_alpha
      if (tid < D) vw2[tid] = an > 1.f ? (vga[tid] - adot * vah[tid]) / an : vga[tid];
      __syncthreads();
      gk_col += col_op<D>(sA, vw2, tid);
#pragma unroll
      for (int j = 0; j < L::W; ++j) {
        const int col = c0 + j;
        gA[i * L::S + col] = fmaf(vw2[i], vk[col], gA[i * L::S + col]);
      }
      // outputs of the readout and state steps
      if (tid % L::P == 0) {
        a.gq[row * D + jc] = gq_col;
        a.gv[row * D + i] = gvi;
      }
      __syncthreads();   // every read of A_t above is done
      // n and A before the token's nudge
      if (tid < D) vn[tid] -= vk[tid];
      if (a.nudge_period > 0 && (a.nudge_phase0 + t) % a.nudge_period == 0) {
#pragma unroll
        for (int j = 0; j < L::W; ++j)
          if (i == c0 + j) sA[i * L::S + c0 + j] -= a.eps;
      }
      // rank-1 steps in reverse
      for (int s = r - 1; s >= 0; --s) {
        const float* z = vz[s];
        const float* uu = vu[s];
        const float delta = a.tdelta[row * r + s];
        const bool fire = a.tfire[row * r + s] != 0.f;
        if (fire) {
#pragma unroll
          for (int j = 0; j < L::W; ++j)
            if (i == c0 + j) sA[i * L::S + c0 + j] -= a.eps;
          if (tid % L::P == 0) a.gu[(row * r + s) * D + jc] = 0.f;
          __syncthreads();
          continue;
        }
        const float w1 = row_op<D>(gA, z, tid);   // (G z)[i]
        const float w2 = col_op<D>(gA, z, tid);   // (G^T z)[jc]
        if (tid % L::P == 0) {
          vw1[i] = w1;
          vw2[jc] = w2;
        }
        __syncthreads();
        const float inv = 1.f / delta;
        const float gdelta = dot_lds<D>(z, vw1) * inv * inv;
        // A_before = A + z z^T/delta; gA += gz u^T, gz = -(w1 + w2)/delta + gdelta u
#pragma unroll
        for (int j = 0; j < L::W; ++j) {
          const int col = c0 + j;
          sA[i * L::S + col] = fmaf(z[i] * inv, z[col], sA[i * L::S + col]);
          const float gzi = fmaf(gdelta, uu[i], -(vw1[i] + vw2[i]) * inv);
          gA[i * L::S + col] = fmaf(gzi, uu[col], gA[i * L::S + col]);
        }
        if (tid < D) vy[tid] = fmaf(gdelta, uu[tid], -(vw1[tid] + vw2[tid]) * inv);   // gz
        __syncthreads();
        const float gu = col_op<D>(sA, vy, tid) + gdelta * z[jc];
        if (tid % L::P == 0) a.gu[(row * r + s) * D + jc] = gu;
        __syncthreads();
      }
      if (tid % L::P == 0) a.gk[row * D + jc] = gk_col;
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < L::W; ++j) {
    const int col = c0 + j;
    a.gA0[(c * D + i) * D + col] = gA[i * L::S + col];
    a.gS0[(c * D + i) * D + col] = gS[i * L::S + col];
  }
  if (tid < D) a.gn0[c * D + tid] = gn_own;
}

size_t bwd_workspace_bytes(int64_t chains, int T, int d, int r) {
  const int64_t nck = (T + kChk - 1) / kChk;
  const int64_t tok = chains * static_cast<int64_t>(T);
  auto al = [](int64_t b) { return static_cast<size_t>((b + 255) / 256 * 256); };
  return al(chains * (nck + 1) * d * d * 4) * 2 + al(chains * (nck + 1) * d * 4) + al(chains * kChk * d * d * 4) +
         al(tok * r * d * 4) + al(tok * r * 4) * 2 + al(tok * d * 4) + al(tok * 4) * 2;
}

void bwd_carve(BwdArgs& a, void* ws, int64_t chains, int T, int d, int r) {
  const int64_t nck = (T + kChk - 1) / kChk;
  const int64_t tok = chains * static_cast<int64_t>(T);
  auto al = [](int64_t b) { return static_cast<size_t>((b + 255) / 256 * 256); };
  char* p = static_cast<char*>(ws);
  a.ckA = reinterpret_cast<float*>(p); p += al(chains * (nck + 1) * d * d * 4);
  a.ckS = reinterpret_cast<float*>(p); p += al(chains * (nck + 1) * d * d * 4);
  a.ckn = reinterpret_cast<float*>(p); p += al(chains * (nck + 1) * d * 4);
  a.sbuf = reinterpret_cast<float*>(p); p += al(chains * kChk * d * d * 4);
  a.tz = reinterpret_cast<float*>(p); p += al(tok * r * d * 4);
  a.tdelta = reinterpret_cast<float*>(p); p += al(tok * r * 4);
  a.tfire = reinterpret_cast<float*>(p); p += al(tok * r * 4);
  a.tah = reinterpret_cast<float*>(p); p += al(tok * d * 4);
  a.tan_ = reinterpret_cast<float*>(p); p += al(tok * 4);
  a.tc = reinterpret_cast<float*>(p);
}

hipError_t launch_backward(const BwdArgs& a, int d, bool bf16, int chains, hipStream_t stream) {
  if (chains <= 0) return hipSuccess;
#define VLA_BWD_LAUNCH(TIN, DD)                                                                             \
  do {                                                                                                      \
    hipLaunchKernelGGL((vla_bwd_tape_kernel<TIN, DD>), dim3(chains), dim3(kThr), 0, stream, a);            \
    hipError_t e_ = hipGetLastError();                                                                      \
    if (e_ != hipSuccess) return e_;                                                                        \
    hipLaunchKernelGGL((vla_bwd_reverse_kernel<TIN, DD>), dim3(chains), dim3(kThr), 0, stream, a);         \
    return hipGetLastError();                                                                               \
  } while (0)
  if (bf16) {
    if (d == 16) VLA_BWD_LAUNCH(uint16_t, 16);
    if (d == 32) VLA_BWD_LAUNCH(uint16_t, 32);
    if (d == 64) VLA_BWD_LAUNCH(uint16_t, 64);
  } else {
    if (d == 16) VLA_BWD_LAUNCH(float, 16);
    if (d == 32) VLA_BWD_LAUNCH(float, 32);
    if (d == 64) VLA_BWD_LAUNCH(float, 64);
  }
#undef VLA_BWD_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace vla
