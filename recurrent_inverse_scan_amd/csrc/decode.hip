// One-token scan step for d = 64: the decode case, where each call advances
// many chains by a single token and the state makes a round trip through HBM.
//
// Method as in the sequential kernel ("Mathematical Primitives", sections
// 2-5; "Variational Linear Attention (VLA)" README, v3 notes; for the
// residual update "Variational Linear Attention: Stable Associative Memory
// for Long-Context Transformers", technical summary 2.3): r guarded
// Sherman-Morrison updates of A, the nudge, the coefficient and its
// normalisation, the state update, the Frobenius cap and the readout.
//
// Layout: one workgroup of 256 threads per chain; thread tid owns row
// rr = tid / 4 of A and S and the 16 columns j = (4 m + cg) * 4 + e
// (m = 0..3, e = 0..3, cg = tid % 4: float4 blocks interleaved so the
// column reads of LDS vectors are conflict-free).  Row sums over a row's four
// threads use DPP; chain-wide scalars are wave sums combined through LDS.
// Every thread issues its state loads at once, and the lean register
// footprint keeps several chains per SIMD in flight, which overlaps one
// chain's loads with another's arithmetic.
#include "vla_common.h"
#include "vla_kernels.h"

namespace vla {
namespace {

constexpr int kD = 64;

template <typename TIn>
__device__ __forceinline__ float4 load4(const TIn* p) {
  if constexpr (sizeof(TIn) == 4) {
    return *reinterpret_cast<const float4*>(p);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
}

// Chain-wide sum of one value per thread (wave sums, then the four waves'
// partials through LDS); every thread receives the total.  Consecutive calls
// must alternate `slot`: a call's writes then come after the barrier of the
// call before, which every thread passes only once it has read the slot of
// the call before that.
__device__ __forceinline__ float block_sum(float x, float (*red)[4], int slot, int w, int lane) {
  x = wave_sum(x);
  if (lane == 0) red[slot][w] = x;
  __syncthreads();
  return (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
}

template <typename TIn, bool RES>
__global__ void __launch_bounds__(256) vla_decode_kernel(ScanArgs a) {
  __shared__ float4 sVec[8][kD / 4];   // u_1..u_r (0..3), k (4), q (5), v (6), scratch vector (7)
  __shared__ float red[2][4];
  const int64_t chain = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rr = tid >> 2, cg = tid & 3;
  const int r = a.r;
  float* vec = reinterpret_cast<float*>(sVec);

  // The token's vectors into LDS (threads 0..15 per vector, 4 values each).
  {
    const int which = tid >> 4, part = tid & 15;
    if (which < 8) {
      const TIn* src = nullptr;
      if (which < r) src = static_cast<const TIn*>(a.u) + (chain * r + which) * kD;
      else if (which == 4) src = static_cast<const TIn*>(a.k) + chain * kD;
      else if (which == 5) src = static_cast<const TIn*>(a.q) + chain * kD;
      else if (which == 6) src = static_cast<const TIn*>(a.v) + chain * kD;
      if (src) sVec[which][part] = load4(src + 4 * part);
    }
  }
  // This thread's row of A and S.
  float A[16], S[16];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int col = (4 * m + cg) * 4;
    float4 av = make_float4(rr == col ? 1.f : 0.f, rr == col + 1 ? 1.f : 0.f, rr == col + 2 ? 1.f : 0.f,
                            rr == col + 3 ? 1.f : 0.f);
    if (a.A0) av = *reinterpret_cast<const float4*>(a.A0 + (chain * kD + rr) * kD + col);
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.S0) sv = *reinterpret_cast<const float4*>(a.S0 + (chain * kD + rr) * kD + col);
    A[4 * m] = av.x; A[4 * m + 1] = av.y; A[4 * m + 2] = av.z; A[4 * m + 3] = av.w;
    S[4 * m] = sv.x; S[4 * m + 1] = sv.y; S[4 * m + 2] = sv.z; S[4 * m + 3] = sv.w;
  }
  float n = a.n0 ? a.n0[chain * kD + rr] : 0.f;
  __syncthreads();

  auto cols = [&](int which, float (&out)[16]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 x = sVec[which][4 * m + cg];
      out[4 * m] = x.x; out[4 * m + 1] = x.y; out[4 * m + 2] = x.z; out[4 * m + 3] = x.w;
    }
  };
  auto add_diag = [&](float s) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (rr == (4 * m + cg) * 4 + e) A[4 * m + e] += s;
  };

  // r guarded Sherman-Morrison updates.
  int guard = 0;
  int bs = 0;   // reductions so far: slot bs & 1 alternates
  for (int i = 0; i < r; ++i) {
    float uJ[16];
    cols(i, uJ);
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) z = fmaf(A[c], uJ[c], z);
    z = group_sum<4>(z);                     // (A u)_rr on all four threads of the row
    const float uI = vec[i * kD + rr];
    const float delta = 1.f + block_sum(cg == 0 ? uI * z : 0.f, red, (bs++) & 1, w, lane);
    if (fabsf(delta) < a.eps) {
      ++guard;
      add_diag(a.eps);
    } else {
      if (cg == 0) vec[7 * kD + rr] = z;
      __syncthreads();
      float zJ[16];
      cols(7, zJ);
      const float zs = z / delta;
#pragma unroll
      for (int c = 0; c < 16; ++c) A[c] = fmaf(-zs, zJ[c], A[c]);
      __syncthreads();                       // zJ read before the next z is written
    }
  }
  if (a.nudge_period > 0 && a.nudge_phase0 == 0) add_diag(a.eps);

  // alpha = A k and its normalisation; the residual prediction S k.
  float kJ[16];
  cols(4, kJ);
  float y = 0.f, pred = 0.f, kn = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    y = fmaf(A[c], kJ[c], y);
    if constexpr (RES) {
      pred = fmaf(S[c], kJ[c], pred);
      kn = fmaf(kJ[c], kJ[c], kn);
    }
  }
  y = group_sum<4>(y);
  if constexpr (RES) {
    pred = group_sum<4>(pred);
    kn = group_sum<4>(kn);                   // |k|^2: a row's four threads cover every column
  }
  const float an = block_sum(cg == 0 ? y * y : 0.f, red, (bs++) & 1, w, lane);
  float ascale;
  if constexpr (RES) {
    const float kinv = 1.f / fmaxf(sqrtf(kn), 1e-12f);
    ascale = kinv / fmaxf(kinv * sqrtf(an), 1e-12f);
    pred *= kinv;
  } else {
    ascale = an > 1.f ? 1.f / sqrtf(an) : 1.f;
  }
  if (cg == 0) vec[7 * kD + rr] = y * ascale;
  __syncthreads();
  float aJ[16], qJ[16];
  cols(7, aJ);
  cols(5, qJ);
  const float vI = vec[6 * kD + rr];
  const float wI = RES ? vI - pred : vI;   // what the row writes along alpha_hat

  // State update, its norm, the cap and the readout.
  float ns = 0.f, po = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    S[c] = fmaf(wI, aJ[c], S[c]);
    ns = fmaf(S[c], S[c], ns);
    po = fmaf(S[c], qJ[c], po);
  }
  po = group_sum<4>(po);
  const float kI = vec[4 * kD + rr], qI = vec[5 * kD + rr];
  n += kI;
  const float ns_all = block_sum(ns, red, (bs++) & 1, w, lane);
  const float nq = block_sum(cg == 0 ? n * qI : 0.f, red, (bs++) & 1, w, lane);
  float oscale = 1.f;
  int capf = 0;
  if (a.cap_on && ns_all > a.cap * a.cap) {
    oscale = a.cap / sqrtf(ns_all);
#pragma unroll
    for (int c = 0; c < 16; ++c) S[c] *= oscale;
    capf = 1;
  }
  const float ov = po * oscale / (nq + a.den_eps);
  bool bad = false;
  if (cg == 0) {
    Elem<TIn>::store(static_cast<TIn*>(a.o) + chain * kD + rr, ov);
    a.n_T[chain * kD + rr] = n;
    bad |= !isfinite(ov) || !isfinite(n);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int col = (4 * m + cg) * 4;
    const float4 av = make_float4(A[4 * m], A[4 * m + 1], A[4 * m + 2], A[4 * m + 3]);
    const float4 sv = make_float4(S[4 * m], S[4 * m + 1], S[4 * m + 2], S[4 * m + 3]);
    *reinterpret_cast<float4*>(a.A_T + (chain * kD + rr) * kD + col) = av;
    *reinterpret_cast<float4*>(a.S_T + (chain * kD + rr) * kD + col) = sv;
#pragma unroll
    for (int e = 0; e < 4; ++e) bad |= !isfinite(A[4 * m + e]) || !isfinite(S[4 * m + e]);
  }
  if (a.stats) {
    const float nbad = block_sum(bad ? 1.f : 0.f, red, (bs++) & 1, w, lane);
    if (tid == 0) {
      int32_t* st = a.stats + chain * 4;
      st[0] = guard;
      st[1] = capf;
      st[2] = nbad > 0.f ? 1 : 0;
      st[3] = capf ? 0 : -1;
    }
  }
}

}  // namespace

hipError_t launch_decode(const ScanArgs& a, bool bf16, int chains, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(chains));
  if (bf16) {
    if (a.residual)
      hipLaunchKernelGGL((vla_decode_kernel<uint16_t, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vla_decode_kernel<uint16_t, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (a.residual)
      hipLaunchKernelGGL((vla_decode_kernel<float, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((vla_decode_kernel<float, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace vla
