// Inverse pass of the time-parallel schedule in blocked form (d = 64, one
// direction per token, bf16 storage), on the gfx950 matrix cores.
//
// Method ("Mathematical Primitives", section 2: rank-1 Sherman-Morrison
// tracking of A = M^{-1}; section 4: alpha_t = A_t k_t; "Variational Linear
// Attention (VLA)" README, v3 notes: alpha_hat = alpha / max(|alpha|, 1)).
// Inside a chunk no nudge falls before its last token, so for a block of m
// tokens starting from A_b the m rank-1 updates compose exactly (Woodbury):
// with C = U^T A_b U and I + C = L D L^T (unit lower L, D diagonal),
//   delta_j = D_jj                     (the Sherman-Morrison denominators),
//   A after token t = A_b - Z_{<=t} D^{-1} Z_{<=t}^T,   Z = A_b U L^{-T},
//   alpha_t = A_b k_t - X_U G[:, t],   G = L^{-T} D^{-1} ((L^{-1} U^T A_b K) o M),
// M_jt = [j <= t], X_U = A_b U, and the block's end state
//   A_{b+1} = A_b - X_U W X_U^T,        W = L^{-T} D^{-1} L^{-1} = (I + C)^{-1}.
// The guard of section 2 (|delta| < eps) is checked on the pivots D_jj; a
// chain where it would fire is flagged for the sequential fallback, which
// reproduces the guarded recurrence exactly.
//
// One wave per chunk, blocks of 32 tokens.  A_b lives in four 32x32
// accumulator tiles for the whole chunk.  The state is kept in a permuted
// feature basis (bits 2 and 3 of the feature index swapped): then every MFMA
// operand a lane gathers from a token row is 8 consecutive features, one
// 16-byte load, while accumulator tiles feed the products directly (A is
// symmetric, so a tile read as the A operand is the block it transposes to).
// Products with fp32 operands use three-term bf16 splits (fp32-grade); u and
// k enter exactly.  The LDL^T elimination of I + C, carried along on E =
// U^T A_b K and on the identity (giving L^{-1} E and L^{-1}), runs in the
// wave over 32 pivots, two per round trip: pivot columns and rows reach
// every lane through LDS.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_mfma.h"
#include "vla_seq.h"

namespace vla {

namespace {

constexpr int kD = 64;   // head dimension
constexpr int kM = 32;   // tokens per block

// Feature held at basis index b: bits 2 and 3 swapped (an involution).
__host__ __device__ constexpr int feat(int b) { return (b & ~12) | ((b & 4) << 1) | ((b & 8) >> 1); }

// Orders a wave's LDS stores before its following LDS loads in the compiler
// (no forwarding of a lane's own store: the loads must see the other lanes'
// stores); the hardware completes one wave's LDS operations in issue order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Keeps the scheduler from hoisting the next group's operand splits above the
// current group's products, which would hold several split operands live at
// once and exceed the register budget of two waves per SIMD.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((address_space(3))) void lds_void;

// bf16 element e (0..7) of a 16-byte operand, as fp32.
__device__ __forceinline__ float frag_elem(const uint4& f, int e) {
  const uint32_t w = e < 2 ? f.x : e < 4 ? f.y : e < 6 ? f.z : f.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <bool UNIT_GATE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
vla_inverse_wy_kernel(const uint16_t* __restrict__ kx, const uint16_t* __restrict__ ux,
                      const float* __restrict__ a_start, float* __restrict__ alpha_out, float* __restrict__ A_T,
                      int32_t* __restrict__ chain_info, int T, int L, int nchunks, int chunk_lo, int chunk_cnt,
                      float eps, int nudge_period, int nudge_phase0) {
  __shared__ float4 sCol[2][2][4];   // pivot columns k, k + 1: [which][lane half][16 rows in slot order]
  __shared__ float4 sRow[kM][2];     // pivot rows k, k + 1 of (I + C, E, T) at column t
  __shared__ __align__(16) float sDinv[kM];     // 1 / pivot
  __shared__ float4 sTok[2][4][kD];   // the block's u and k operands: [u / k][k step][lane]

  const int64_t chain = blockIdx.x / chunk_cnt;
  const int chunk = chunk_lo + static_cast<int>(blockIdx.x % chunk_cnt);
  const int tbeg = chunk * L, tend = min(T, tbeg + L);
  const int lane0 = threadIdx.x, c0 = lane0 & 31, h0 = lane0 >> 5;

  // ---- A_b: tile (F, I) slot s = A[feat(32F + acc_row(s, h))][feat(32I + c)].
  // Slot s = 4 q + e sits at row 32F + 16 (q >> 1) + 8 h + 4 (q & 1) + e: a
  // per-lane byte offset plus a constant one, passed as the buffer access's
  // scalar offset so no per-element address stays live.
  const int a_voff = (8 * h0 * kD + feat(c0)) * 4;
  auto a_soff = [](int F, int I, int s) {
    const int q = s >> 2, e = s & 3;
    return ((32 * F + 16 * (q >> 1) + 4 * (q & 1) + e) * kD + 32 * I) * 4;
  };
  f32x16 Acc[2][2];
  {
    const auto ra = make_rsrc(a_start + (chain * nchunks + chunk) * kD * kD, kD * kD * 4);
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int s = 0; s < 16; ++s)
          Acc[F][I][s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, a_voff, a_soff(F, I, s), 0));
  }

  // Token rows go from HBM straight into LDS (buffer-to-LDS copies, no
  // registers held while they fly): lane (c, h) takes features 16 kappa +
  // 8 h .. + 7 of token c of the block for k step kappa.  The buffers end at
  // the chunk's last token, so rows past it read as zero.
  // Both buffers start at the chunk's first token, so their extents and
  // offsets stay below one chunk (at most 512 tokens) whatever T is.
  const int64_t row0 = chain * T + tbeg;
  const auto ru = make_rsrc(ux + row0 * kD, (tend - tbeg) * kD * 2);
  const auto rk = make_rsrc(kx + row0 * kD, (tend - tbeg) * kD * 2);
  auto copy_tokens = [&](int tb) {
    const int vo = ((tb - tbeg + c0) * kD + 8 * h0) * 2;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void*)&sTok[0][kp][0], 16, vo + 32 * kp, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)&sTok[1][kp][0], 16, vo + 32 * kp, 0, 0, 0);
    }
  };

  const bool nudge_last = nudge_period > 0 && tend > tbeg && (nudge_phase0 + tend - 1) % nudge_period == 0;
  int guard = 0;
  bool bad = false;
  copy_tokens(tbeg);

  for (int tb = tbeg; tb < tend; tb += kM) {
    // Lane indices laundered per block: values derived from them are then
    // recomputed in each block instead of being hoisted and kept live.
    int c = c0, h = h0;
    asm volatile("" : "+v"(c), "+v"(h));
    const int lane = c + 32 * h;
    // This wave's copies of the block's rows have landed (the compiler does
    // not order LDS reads after buffer-to-LDS copies by itself).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint4 uf[4], kf[4];
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const float4 a = sTok[0][kp][lane], b = sTok[1][kp][lane];
      uf[kp] = make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
      kf[kp] = make_uint4(__float_as_uint(b.x), __float_as_uint(b.y), __float_as_uint(b.z), __float_as_uint(b.w));
    }
    // ---- X_U = A U, X_K = A K (rows: basis features, columns: tokens) and
    // X_U^T (rows: tokens, columns: basis features).
    f32x16 XU[2] = {zero16(), zero16()}, XK[2] = {zero16(), zero16()}, XUT[2] = {zero16(), zero16()};
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int kp = 2 * F + g;
        const bf16x8 ub = __builtin_bit_cast(bf16x8, uf[kp]), kb = __builtin_bit_cast(bf16x8, kf[kp]);
#pragma unroll
        for (int I = 0; I < 2; ++I) {
          const Split3 af = split_slots(Acc[F][I], g);
          XU[I] = mma_split(af, ub, XU[I]);
          XK[I] = mma_split(af, kb, XK[I]);
          XUT[I] = mma_split(ub, af, XUT[I]);
          sched_fence();
        }
      }

    // ---- C = U^T X_U, E = U^T X_K (tokens x tokens).
    f32x16 Cm = zero16(), Em = zero16();
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const bf16x8 ub = __builtin_bit_cast(bf16x8, uf[2 * I + g]);
        Cm = mma_split(ub, split_slots(XU[I], g), Cm);
        Em = mma_split(ub, split_slots(XK[I], g), Em);
        sched_fence();
      }

    // The next block's rows start their copy (this block's stay in
    // registers; the last block keeps them for the nudge).
    if (tb + kM < tend) {
      lds_order();
      copy_tokens(tb + kM);
    }

    // ---- LDL^T elimination of I + C, applied to E and to the identity.
    // Lane (c, h) holds column c of each; pivot k sits in lane half
    // (k >> 2) & 1, slot 4 (k >> 3) + (k & 3).
    // Plain arrays from here: element updates of the accumulator vectors
    // would keep extra copies of the register tuples alive.
    float cm[16], em[16], tm[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const bool dg = acc_row(s, h) == c;
      cm[s] = Cm[s] + (dg ? 1.f : 0.f);
      em[s] = Em[s];
      tm[s] = dg ? 1.f : 0.f;
    }
    const float hf = static_cast<float>(h);
    // Two pivots per LDS round trip: the lanes get columns k and k + 1 and
    // rows k and k + 1 as they stood before pivot k, and apply pivot k to
    // their copies of column and row k + 1 themselves.
#pragma unroll
    for (int k = 0; k < kM; k += 2) {
      const int hk = (k >> 2) & 1, sk = 4 * (k >> 3) + (k & 3);   // pivots k, k + 1: slots sk, sk + 1
      if (c == k || c == k + 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sCol[c - k][h][q] = make_float4(cm[4 * q], cm[4 * q + 1], cm[4 * q + 2], cm[4 * q + 3]);
      }
      if (h == hk) {
        sRow[c][0] = make_float4(cm[sk], em[sk], tm[sk], cm[sk + 1]);
        sRow[c][1] = make_float4(em[sk + 1], tm[sk + 1], 0.f, 0.f);
      }
      lds_order();
      float na[16], nb[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = sCol[0][h][q], w = sCol[1][h][q];
        na[4 * q] = v.x; na[4 * q + 1] = v.y; na[4 * q + 2] = v.z; na[4 * q + 3] = v.w;
        nb[4 * q] = w.x; nb[4 * q + 1] = w.y; nb[4 * q + 2] = w.z; nb[4 * q + 3] = w.w;
      }
      // M[k][k], M[k+1][k] from column k; M[k][k+1], M[k+1][k+1] from column k + 1.
      const float2 pa = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(sCol[0][hk]) + sk);
      const float2 pb = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(sCol[1][hk]) + sk);
      const float4 r0 = sRow[c][0], r1 = sRow[c][1];
      float ia = __builtin_amdgcn_rcpf(pa.x);
      ia = fmaf(fmaf(-pa.x, ia, 1.f), ia, ia);
      const float a0 = r0.x * ia, a1 = r0.y * ia, a2 = r0.z * ia;
      // Row k + 1 at column c and pivot k + 1, as pivot k leaves them.
      const float q0 = fmaf(-pa.y, a0, r0.w), q1 = fmaf(-pa.y, a1, r1.x), q2 = fmaf(-pa.y, a2, r1.y);
      const float gab = pb.x * ia;
      const float pk1 = fmaf(-pa.y, gab, pb.y);
      float ib = __builtin_amdgcn_rcpf(pk1);
      ib = fmaf(fmaf(-pk1, ib, 1.f), ib, ib);
      const float b0 = q0 * ib, b1 = q1 * ib, b2 = q2 * ib;
      guard += (fabsf(pa.x) < eps ? 1 : 0) + (fabsf(pk1) < eps ? 1 : 0);
      asm volatile("" : "+v"(guard));
      if (lane == 0) {
        sDinv[k] = ia;
        sDinv[k + 1] = ib;
      }
      lds_order();
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int base = 8 * (s >> 2) + (s & 3);   // row of slot s is base + 4 h
        if (base + 4 <= k) continue;                // row <= k in both halves
        // Pivot k on the rows below it.
        const float xa = base > k ? na[s] : na[s] * hf;
        cm[s] = fmaf(-xa, a0, cm[s]);
        em[s] = fmaf(-xa, a1, em[s]);
        tm[s] = fmaf(-xa, a2, tm[s]);
        // Pivot k + 1 on the rows below it, with column k + 1 as pivot k left it.
        if (base + 4 > k + 1) {
          const float nk = fmaf(-na[s], gab, nb[s]);
          const float xb = base > k + 1 ? nk : nk * hf;
          cm[s] = fmaf(-xb, b0, cm[s]);
          em[s] = fmaf(-xb, b1, em[s]);
          tm[s] = fmaf(-xb, b2, tm[s]);
        }
        // Pin the updated values: left alone, the compiler defers these
        // products to the values' next uses and keeps every factor live.
        asm volatile("" : "+v"(cm[s]), "+v"(em[s]), "+v"(tm[s]));
      }
    }

    // ---- W = T^T D^{-1} T and G = T^T D^{-1} (F o M) with T = L^{-1}, F = L^{-1} E.
    float dv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(sDinv + 8 * q + 4 * h);
      dv[4 * q] = v.x; dv[4 * q + 1] = v.y; dv[4 * q + 2] = v.z; dv[4 * q + 3] = v.w;
    }
    f32x16 Wm = zero16(), Gm = zero16();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float td[8], tt[8], ff[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = 8 * g + e;
        td[e] = tm[s] * dv[s];
        tt[e] = tm[s];
        ff[e] = acc_row(s, h) <= c ? em[s] : 0.f;
      }
      const Split3 TD = split3(td);
      Wm = mma_split(TD, split3(tt), Wm);
      Gm = mma_split(TD, split3(ff), Gm);
    }

    // ---- P = W X_U^T (tokens x basis features); alpha = X_K - X_U G.
    Split3 XS[2][2];
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
      for (int g = 0; g < 2; ++g) XS[I][g] = split_slots(XUT[I], g);
    f32x16 PT[2] = {zero16(), zero16()};
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const Split3 WS = split_slots(Wm, g), GS = split_slots(Gm, g, -1.f);
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        PT[I] = mma_split(WS, XS[I][g], PT[I]);
        XK[I] = mma_split(XS[I][g], GS, XK[I]);
      }
    }

    // ---- alpha_hat of the block's tokens (token c, basis rows of XK).
    const int tcount = min(kM, tend - tb);
    if (nudge_last && tb + kM >= tend && c == tcount - 1) {
      // The chunk's last token is nudged: alpha = (A + eps I) k.
#pragma unroll
      for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int s = 0; s < 16; ++s) XK[I][s] = fmaf(eps, frag_elem(kf[2 * I + (s >> 3)], s & 7), XK[I][s]);
    }
    float nrm = 0.f;
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
      for (int s = 0; s < 16; ++s) nrm = fmaf(XK[I][s], XK[I][s], nrm);
    nrm += __shfl_xor(nrm, 32);
    float ascale = nrm > 1.f ? 1.f / sqrtf(nrm) : 1.f;
    if constexpr (UNIT_GATE) {
      // The residual update's gate: the unit vector along A k_hat, k_hat = k / |k|.
      float kn = 0.f;
#pragma unroll
      for (int kp = 0; kp < 4; ++kp)
#pragma unroll
        for (int e = 0; e < 8; ++e) kn = fmaf(frag_elem(kf[kp], e), frag_elem(kf[kp], e), kn);
      kn += __shfl_xor(kn, 32);
      const float kinv = 1.f / fmaxf(sqrtf(kn), 1e-12f);
      ascale = kinv / fmaxf(kinv * sqrtf(nrm), 1e-12f);
    }
    if (c < tcount) {
      float* dst = alpha_out + (chain * T + tb + c) * kD;
#pragma unroll
      for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = make_float4(XK[I][4 * q] * ascale, XK[I][4 * q + 1] * ascale, XK[I][4 * q + 2] * ascale,
                                       XK[I][4 * q + 3] * ascale);
          bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
          *reinterpret_cast<float4*>(dst + feat(32 * I + 4 * (2 * q + h))) = v;
        }
    }

    // ---- A_{b+1} = A_b - P^T X_U^T.
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int F = 0; F < 2; ++F) {
        const Split3 PS = split_slots(PT[F], g, -1.f);
#pragma unroll
        for (int I = 0; I < 2; ++I) Acc[F][I] = mma_split(PS, XS[I][g], Acc[F][I]);
      }
  }

  // ---- the chunk's end state: nudge, and A_T from the last chunk.
  if (nudge_last) {
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int s = 0; s < 16; ++s) Acc[F][F][s] += acc_row(s, h0) == c0 ? eps : 0.f;
  }
  if (chunk == nchunks - 1) {
    const auto rt = make_rsrc(A_T + chain * kD * kD, kD * kD * 4);
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const float v = Acc[F][I][s];
          bad |= !isfinite(v);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rt, a_voff, a_soff(F, I, s), 0);
        }
  }
  const bool wave_bad = __any(bad);
  if (lane0 == 0) {
    int32_t* info = chain_info + chain * 4;
    if (guard > 0) {
      atomicAdd(info + kInfoGuard, guard);
      atomicOr(info + kInfoFallback, 1);
    }
    if (wave_bad) atomicOr(info + kInfoNonfinite, 1);
  }
}

}  // namespace

hipError_t launch_inverse_wy(const ScanArgs& a, const float* a_start, float* alpha_out, int32_t* chain_info,
                             int chunk_len, int nchunks, int chunk_lo, int chunk_cnt, int chains, hipStream_t stream) {
  if (chunk_cnt <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(chains * chunk_cnt));
  if (a.residual)
    hipLaunchKernelGGL(vla_inverse_wy_kernel<true>, grid, dim3(64), 0, stream, static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.u), a_start, alpha_out, a.A_T, chain_info, a.T, chunk_len,
                       nchunks, chunk_lo, chunk_cnt, a.eps, a.nudge_period, a.nudge_phase0);
  else
    hipLaunchKernelGGL(vla_inverse_wy_kernel<false>, grid, dim3(64), 0, stream, static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.u), a_start, alpha_out, a.A_T, chain_info, a.T, chunk_len,
                       nchunks, chunk_lo, chunk_cnt, a.eps, a.nudge_period, a.nudge_phase0);
  return hipGetLastError();
}

}  // namespace vla
