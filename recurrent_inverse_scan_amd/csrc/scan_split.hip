// Sequential VLA scan for d <= 64 with the two recurrences on separate waves.
//
// Method as in the sequential kernel ("Mathematical Primitives", sections
// 2-5; "Variational Linear Attention (VLA)" README, v3 notes; the residual
// update from "Variational Linear Attention: Stable Associative Memory for
// Long-Context Transformers", technical summary 2.3).  Per token the inverse
// recurrence (r guarded Sherman-Morrison updates of A, the nudge, alpha = A k)
// never reads the state S, and the state recurrence (S += w alpha_hat^T, the
// cap, n += k, the readout) needs only alpha from it.  So one workgroup runs
// a chain: wave 0 the inverse side, wave 2 the state side one LDS stage (8
// or 16 tokens) behind, alpha passed through LDS and normalised by the state
// wave (it holds the columns of alpha and k, so both norms are group sums).
// A token then costs the longer of the two halves instead of their sum; each
// wave keeps only its own matrix in registers.  Wave 1 does no work and only
// takes part in the barriers: with the two sides as waves 0 and 1 they were
// measured to compete for issue (recall workload 0.73 ms, against 0.56 ms
// with the middle wave, which equals the inverse side's time alone).
//
// Synchronisation: every loop iteration ends with the one workgroup barrier,
// taken by all three waves the same number of times (the trip count depends
// on T only).  Inside a side, the vector broadcasts go through LDS within one
// wave: the hardware completes a wave's LDS operations in issue order, and
// lds_order() keeps the compiler from moving a load above an earlier store.
// Stage buffers rotate over three slots: the one being filled, the one the
// inverse wave reads, the one the state wave reads.
//
// Fused prologue (FUSED): the kernel streams q_raw, k_raw and v and builds the
// rest of each token itself: u_i = normalize(W_u[i] k_raw) ("Variational
// Linear Attention (VLA)" README, v3 notes item 2) and q, k = ELU(.) + 1
// (item 1), so u never exists in HBM.  Wave 1, otherwise idle, does it one
// stage ahead of the inverse wave (a fourth slot): the projection of a
// stage's 16-token tile on the matrix cores (bf16 storage: 16x16x32 bf16,
// float32: 16x16x4 f32, accumulating in float32), the row norms by 16-lane
// sums, then the feature map in place.  Features and u are rounded to the
// storage dtype, as when they are computed upstream and stored.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_seq.h"
#include "vla_wave.h"

namespace vla {

namespace {

constexpr int kSplitSlots = 3;   // stage buffers in rotation
constexpr int kFusedSlots = 4;   // with the fused prologue: one more, for wave 1's stage
constexpr int kSplitThreads = 192;   // inverse wave, spacer wave, state wave
constexpr int kStageThreads = 128;   // the two working waves stage the rows

__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Tokens per LDS stage: 16 when the stage fits the staging registers and the
// three slots stay within 60 KiB, else 8.
// (NV rows per token in LDS, NL of them loaded from HBM, `slots` buffers;
// two workgroups still fit a compute unit's 160 KiB with four slots.)
template <typename TIn, int D>
__host__ __device__ constexpr int split_stage_tokens(int NV, int NL, int slots) {
  const int vpr = D / Elem<TIn>::kPer16B;
  const int lds16 = static_cast<int>(sizeof(float)) * (slots * 16 * NV * D + 2 * 16 * D + D + 8);
  const int cap = (slots == kFusedSlots ? 78 : 60) * 1024;
  return (16 * NL * vpr <= kMaxStageVecs * kStageThreads && lds16 <= cap) ? 16 : 8;
}
template <typename TIn, int D>
inline size_t split_lds_bytes(int NV, int NL, int slots) {
  const int TT = split_stage_tokens<TIn, D>(NV, NL, slots);
  return sizeof(float) * (static_cast<size_t>(slots) * TT * NV * D + 2 * TT * D + D + 8);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float round_to(float x, const float*) { return x; }
__device__ __forceinline__ float round_to(float x, const uint16_t*) { return bf16_to_f32(f32_to_bf16(x)); }

// Wave 1's prologue for one stage (fused mode): slot rows per token are
// q_raw, k_raw, v, then u_1..u_r to be written; tokens >= TT do not exist.
// The projection runs on 16-token tiles: lane l is token l % 16 of the A
// operand and output column l % 16 of the B operand, k slice by l / 16; the
// accumulator holds rows 4 (l / 16) + s.
template <typename TIn, int D>
__device__ __forceinline__ void fused_prologue(float* sb, int NV, int TT, int r, const TIn* __restrict__ W,
                                               int lane) {
  const int tok = lane & 15, grp = lane >> 4;
  constexpr int NB = D / 16 > 0 ? D / 16 : 1;   // 16-column output tiles
  for (int i = 0; i < r; ++i) {
    f32x4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const TIn* Wi = W + static_cast<int64_t>(i) * D * D;
    if constexpr (sizeof(TIn) == 2) {
      constexpr int KS = (D + 31) / 32;   // 32-wide k steps (d = 16 pads with zeros)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k0 = 32 * ks + 8 * grp;
        uint32_t aw[4] = {0u, 0u, 0u, 0u};
        if (tok < TT && k0 < D) {
          const float* src = sb + (tok * NV + 1) * D + k0;   // k_raw row: exact bf16 values
#pragma unroll
          for (int h = 0; h < 4; ++h)
            aw[h] = (__float_as_uint(src[2 * h]) >> 16) | (__float_as_uint(src[2 * h + 1]) & 0xffff0000u);
        }
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          uint4 bw = make_uint4(0u, 0u, 0u, 0u);
          if (k0 < D) bw = *reinterpret_cast<const uint4*>(Wi + (nb * 16 + tok) * D + k0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bw), acc[nb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < D / 4; ++kb) {
        const int kk = 4 * kb + grp;
        const float a = tok < TT ? sb[(tok * NV + 1) * D + kk] : 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Wi[(nb * 16 + tok) * D + kk], acc[nb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float ss = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) ss = fmaf(acc[nb][s], acc[nb][s], ss);
      ss = group_sum<16>(ss);   // the 16 lanes of this row's columns
      const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
      const int t = 4 * grp + s;
      if (t < TT) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          if (nb * 16 + tok < D)
            sb[(t * NV + 3 + i) * D + nb * 16 + tok] = round_to(acc[nb][s] * inv, static_cast<const TIn*>(nullptr));
      }
    }
  }
  // The projection's reads of k_raw come before the feature map overwrites it
  // (one wave's LDS operations complete in order).
  asm volatile("" ::: "memory");
  for (int e = lane; e < TT * 2 * D; e += 64) {
    const int t = e / (2 * D), rr = (e / D) & 1, c = e % D;
    float* p = sb + (t * NV + rr) * D + c;
    const float x = *p;
    *p = round_to((x > 0.f ? x : expm1f(x)) + 1.f, static_cast<const TIn*>(nullptr));
  }
}

template <typename TIn, int D, int CG, bool RES, bool FUSED>
__global__ void __launch_bounds__(kSplitThreads) vla_scan_split_kernel(ScanArgs a) {
  using L = TileLayout<D, 1, CG>;
  constexpr int R = L::R, C = L::C;
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);

  const int64_t chain = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const bool inverse_side = wave == 0, spacer = wave == 1;
  const int tid = inverse_side ? threadIdx.x : threadIdx.x - 64;   // 0..127 over the working waves
  const int lane = threadIdx.x & 63;
  const int cg = lane % CG, rg = lane / CG;
  const int row0 = rg * R;
  const int r = a.r;
  const int NV = 3 + r;   // q, k, v, u_1..u_r
  const int NL = FUSED ? 3 : NV;   // rows per token loaded from HBM
  constexpr int kSlots = FUSED ? kFusedSlots : kSplitSlots;
  constexpr int kLag = FUSED ? 1 : 0;   // stages between staging and the inverse wave
  constexpr int row_q = 0, row_k = 1, row_v = 2, row_u = 3;
  const int TT = split_stage_tokens<TIn, D>(NV, NL, kSlots);
  const int slot_floats = TT * NV * D;

  float* stage = smem;                                   // [kSlots][TT][NV][D]
  float* ahat = stage + kSlots * slot_floats;            // [2][TT][D]
  float* zb = ahat + 2 * TT * D;                   // [D]
  int32_t* fin = reinterpret_cast<int32_t*>(zb + D);     // [8] per-side statistics (exact counts)

  const int64_t tok0 = chain * a.T;
  RowSource<TIn, D> src;
  src.n = NL;
  src.nfix = 3;
  src.fix0 = static_cast<const TIn*>(a.q) + tok0 * D;
  src.fix1 = static_cast<const TIn*>(a.k) + tok0 * D;
  src.fix2 = static_cast<const TIn*>(a.v) + tok0 * D;
  src.ubase = FUSED ? nullptr : static_cast<const TIn*>(a.u) + tok0 * r * D;
  src.ustride = static_cast<int64_t>(r) * D;
  Stager<TIn, D, kStageThreads> st;

  // Registers of each side: A on the inverse wave, S and n on the state wave.
  float M[R][C], n[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      float4 mv;
      if (inverse_side) {
        mv = make_float4(row == col ? 1.f : 0.f, row == col + 1 ? 1.f : 0.f, row == col + 2 ? 1.f : 0.f,
                         row == col + 3 ? 1.f : 0.f);
        if (a.A0) mv = *reinterpret_cast<const float4*>(a.A0 + (chain * D + row) * D + col);
      } else {
        mv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a.S0) mv = *reinterpret_cast<const float4*>(a.S0 + (chain * D + row) * D + col);
      }
      M[i][4 * m] = mv.x; M[i][4 * m + 1] = mv.y; M[i][4 * m + 2] = mv.z; M[i][4 * m + 3] = mv.w;
    }
    n[i] = (!inverse_side && a.n0) ? a.n0[chain * D + row] : 0.f;
  }

  int guard_fires = 0, cap_fires = 0, first_cap = -1;
  bool bad = false;
  // The eps*I shifts are carried as a scalar: the inverse is M + shift*I.
  float shift = 0.f;
  int phase = a.nudge_period > 0 ? a.nudge_phase0 % a.nudge_period : 0;
  const float cap2 = a.cap * a.cap;

  const int nstage = (a.T + TT - 1) / TT;
  if (nstage > 0 && !spacer) {
    st.load(src, 0, TT, a.T, tid);
    st.store(stage, TT, NL, tid, NV);
  }
  __syncthreads();

  for (int it = 0; it <= nstage + kLag; ++it) {
    if (it + 1 < nstage && !spacer) st.load(src, (it + 1) * TT, TT, a.T, tid);
    const int si = it - kLag;   // the inverse wave's stage

    if constexpr (FUSED) {
      if (spacer && it < nstage)
        fused_prologue<TIn, D>(stage + (it % kSlots) * slot_floats, NV, TT, r, static_cast<const TIn*>(a.W_u), lane);
    }
    if (inverse_side && si >= 0 && si < nstage) {
      // ---- inverse recurrence over stage si ------------------------------
      const float* sbuf = stage + (si % kSlots) * slot_floats;
      float* aout = ahat + (si & 1) * TT * D;
      const int tcount = min(TT, a.T - si * TT);
      for (int tt = 0; tt < tcount; ++tt) {
        const float* tblk = sbuf + tt * NV * D;
        const float* tk = tblk + row_k * D;
        float kI[R], y[R];
        lds_rows<R>(tk + row0, kI);
        bool last_fired = false;
        for (int i = 0; i < r; ++i) {
          const float* tu = tblk + (row_u + i) * D;
          const bool last = i == r - 1;
          float uJ[C], z[R];
          lds_cols<CG, C>(tu, cg, uJ);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) acc = fmaf(M[ii][c], uJ[c], acc);
            z[ii] = acc;
          }
          if (last) {
            float kJ[C];
            lds_cols<CG, C>(tk, cg, kJ);
#pragma unroll
            for (int ii = 0; ii < R; ++ii) {
              float acc = 0.f;
#pragma unroll
              for (int c = 0; c < C; ++c) acc = fmaf(M[ii][c], kJ[c], acc);
              y[ii] = fmaf(shift, kI[ii], group_sum<CG>(acc));
            }
          }
          float uI[R];
          lds_rows<R>(tu + row0, uI);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) z[ii] = fmaf(shift, uI[ii], group_sum<CG>(z[ii]));
          // z goes to LDS first, so its round trip overlaps the reductions.
          lds_order();   // the previous sub-update's reads of zb come first
          if (cg == 0) lds_store_rows<R>(zb + row0, z);
          lds_order();
          float du = 0.f, dk = 0.f;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            du = fmaf(z[ii], uI[ii], du);
            dk = fmaf(z[ii], kI[ii], dk);
          }
          du = wave_total(cg == 0 ? du : 0.f);
          if (last) dk = wave_total(cg == 0 ? dk : 0.f);
          float zJ[C];
          lds_cols<CG, C>(zb, cg, zJ);
          const float delta = 1.f + du;
          const bool fire = fabsf(delta) < a.eps;
          if (fire) {
            // Singularity guard: inject eps*I and skip this rank-1 update.
            ++guard_fires;
            shift += a.eps;
            if (last) last_fired = true;
          }
          // A zero coefficient when the guard fired keeps A in place.
          const float inv = fire ? 0.f : 1.f / delta;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            const float zs = z[ii] * inv;
#pragma unroll
            for (int c = 0; c < C; ++c) M[ii][c] = fmaf(-zs, zJ[c], M[ii][c]);
          }
          if (last) {
            const float g = dk * inv;
#pragma unroll
            for (int ii = 0; ii < R; ++ii) y[ii] = fmaf(-z[ii], g, y[ii]);
          }
        }
        // Nudge and coefficient; the state wave normalises it (it holds the
        // columns of alpha and of k, so both norms need no wave reduction).
        float alpha[R];
#pragma unroll
        for (int ii = 0; ii < R; ++ii) alpha[ii] = last_fired ? fmaf(a.eps, kI[ii], y[ii]) : y[ii];
        if (a.nudge_period > 0) {
          if (phase == 0) {
#pragma unroll
            for (int ii = 0; ii < R; ++ii) alpha[ii] = fmaf(a.eps, kI[ii], alpha[ii]);
            shift += a.eps;
          }
          phase = (phase + 1 == a.nudge_period) ? 0 : phase + 1;
        }
        if (cg == 0) {
#pragma unroll
          for (int ii = 0; ii < R; ++ii) bad |= !isfinite(alpha[ii]);
          lds_store_rows<R>(aout + tt * D + row0, alpha);
        }
      }
    } else if (!inverse_side && !spacer && si >= 1) {
      // ---- state recurrence over stage si - 1 ----------------------------
      const int sidx = si - 1;
      const float* sbuf = stage + (sidx % kSlots) * slot_floats;
      const float* ain = ahat + (sidx & 1) * TT * D;
      const int tb = sidx * TT;
      const int tcount = min(TT, a.T - tb);
      for (int tt = 0; tt < tcount; ++tt) {
        const int t = tb + tt;
        const float* tblk = sbuf + tt * NV * D;
        const float* tq = tblk + row_q * D;
        const float* tk = tblk + row_k * D;
        const float* tv = tblk + row_v * D;
        float kI[R], vI[R], qI[R], qJ[C], aJ[C];
        lds_rows<R>(tk + row0, kI);
        lds_rows<R>(tv + row0, vI);
        float kinv = 1.f;
        if constexpr (RES) {
          // v - S_{t-1} k_hat, the prediction taken before the update.
          float kJ[C];
          lds_cols<CG, C>(tk, cg, kJ);
          float kn = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) kn = fmaf(kJ[c], kJ[c], kn);
          kn = group_sum<CG>(kn);   // a row group's lanes hold every column
          kinv = 1.f / fmaxf(sqrtf(kn), 1e-12f);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) acc = fmaf(M[ii][c], kJ[c], acc);
            vI[ii] = fmaf(-group_sum<CG>(acc), kinv, vI[ii]);
          }
        }
        lds_rows<R>(tq + row0, qI);
        lds_cols<CG, C>(tq, cg, qJ);
        lds_cols<CG, C>(ain + tt * D, cg, aJ);
        {
          // alpha_hat: additive, alpha / max(|alpha|, 1); residual, the unit
          // vector along A k_hat = kinv A k.
          float an = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) an = fmaf(aJ[c], aJ[c], an);
          an = group_sum<CG>(an);
          const float ascale = RES ? kinv / fmaxf(kinv * sqrtf(an), 1e-12f) : (an > 1.f ? 1.f / sqrtf(an) : 1.f);
#pragma unroll
          for (int c = 0; c < C; ++c) aJ[c] *= ascale;
        }
        float ns = 0.f, po[R];
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) {
            M[ii][c] = fmaf(vI[ii], aJ[c], M[ii][c]);
            ns = fmaf(M[ii][c], M[ii][c], ns);
            acc = fmaf(M[ii][c], qJ[c], acc);
          }
          po[ii] = group_sum<CG>(acc);
        }
        float nq = 0.f;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          n[ii] += kI[ii];
          nq = fmaf(n[ii], qI[ii], nq);
        }
        ns = wave_total(ns);
        nq = wave_total(cg == 0 ? nq : 0.f);
        float oscale = 1.f;
        if (a.cap_on && ns > cap2) {
          // Frobenius renormalisation: S <- S * cap / |S|_F.
          oscale = a.cap / sqrtf(ns);
#pragma unroll
          for (int ii = 0; ii < R; ++ii)
#pragma unroll
            for (int c = 0; c < C; ++c) M[ii][c] *= oscale;
          if (first_cap < 0) first_cap = t;
          ++cap_fires;
        }
        const float f = oscale / (nq + a.den_eps);
        if (cg == 0) {
          TIn* op = static_cast<TIn*>(a.o) + (tok0 + t) * D + row0;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            const float ov = po[ii] * f;
            bad |= !isfinite(ov);
            Elem<TIn>::store(op + ii, ov);
          }
        }
      }
    }

    if (it + 1 < nstage && !spacer) st.store(stage + ((it + 1) % kSlots) * slot_floats, TT, NL, tid, NV);
    __syncthreads();
  }

  // ---- final state and statistics ---------------------------------------
  if (inverse_side) add_to_diagonal<R, C, CG>(M, row0, cg, shift);
  float* dstM = inverse_side ? a.A_T : a.S_T;
#pragma unroll
  for (int i = 0; i < (spacer ? 0 : R); ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      *reinterpret_cast<float4*>(dstM + (chain * D + row) * D + col) =
          make_float4(M[i][4 * m], M[i][4 * m + 1], M[i][4 * m + 2], M[i][4 * m + 3]);
#pragma unroll
      for (int c = 0; c < 4; ++c) bad |= !isfinite(M[i][4 * m + c]);
    }
    if (!inverse_side && cg == 0) {
      a.n_T[chain * D + row] = n[i];
      bad |= !isfinite(n[i]);
    }
  }
  if (a.stats) {
    const bool wave_bad = __any(bad);
    if (lane == 0 && !spacer) {
      if (inverse_side) {
        fin[0] = guard_fires;
        fin[1] = wave_bad ? 1 : 0;
      } else {
        fin[2] = cap_fires;
        fin[3] = first_cap;
        fin[4] = wave_bad ? 1 : 0;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int32_t* s = a.stats + chain * 4;
      s[0] = fin[0];
      s[1] = fin[2];
      s[2] = (fin[1] | fin[4]) ? 1 : 0;
      s[3] = fin[3];
    }
  }
}

template <typename TIn, int D, int CG>
hipError_t launch_split(const ScanArgs& a, int chains, hipStream_t stream) {
  using L = TileLayout<D, 1, CG>;
  static_assert(L::R >= 1, "layout");
  const int NV = 3 + a.r;
  const bool fused = a.fused != 0;
  const int NL = fused ? 3 : NV;
  const int slots = fused ? kFusedSlots : kSplitSlots;
  // Every stage fits the staging registers of the workgroup.
  if (8 * NL * (D / Elem<TIn>::kPer16B) > kMaxStageVecs * kStageThreads) return hipErrorInvalidValue;
  if (fused && (a.r > 4 || !a.W_u)) return hipErrorInvalidValue;
  const size_t lds = split_lds_bytes<TIn, D>(NV, NL, slots);
  const dim3 grid(static_cast<unsigned>(chains));
#define VLA_SPLIT(RES_, FUSED_) \
  hipLaunchKernelGGL((vla_scan_split_kernel<TIn, D, CG, RES_, FUSED_>), grid, dim3(kSplitThreads), lds, stream, a)
  if (fused) {
    if (a.residual) VLA_SPLIT(true, true); else VLA_SPLIT(false, true);
  } else {
    if (a.residual) VLA_SPLIT(true, false); else VLA_SPLIT(false, false);
  }
#undef VLA_SPLIT
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_split(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream) {
  if (chains <= 0) return hipSuccess;
  switch (d) {
    case 16: return bf16 ? launch_split<uint16_t, 16, 4>(a, chains, stream) : launch_split<float, 16, 4>(a, chains, stream);
    case 32: return bf16 ? launch_split<uint16_t, 32, 4>(a, chains, stream) : launch_split<float, 32, 4>(a, chains, stream);
    case 64: return bf16 ? launch_split<uint16_t, 64, 4>(a, chains, stream) : launch_split<float, 64, 4>(a, chains, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_split_fused(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream) {
  if (!a.fused) return hipErrorInvalidValue;
  return launch_scan_split(a, d, bf16, chains, stream);
}

}  // namespace vla
