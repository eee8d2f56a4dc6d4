// Sequential-schedule VLA scan kernel for gfx950 (CDNA4, wave64).
//
// One workgroup owns one (batch, head) chain for a run of tokens, starting
// from a given state (A, S, n) and ending by writing the final state.  The
// tracked inverse A and the fast-weight state S stay in registers for the
// whole run; q, k, v, u stream through a double-buffered LDS stage.
//
// Method ("Mathematical Primitives", sections 2-5; "Variational Linear
// Attention (VLA)" README, v3 notes): per token, r guarded Sherman-Morrison
// rank-1 updates of A, the periodic eps*I nudge, alpha = A_t k_t clamped to
// norm <= 1, S += v alpha_hat^T, the Frobenius cap, n += k and the readout
// o = S q / (n.q + den_eps).
//
// Register layout.  The NW waves of a workgroup split the d rows of A and S
// into slabs of RW = d/NW rows.  Inside a wave, lane = rg*CG + cg: the lane
// owns R = RW/(64/CG) consecutive rows and C = d/CG columns, the columns
// interleaved in float4 blocks, j = (m*CG + cg)*4 + e.  A row of a matrix
// vector product is therefore split over the CG lanes of a row group and
// summed with DPP; the column-indexed vectors every lane needs (u, k, q, z,
// alpha) are read from LDS, conflict-free, as float4 blocks.
//
// Fusion: the first matrix-vector sweep of a token computes both z = A u_r
// and y = A k (same A), and alpha = A_t k follows as y - z (z.k)/delta (or
// y + eps k when the guard fires), so A is swept twice per rank-1 update
// (product and update) instead of three times.
#include "vla_common.h"
#include "vla_kernels.h"

namespace vla {

namespace {

constexpr int kMaxStageVecs = 8;   // 16-byte staging registers per thread

template <int D, int NW, int CG>
struct Layout {
  static constexpr int kThreads = 64 * NW;
  static constexpr int RW = D / NW;    // rows per wave
  static constexpr int RG = 64 / CG;   // row groups per wave
  static constexpr int R = RW / RG;    // rows per lane
  static constexpr int C = D / CG;     // columns per lane
  static_assert(RW % RG == 0 && R >= 1, "each lane needs at least one row");
  static_assert(C % 4 == 0, "columns come in float4 blocks");
};

// Reads this lane's C columns of an LDS vector.
template <int D, int CG, int C>
__device__ __forceinline__ void lds_cols(const float* vec, int cg, float (&out)[C]) {
#pragma unroll
  for (int m = 0; m < C / 4; ++m) {
    const float4 x = *reinterpret_cast<const float4*>(vec + (m * CG + cg) * 4);
    out[4 * m + 0] = x.x; out[4 * m + 1] = x.y; out[4 * m + 2] = x.z; out[4 * m + 3] = x.w;
  }
}

// Reads this lane's R consecutive rows of an LDS vector.
template <int R>
__device__ __forceinline__ void lds_rows(const float* vec, float (&out)[R]) {
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(vec + 4 * i);
      out[4 * i + 0] = x.x; out[4 * i + 1] = x.y; out[4 * i + 2] = x.z; out[4 * i + 3] = x.w;
    }
  } else if constexpr (R == 2) {
    const float2 x = *reinterpret_cast<const float2*>(vec);
    out[0] = x.x; out[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) out[i] = vec[i];
  }
}

template <int R>
__device__ __forceinline__ void lds_store_rows(float* vec, const float (&in)[R]) {
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int i = 0; i < R / 4; ++i)
      *reinterpret_cast<float4*>(vec + 4 * i) = make_float4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
  } else if constexpr (R == 2) {
    *reinterpret_cast<float2*>(vec) = make_float2(in[0], in[1]);
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) vec[i] = in[i];
  }
}

// Streams tokens of one chain from HBM into an LDS stage [TT][NV][D] of
// float32, NV = 3 + r vectors per token (q, k, v, u_1..u_r).  Each thread
// moves up to kMaxStageVecs 16-byte vectors; tokens at or past T read as 0.
template <typename TIn, int D, int NTH>
struct Stager {
  static constexpr int EPV = Elem<TIn>::kPer16B;  // elements per 16 bytes
  static constexpr int VPR = D / EPV;             // 16-byte vectors per row
  uint4 reg[kMaxStageVecs];

  __device__ __forceinline__ void load(const ScanArgs& a, int64_t chain, int tb, int TT, int NV, int tid) {
    const int nvec = TT * NV * VPR;
#pragma unroll
    for (int j = 0; j < kMaxStageVecs; ++j) {
      const int e = tid + j * NTH;
      reg[j] = make_uint4(0, 0, 0, 0);
      if (e < nvec) {
        const int rho = e / VPR, c = e % VPR;
        const int tt = rho / NV, vv = rho - tt * NV;
        const int t = tb + tt;
        if (t < a.T) {
          const TIn* base;
          int64_t off;
          if (vv < 3) {
            base = static_cast<const TIn*>(vv == 0 ? a.q : (vv == 1 ? a.k : a.v));
            off = (chain * a.T + t) * D;
          } else {
            base = static_cast<const TIn*>(a.u);
            off = ((chain * a.T + t) * a.r + (vv - 3)) * D;
          }
          reg[j] = *reinterpret_cast<const uint4*>(base + off + c * EPV);
        }
      }
    }
  }

  __device__ __forceinline__ void store(float* stage, int TT, int NV, int tid) const {
    const int nvec = TT * NV * VPR;
#pragma unroll
    for (int j = 0; j < kMaxStageVecs; ++j) {
      const int e = tid + j * NTH;
      if (e < nvec) {
        const int rho = e / VPR, c = e % VPR;
        float* dst = stage + rho * D + c * EPV;
        if constexpr (EPV == 4) {
          *reinterpret_cast<uint4*>(dst) = reg[j];
        } else {
          const uint32_t w[4] = {reg[j].x, reg[j].y, reg[j].z, reg[j].w};
          float f[8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            f[2 * h] = __uint_as_float(w[h] << 16);
            f[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
          }
          *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
    }
  }
};

}  // namespace

// Number of tokens per LDS stage for this (D, NW, r, dtype): one stage fits
// the per-thread staging registers and the two stages stay within 48 KiB.
template <typename TIn, int D, int NW>
__host__ __device__ constexpr int stage_tokens(int r) {
  constexpr int VPR = D / Elem<TIn>::kPer16B;
  int cap = (kMaxStageVecs * 64 * NW) / ((3 + r) * VPR);
  const int lds_cap = (48 * 1024) / (2 * (3 + r) * D * static_cast<int>(sizeof(float)));
  cap = cap < lds_cap ? cap : lds_cap;
  return cap >= 8 ? 8 : (cap < 1 ? 1 : cap);
}

template <typename TIn, int D, int NW, int CG>
__global__ void __launch_bounds__(64 * NW)
vla_scan_seq_kernel(ScanArgs a) {
  using L = Layout<D, NW, CG>;
  constexpr int R = L::R, C = L::C, RW = L::RW;
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int cg = lane % CG, rg = lane / CG;
  const int row0 = w * RW + rg * R;
  const int64_t chain = blockIdx.x;
  const int r = a.r, NV = 3 + r;
  const int TT = stage_tokens<TIn, D, NW>(r);

  float* stage = smem;                              // [2][TT][NV][D]
  float* zbuf = stage + 2 * TT * NV * D;            // [2][D]
  float* abuf = zbuf + 2 * D;                       // [2][D]
  float* red = abuf + 2 * D;                        // [2][NW][4]

  // ---- initial state --------------------------------------------------
  float A[R][C], S[R][C], n[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      float4 av = make_float4(row == col ? 1.f : 0.f, row == col + 1 ? 1.f : 0.f,
                              row == col + 2 ? 1.f : 0.f, row == col + 3 ? 1.f : 0.f);
      float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.A0) av = *reinterpret_cast<const float4*>(a.A0 + (chain * D + row) * D + col);
      if (a.S0) sv = *reinterpret_cast<const float4*>(a.S0 + (chain * D + row) * D + col);
      A[i][4 * m] = av.x; A[i][4 * m + 1] = av.y; A[i][4 * m + 2] = av.z; A[i][4 * m + 3] = av.w;
      S[i][4 * m] = sv.x; S[i][4 * m + 1] = sv.y; S[i][4 * m + 2] = sv.z; S[i][4 * m + 3] = sv.w;
    }
    n[i] = a.n0 ? a.n0[chain * D + row] : 0.f;
  }

  int guard_fires = 0, cap_fires = 0, first_cap = -1;
  bool bad = false;
  int par = 0;
  int phase = a.nudge_phase0;  // (t0 + 1 + t) mod P for the current token
  const float cap2 = a.cap * a.cap;

  Stager<TIn, D, L::kThreads> st;
  const int nstage = (a.T + TT - 1) / TT;
  if (nstage > 0) {
    st.load(a, chain, 0, TT, NV, tid);
    st.store(stage, TT, NV, tid);
  }
  __syncthreads();

  for (int sidx = 0; sidx < nstage; ++sidx) {
    const int tb = sidx * TT;
    if (sidx + 1 < nstage) st.load(a, chain, tb + TT, TT, NV, tid);
    const float* sbuf = stage + (sidx & 1) * TT * NV * D;
    const int tcount = min(TT, a.T - tb);

    for (int tt = 0; tt < tcount; ++tt) {
      const int t = tb + tt;
      const float* tq = sbuf + (tt * NV + 0) * D;
      const float* tk = tq + D;
      const float* tv = tq + 2 * D;

      float kI[R];
      lds_rows<R>(tk + row0, kI);
      float y[R];
      bool last_fired = false;

      // ---- r guarded Sherman-Morrison sub-updates -------------------------
      for (int i = 0; i < r; ++i) {
        const float* tu = tq + (3 + i) * D;
        const bool last = (i == r - 1);
        float uJ[C];
        lds_cols<D, CG, C>(tu, cg, uJ);
        float z[R];
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) acc = fmaf(A[ii][c], uJ[c], acc);
          z[ii] = acc;
        }
        if (last) {
          float kJ[C];
          lds_cols<D, CG, C>(tk, cg, kJ);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) acc = fmaf(A[ii][c], kJ[c], acc);
            y[ii] = acc;
          }
        }
#pragma unroll
        for (int ii = 0; ii < R; ++ii) z[ii] = group_sum<CG>(z[ii]);
        if (last) {
#pragma unroll
          for (int ii = 0; ii < R; ++ii) y[ii] = group_sum<CG>(y[ii]);
        }
        float uI[R];
        lds_rows<R>(tu + row0, uI);
        float du = 0.f, dk = 0.f;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          du = fmaf(z[ii], uI[ii], du);
          dk = fmaf(z[ii], kI[ii], dk);
        }
        du = wave_sum(cg == 0 ? du : 0.f);
        dk = wave_sum(cg == 0 ? dk : 0.f);
        float* zb = zbuf + par * D;
        if (cg == 0) lds_store_rows<R>(zb + row0, z);
        if constexpr (NW > 1) {
          if (lane == 0) { red[(par * NW + w) * 4 + 0] = du; red[(par * NW + w) * 4 + 1] = dk; }
        }
        __syncthreads();
        if constexpr (NW > 1) {
          du = 0.f; dk = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) { du += red[(par * NW + ww) * 4 + 0]; dk += red[(par * NW + ww) * 4 + 1]; }
        }
        const float delta = 1.f + du;
        if (fabsf(delta) < a.eps) {
          // Singularity guard: inject eps*I and skip this rank-1 update.
          ++guard_fires;
#pragma unroll
          for (int ii = 0; ii < R; ++ii)
#pragma unroll
            for (int m = 0; m < C / 4; ++m)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row0 + ii == (m * CG + cg) * 4 + e) A[ii][4 * m + e] += a.eps;
          if (last) last_fired = true;
        } else {
          float zJ[C];
          lds_cols<D, CG, C>(zb, cg, zJ);
          const float inv = 1.f / delta;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            const float zs = z[ii] * inv;
#pragma unroll
            for (int c = 0; c < C; ++c) A[ii][c] = fmaf(-zs, zJ[c], A[ii][c]);
          }
          if (last) {
            const float g = dk * inv;
#pragma unroll
            for (int ii = 0; ii < R; ++ii) y[ii] = fmaf(-z[ii], g, y[ii]);
          }
        }
        par ^= 1;
      }

      // ---- nudge, coefficient and its clamp --------------------------------
      float alpha[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) alpha[ii] = last_fired ? fmaf(a.eps, kI[ii], y[ii]) : y[ii];
      if (a.nudge_period > 0) {
        if (phase == 0) {
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            alpha[ii] = fmaf(a.eps, kI[ii], alpha[ii]);
#pragma unroll
            for (int m = 0; m < C / 4; ++m)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row0 + ii == (m * CG + cg) * 4 + e) A[ii][4 * m + e] += a.eps;
          }
        }
        phase = (phase + 1 == a.nudge_period) ? 0 : phase + 1;
      }
      float an = 0.f;
#pragma unroll
      for (int ii = 0; ii < R; ++ii) an = fmaf(alpha[ii], alpha[ii], an);
      an = wave_sum(cg == 0 ? an : 0.f);
      float* ab = abuf + par * D;
      if (cg == 0) lds_store_rows<R>(ab + row0, alpha);
      if constexpr (NW > 1) {
        if (lane == 0) red[(par * NW + w) * 4 + 0] = an;
      }
      __syncthreads();
      if constexpr (NW > 1) {
        an = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) an += red[(par * NW + ww) * 4 + 0];
      }
      const float ascale = an > 1.f ? 1.f / sqrtf(an) : 1.f;
      float aJ[C];
      lds_cols<D, CG, C>(ab, cg, aJ);
      par ^= 1;

      // ---- state update, norm and readout ---------------------------------
      float vI[R], qI[R], qJ[C];
      lds_rows<R>(tv + row0, vI);
      lds_rows<R>(tq + row0, qI);
      lds_cols<D, CG, C>(tq, cg, qJ);
      float ns = 0.f, po[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) {
        const float vs = vI[ii] * ascale;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          S[ii][c] = fmaf(vs, aJ[c], S[ii][c]);
          ns = fmaf(S[ii][c], S[ii][c], ns);
          acc = fmaf(S[ii][c], qJ[c], acc);
        }
        po[ii] = acc;
      }
#pragma unroll
      for (int ii = 0; ii < R; ++ii) po[ii] = group_sum<CG>(po[ii]);
      float nq = 0.f;
#pragma unroll
      for (int ii = 0; ii < R; ++ii) {
        n[ii] += kI[ii];
        nq = fmaf(n[ii], qI[ii], nq);
      }
      ns = wave_sum(ns);
      nq = wave_sum(cg == 0 ? nq : 0.f);
      if constexpr (NW > 1) {
        if (lane == 0) { red[(par * NW + w) * 4 + 0] = ns; red[(par * NW + w) * 4 + 1] = nq; }
        __syncthreads();
        ns = 0.f; nq = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) { ns += red[(par * NW + ww) * 4 + 0]; nq += red[(par * NW + ww) * 4 + 1]; }
        par ^= 1;
      }
      float oscale = 1.f;
      if (a.cap_on && ns > cap2) {
        // Frobenius renormalisation: S <- S * cap / |S|_F.
        oscale = a.cap / sqrtf(ns);
#pragma unroll
        for (int ii = 0; ii < R; ++ii)
#pragma unroll
          for (int c = 0; c < C; ++c) S[ii][c] *= oscale;
        if (first_cap < 0) first_cap = t;
        ++cap_fires;
      }
      const float f = oscale / (nq + a.den_eps);
      if (cg == 0) {
        TIn* op = static_cast<TIn*>(a.o) + (chain * a.T + t) * D + row0;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          const float ov = po[ii] * f;
          bad |= !isfinite(ov);
          Elem<TIn>::store(op + ii, ov);
        }
      }
    }

    if (sidx + 1 < nstage) st.store(stage + ((sidx + 1) & 1) * TT * NV * D, TT, NV, tid);
    __syncthreads();
  }

  // ---- final state and statistics ---------------------------------------
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      const float4 av = make_float4(A[i][4 * m], A[i][4 * m + 1], A[i][4 * m + 2], A[i][4 * m + 3]);
      const float4 sv = make_float4(S[i][4 * m], S[i][4 * m + 1], S[i][4 * m + 2], S[i][4 * m + 3]);
      *reinterpret_cast<float4*>(a.A_T + (chain * D + row) * D + col) = av;
      *reinterpret_cast<float4*>(a.S_T + (chain * D + row) * D + col) = sv;
#pragma unroll
      for (int c = 0; c < 4; ++c) bad |= !isfinite(A[i][4 * m + c]) || !isfinite(S[i][4 * m + c]);
    }
    if (cg == 0) {
      a.n_T[chain * D + row] = n[i];
      bad |= !isfinite(n[i]);
    }
  }
  if (a.stats) {
    const bool wave_bad = __any(bad);
    if constexpr (NW > 1) {
      if (lane == 0) red[w * 4] = wave_bad ? 1.f : 0.f;
      __syncthreads();
    }
    if (tid == 0) {
      bool any_bad = wave_bad;
      if constexpr (NW > 1) {
        for (int ww = 0; ww < NW; ++ww) any_bad |= red[ww * 4] != 0.f;
      }
      int32_t* s = a.stats + chain * 4;
      s[0] = guard_fires;
      s[1] = cap_fires;
      s[2] = any_bad ? 1 : 0;
      s[3] = first_cap;
    }
  }
}

template <typename TIn, int D, int NW, int CG>
static size_t seq_lds_bytes(int r) {
  const int TT = stage_tokens<TIn, D, NW>(r);
  return sizeof(float) * (2 * TT * (3 + r) * D + 4 * D + 2 * NW * 4);
}

template <typename TIn, int D, int NW, int CG>
static hipError_t launch_seq(const ScanArgs& a, int chains, hipStream_t stream) {
  const size_t lds = seq_lds_bytes<TIn, D, NW, CG>(a.r);
  hipLaunchKernelGGL((vla_scan_seq_kernel<TIn, D, NW, CG>), dim3(chains), dim3(64 * NW), lds, stream, a);
  return hipGetLastError();
}

// Workgroup shape per head dimension: d <= 64 runs one wave per chain with
// quads of lanes sharing a row; d = 128 splits the rows over 4 waves.
template <typename TIn>
static hipError_t dispatch_seq(const ScanArgs& a, int d, int chains, hipStream_t stream) {
  switch (d) {
    case 16: return launch_seq<TIn, 16, 1, 4>(a, chains, stream);
    case 32: return launch_seq<TIn, 32, 1, 4>(a, chains, stream);
    case 64: return launch_seq<TIn, 64, 1, 4>(a, chains, stream);
    case 128: return launch_seq<TIn, 128, 4, 8>(a, chains, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_sequential(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream) {
  return bf16 ? dispatch_seq<uint16_t>(a, d, chains, stream) : dispatch_seq<float>(a, d, chains, stream);
}

}  // namespace vla
