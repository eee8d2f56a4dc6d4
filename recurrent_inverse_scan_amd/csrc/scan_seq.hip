// Sequential VLA scan kernels for gfx950 (CDNA4, wave64).
//
// One workgroup owns one (batch, head) chain for a run of tokens, starting
// from a given state and ending by writing the final state.  The tracked
// inverse A and the fast-weight state S stay in registers for the whole run;
// the per-token vectors stream through a double-buffered LDS stage.
//
// Method ("Mathematical Primitives", sections 2-5; "Variational Linear
// Attention (VLA)" README, v3 notes): per token, r guarded Sherman-Morrison
// rank-1 updates of A, the periodic eps*I nudge, alpha = A_t k_t clamped to
// norm <= 1, S += v alpha_hat^T, the Frobenius cap, n += k and the readout
// o = S q / (n.q + den_eps).
//
// The residual (delta-rule) update ("Variational Linear Attention: Stable
// Associative Memory for Long-Context Transformers", technical summary 2.3)
// is a variant of kFull (template flag RES): the gate is the unit vector
// along A_t k_hat with k_hat = k / |k|, and S += (v - S k_hat) alpha_hat^T,
// the prediction S_{t-1} k_hat taken before the update.  Since A_t k_hat is a
// multiple of A_t k, the gate comes from the same fused y = A k; the
// prediction is one more sweep of S per token.
//
// Three modes share this code:
//  * kFull: the whole recurrence (the sequential schedule at d = 128 and for
//    calls of at most 16 tokens, longer calls at d <= 64 running the
//    two-wave kernel of scan_split.hip; and the per-chain fallback of the
//    time-parallel schedule, gated by a per-chain flag);
//  * kInverseOnly: the inverse recurrence of one chunk of tokens, started
//    from the chunk-start inverse the time-parallel schedule computed, and
//    writing alpha_hat (one workgroup per chunk);
//  * kStateOnly: only the S/n recurrence, cap and readout, reading that
//    alpha_hat (one workgroup per chain).
//
// Register layout.  The NW waves of a workgroup split the d rows of A and S
// into slabs of RW = d/NW rows.  Inside a wave, lane = rg*CG + cg: the lane
// owns R = RW/(64/CG) consecutive rows and C = d/CG columns, the columns
// interleaved in float4 blocks, j = (m*CG + cg)*4 + e.  A row of a matrix
// vector product is split over the CG lanes of a row group and summed with
// DPP; the column-indexed vectors every lane needs (u, k, q, z, alpha) are
// read from LDS, conflict-free, as float4 blocks.
//
// Fusion: the first matrix-vector sweep of a token computes both z = A u_r
// and y = A k (same A), and alpha = A_t k follows as y - z (z.k)/delta (or
// y + eps k when the guard fires), so A is swept twice per rank-1 update
// (product and update) instead of three times.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_seq.h"
#include "vla_wave.h"

namespace vla {

// Scalars of the blocked rank-r update: u_i . w_l (4 x 4) and k . w_l (4).
constexpr int kBlkScalars = 20;

template <typename TIn, int D, int NW, int CG, SeqMode MODE, bool RES>
__global__ void __launch_bounds__(64 * NW)
vla_scan_seq_kernel(ScanArgs a, SeqExtra x) {
  static_assert(!RES || MODE == SeqMode::kFull, "the residual update runs in the full recurrence only");
  using L = TileLayout<D, NW, CG>;
  constexpr int R = L::R, C = L::C, RW = L::RW, NTH = L::kThreads;
  constexpr int kGroups = NW * 64 / CG;          // row groups of the workgroup
  constexpr int kBlkStride = kGroups + 4;         // LDS row of one blocked-update scalar
  constexpr bool kFull = MODE == SeqMode::kFull;
  constexpr bool kInv = MODE == SeqMode::kInverseOnly;
  constexpr bool kHasA = MODE != SeqMode::kStateOnly;   // runs the inverse recurrence
  constexpr bool kHasS = MODE != SeqMode::kInverseOnly; // runs the state recurrence
  extern __shared__ float4 smem4[];
  float* smem = reinterpret_cast<float*>(smem4);

  const int64_t chain = kInv ? blockIdx.x / x.chunk_cnt : blockIdx.x;
  const int chunk = kInv ? x.chunk_lo + static_cast<int>(blockIdx.x % x.chunk_cnt) : 0;
  if constexpr (kFull) {
    if (x.only_if && x.only_if[chain * 4 + kInfoFallback] == 0) return;   // uniform per workgroup
  }
  // Tokens [tbeg, tend) of the chain.  A fallback run (only_if) starts at the
  // chain's restart token, from the state the caller left for it in A0, S0
  // and n0.
  int tbeg = kInv ? chunk * x.chunk_len : 0;
  if constexpr (kFull) {
    if (x.only_if) tbeg = x.only_if[chain * 4 + kInfoRestart];
  }
  const int tend = kInv ? min(a.T, tbeg + x.chunk_len) : a.T;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int cg = lane % CG, rg = lane / CG;
  const int row0 = w * RW + rg * R;
  const int r = a.r;
  const int NV = seq_rows_per_token<TIn, D, NW>(MODE, r);
  const int TT = seq_stage_tokens<TIn, D, NW>(MODE, r);
  // Row of each stream inside a token's stage block.
  const int row_q = 0, row_v = 2;
  const int row_k = kInv ? 0 : 1;
  const int row_u = kInv ? 1 : 3;

  float* stage = smem;                                       // [2][TT][NV][D]
  float* astage = stage + 2 * TT * NV * D;                   // [2][TT][D]   (kStateOnly)
  float* zbuf = astage + (kHasA ? 0 : 2 * TT * D);           // [2][D]
  float* abuf = zbuf + 2 * D;                                // [2][D]
  float* red = abuf + 2 * D;                                 // [2][NW][4]
  float* zb4 = red + 2 * NW * 4;                             // [4][D] z rows of the blocked rank-r update
  float* scl = zb4 + 4 * D;                                  // [kBlkScalars][kBlkStride] row-group partials
  // Inverse-only pass on several waves: each stage's alpha rows [2][TT][D],
  // normalised and written out after the stage's closing barrier.
  float* apend = scl + kBlkScalars * kBlkStride;

  // ---- initial state --------------------------------------------------
  float A[kHasA ? R : 1][kHasA ? C : 4];
  float S[kHasS ? R : 1][kHasS ? C : 4], n[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      if constexpr (kHasA) {
        float4 av = make_float4(row == col ? 1.f : 0.f, row == col + 1 ? 1.f : 0.f,
                                row == col + 2 ? 1.f : 0.f, row == col + 3 ? 1.f : 0.f);
        if constexpr (kInv) {
          av = *reinterpret_cast<const float4*>(x.a_start + ((chain * x.nchunks + chunk) * D + row) * D + col);
        } else {
          if (a.A0) av = *reinterpret_cast<const float4*>(a.A0 + (chain * D + row) * D + col);
        }
        A[i][4 * m] = av.x; A[i][4 * m + 1] = av.y; A[i][4 * m + 2] = av.z; A[i][4 * m + 3] = av.w;
      }
      if constexpr (kHasS) {
        float4 sv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a.S0) sv = *reinterpret_cast<const float4*>(a.S0 + (chain * D + row) * D + col);
        S[i][4 * m] = sv.x; S[i][4 * m + 1] = sv.y; S[i][4 * m + 2] = sv.z; S[i][4 * m + 3] = sv.w;
      }
    }
    n[i] = (kHasS && a.n0) ? a.n0[chain * D + row] : 0.f;
  }

  int guard_fires = 0, cap_fires = 0, first_cap = -1;
  // The eps*I shifts (guard and nudge) are carried as a scalar: the tracked
  // inverse is A + shift*I, and the registers hold A.  Matrix-vector products
  // add shift*x, rank-1 updates apply to A unchanged, and the final store
  // folds shift into the diagonal.  The shifts then cost no register sweep.
  float shift = 0.f;
  bool bad = false;
  int par = 0;
  // (t0 + 1 + t) mod P for the current token t.
  int phase = a.nudge_period > 0 ? (a.nudge_phase0 + tbeg) % a.nudge_period : 0;
  const float cap2 = a.cap * a.cap;

  // Per-token rows in TIn (see row_*), and alpha_hat in fp32 for kStateOnly.
  const int64_t tok0 = chain * a.T;
  RowSource<TIn, D> src;
  src.n = NV;
  if constexpr (kHasS) {
    src.nfix = 3;
    src.fix0 = static_cast<const TIn*>(a.q) + tok0 * D;
    src.fix1 = static_cast<const TIn*>(a.k) + tok0 * D;
    src.fix2 = static_cast<const TIn*>(a.v) + tok0 * D;
  } else {
    src.nfix = 1;
    src.fix0 = static_cast<const TIn*>(a.k) + tok0 * D;
    src.fix1 = src.fix2 = src.fix0;
  }
  src.ubase = kHasA ? static_cast<const TIn*>(a.u) + tok0 * r * D : src.fix0;
  src.ustride = static_cast<int64_t>(r) * D;
  RowSource<float, D> asrc;
  asrc.n = 1;
  asrc.nfix = 1;
  asrc.fix0 = asrc.fix1 = asrc.fix2 = asrc.ubase = kHasA ? nullptr : x.alpha + tok0 * D;
  asrc.ustride = D;

  Stager<TIn, D, NTH, seq_stage_slots<TIn, D, NW>(MODE)> st;
  Stager<float, D, NTH, (kHasA ? 1 : kMaxStageVecs)> ast;
  const int nstage = (tend - tbeg + TT - 1) / TT;
  if (nstage > 0) {
    st.load(src, tbeg, TT, tend, tid);
    st.store(stage, TT, NV, tid);
    if constexpr (!kHasA) {
      ast.load(asrc, tbeg, TT, tend, tid);
      ast.store(astage, TT, 1, tid);
    }
  }
  __syncthreads();

  for (int sidx = 0; sidx < nstage; ++sidx) {
    const int tb = tbeg + sidx * TT;
    if (sidx + 1 < nstage) {
      st.load(src, tb + TT, TT, tend, tid);
      if constexpr (!kHasA) ast.load(asrc, tb + TT, TT, tend, tid);
    }
    const float* sbuf = stage + (sidx & 1) * TT * NV * D;
    const int tcount = min(TT, tend - tb);

    for (int tt = 0; tt < tcount; ++tt) {
      const int t = tb + tt;
      const float* tblk = sbuf + tt * NV * D;
      const float* tq = tblk + row_q * D;
      const float* tk = tblk + row_k * D;
      const float* tv = tblk + row_v * D;

      float kI[R];
      lds_rows<R>(tk + row0, kI);
      float aJ[C];
      // Residual update: 1/|k| and the prediction S_{t-1} k (rows of this lane).
      float kinv = 1.f, pred[RES ? R : 1];
      if constexpr (RES) {
        float kJ[C];
        lds_cols<CG, C>(tk, cg, kJ);
        float kn = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) kn = fmaf(kJ[c], kJ[c], kn);
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) acc = fmaf(S[ii][c], kJ[c], acc);
          pred[ii] = acc;
        }
        kn = group_sum<CG>(kn);
#pragma unroll
        for (int ii = 0; ii < R; ++ii) pred[ii] = group_sum<CG>(pred[ii]);
        kinv = 1.f / fmaxf(sqrtf(kn), 1e-12f);
      }

      if constexpr (kHasA) {
        float y[R];
        bool last_fired = false;

        // ---- r > 1: the r sub-updates in one sweep and one rank-r update ----
        // With w_l = A u_l (A before the token), the sequential steps satisfy
        // z_i = w_i - sum_{j<i} z_j (z_j . u_i) / delta_j: each z_i is a
        // combination of the w_l, so every z_j . u_i, z_i . k and delta_i
        // follow from the products u_i . w_l and k . w_l by the same
        // recurrence.  A then takes the whole update A - sum_i z_i z_i^T / delta_i
        // and A_t k = A k - sum_i z_i (z_i . k) / delta_i.  One chain-wide
        // reduction and one broadcast replace r of each.  Should any delta
        // trip the guard, the token runs the sub-updates one by one instead
        // (A is untouched until then).
        bool blocked = false;
        if (r > 1) {
          float wl[4][R], wk[R];
          float kJ[C];
          lds_cols<CG, C>(tk, cg, kJ);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) acc = fmaf(A[ii][c], kJ[c], acc);
            wk[ii] = fmaf(shift, kI[ii], group_sum<CG>(acc));
          }
#pragma unroll
          for (int l = 0; l < 4; ++l) {
            if (l < r) {
              float uJ[C], uR[R];
              lds_cols<CG, C>(tblk + (row_u + l) * D, cg, uJ);
              lds_rows<R>(tblk + (row_u + l) * D + row0, uR);
#pragma unroll
              for (int ii = 0; ii < R; ++ii) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) acc = fmaf(A[ii][c], uJ[c], acc);
                wl[l][ii] = fmaf(shift, uR[ii], group_sum<CG>(acc));
              }
            } else {
#pragma unroll
              for (int ii = 0; ii < R; ++ii) wl[l][ii] = 0.f;
            }
          }
          // Scalars: sc[4 i + l] = u_i . w_l (i, l < r) and sc[16 + l] = k . w_l.
          // Each row group's leader writes its partials to LDS, lane e of every
          // wave sums scalar e over the row groups, and readlane broadcasts.
          float sc[kBlkScalars];
          if (cg == 0) {
            float* dst = scl + w * (64 / CG) + rg;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float uI[R];
              if (i < r) lds_rows<R>(tblk + (row_u + i) * D + row0, uI);
#pragma unroll
              for (int l = 0; l < 4; ++l) {
                float acc = 0.f;
                if (i < r && l < r) {
#pragma unroll
                  for (int ii = 0; ii < R; ++ii) acc = fmaf(uI[ii], wl[l][ii], acc);
                }
                dst[(4 * i + l) * kBlkStride] = acc;
              }
            }
#pragma unroll
            for (int l = 0; l < 4; ++l) {
              float acc = 0.f;
#pragma unroll
              for (int ii = 0; ii < R; ++ii) acc = fmaf(kI[ii], wl[l][ii], acc);
              dst[(16 + l) * kBlkStride] = acc;
            }
          }
          __syncthreads();
          {
            float t = 0.f;
            if (lane < kBlkScalars) {
              const float4* src4 = reinterpret_cast<const float4*>(scl + lane * kBlkStride);
              float4 acc4 = src4[0];
#pragma unroll
              for (int g = 1; g < kGroups / 4; ++g) {
                const float4 v4 = src4[g];
                acc4.x += v4.x; acc4.y += v4.y; acc4.z += v4.z; acc4.w += v4.w;
              }
              t = (acc4.x + acc4.y) + (acc4.z + acc4.w);
            }
#pragma unroll
            for (int e = 0; e < kBlkScalars; ++e)
              sc[e] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), e));
          }
          // The recurrence, in place: row i of wl becomes z_i, and the scalars
          // follow it (sc[4 m + i] = u_m . z_i, sc[16 + i] = k . z_i).
          float dl[4], dinv[4];
          bool fire = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dl[i] = 1.f;
            dinv[i] = 1.f;
            if (i < r) {
#pragma unroll
              for (int j = 0; j < i; ++j) {
                const float f = sc[4 * i + j] * dinv[j];   // (z_j . u_i) / delta_j
#pragma unroll
                for (int ii = 0; ii < R; ++ii) wl[i][ii] = fmaf(-f, wl[j][ii], wl[i][ii]);
#pragma unroll
                for (int m = 0; m < 4; ++m) sc[4 * m + i] = fmaf(-f, sc[4 * m + j], sc[4 * m + i]);
                sc[16 + i] = fmaf(-f, sc[16 + j], sc[16 + i]);
              }
              dl[i] = 1.f + sc[4 * i + i];
              dinv[i] = 1.f / dl[i];
              fire |= fabsf(dl[i]) < a.eps;
            }
          }
          if (!fire) {
            blocked = true;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < r && cg == 0) lds_store_rows<R>(zb4 + i * D + row0, wl[i]);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (i < r) {
                float zJ[C];
                lds_cols<CG, C>(zb4 + i * D, cg, zJ);
                const float inv = dinv[i];
#pragma unroll
                for (int ii = 0; ii < R; ++ii) {
                  const float zs = wl[i][ii] * inv;
#pragma unroll
                  for (int c = 0; c < C; ++c) A[ii][c] = fmaf(-zs, zJ[c], A[ii][c]);
                }
              }
            }
#pragma unroll
            for (int ii = 0; ii < R; ++ii) {
              float yy = wk[ii];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (i < r) yy = fmaf(-wl[i][ii], sc[16 + i] * dinv[i], yy);
              y[ii] = yy;
            }
          }
        }

        // ---- r guarded Sherman-Morrison sub-updates -----------------------
        for (int i = 0; i < (blocked ? 0 : r); ++i) {
          const float* tu = tblk + (row_u + i) * D;
          const bool last = (i == r - 1);
          float uJ[C];
          lds_cols<CG, C>(tu, cg, uJ);
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
            lds_cols<CG, C>(tk, cg, kJ);
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
            for (int ii = 0; ii < R; ++ii) y[ii] = fmaf(shift, kI[ii], group_sum<CG>(y[ii]));
          }
          float uI[R];
          lds_rows<R>(tu + row0, uI);
#pragma unroll
          for (int ii = 0; ii < R; ++ii) z[ii] = fmaf(shift, uI[ii], z[ii]);
          float du = 0.f, dk = 0.f;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            du = fmaf(z[ii], uI[ii], du);
            dk = fmaf(z[ii], kI[ii], dk);
          }
          du = wave_total(cg == 0 ? du : 0.f);
          if (last) dk = wave_total(cg == 0 ? dk : 0.f);
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
          const bool fire = fabsf(delta) < a.eps;
          if (fire) {
            // Singularity guard: inject eps*I and skip this rank-1 update.
            ++guard_fires;
            shift += a.eps;
            if (last) last_fired = true;
          }
          // The update runs either way, with a zero coefficient when the guard
          // fired: A then stays in the same registers on both paths.
          const float inv = fire ? 0.f : 1.f / delta;
          {
            float zJ[C];
            lds_cols<CG, C>(zb, cg, zJ);
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

        // ---- nudge, coefficient and its clamp ------------------------------
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
        if constexpr (kInv && NW > 1) {
          // The norm needs every wave's rows: the rows wait in LDS until the
          // stage ends (below), so no barrier is spent on it here.
          if (cg == 0) lds_store_rows<R>(apend + ((sidx & 1) * TT + tt) * D + row0, alpha);
          continue;
        }
        if constexpr (kInv) {
          float an = 0.f, kn = 0.f;
#pragma unroll
          for (int ii = 0; ii < R; ++ii) {
            an = fmaf(alpha[ii], alpha[ii], an);
            kn = fmaf(kI[ii], kI[ii], kn);
          }
          an = wave_total(cg == 0 ? an : 0.f);
          if (a.residual) kn = wave_total(cg == 0 ? kn : 0.f);
          // alpha_hat of this token goes to HBM for the state pass: the
          // clamped coefficient, or for the residual update the unit vector
          // along A k_hat with k_hat = k / |k|.
          float ascale = an > 1.f ? 1.f / sqrtf(an) : 1.f;
          if (a.residual) {
            const float kinv = 1.f / fmaxf(sqrtf(kn), 1e-12f);
            ascale = kinv / fmaxf(kinv * sqrtf(an), 1e-12f);
          }
          if (cg == 0) {
            float ah[R];
#pragma unroll
            for (int ii = 0; ii < R; ++ii) {
              ah[ii] = alpha[ii] * ascale;
              bad |= !isfinite(ah[ii]);
            }
            float* dst = x.alpha_out + (tok0 + t) * D + row0;
            if constexpr (R % 4 == 0) {
#pragma unroll
              for (int ii = 0; ii < R; ii += 4)
                *reinterpret_cast<float4*>(dst + ii) = make_float4(ah[ii], ah[ii + 1], ah[ii + 2], ah[ii + 3]);
            } else {
#pragma unroll
              for (int ii = 0; ii < R; ++ii) dst[ii] = ah[ii];
            }
          }
          continue;
        }
        float* ab = abuf + par * D;
        if (cg == 0) lds_store_rows<R>(ab + row0, alpha);
        __syncthreads();
        // |alpha|^2 from the columns: a row group's lanes hold every column,
        // so a group sum replaces the reduction over the workgroup.
        lds_cols<CG, C>(ab, cg, aJ);
        float an = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) an = fmaf(aJ[c], aJ[c], an);
        an = group_sum<CG>(an);
        // Additive: alpha / max(|alpha|, 1).  Residual: the unit vector along
        // A k_hat = kinv * A k, i.e. kinv / max(kinv |A k|, 1e-12) times A k.
        const float ascale = RES ? kinv / fmaxf(kinv * sqrtf(an), 1e-12f) : (an > 1.f ? 1.f / sqrtf(an) : 1.f);
#pragma unroll
        for (int c = 0; c < C; ++c) aJ[c] *= ascale;
        par ^= 1;
      } else {
        // alpha_hat of this token, precomputed by the inverse pass.
        lds_cols<CG, C>(astage + ((sidx & 1) * TT + tt) * D, cg, aJ);
      }

      // ---- state update, norm and readout ---------------------------------
      if constexpr (kHasS) {
      float vI[R], qI[R], qJ[C];
      lds_rows<R>(tv + row0, vI);
      if constexpr (RES) {
#pragma unroll
        for (int ii = 0; ii < R; ++ii) vI[ii] = fmaf(-pred[ii], kinv, vI[ii]);   // v - S_{t-1} k_hat
      }
      lds_rows<R>(tq + row0, qI);
      lds_cols<CG, C>(tq, cg, qJ);
      float ns = 0.f, po[R];
#pragma unroll
      for (int ii = 0; ii < R; ++ii) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          S[ii][c] = fmaf(vI[ii], aJ[c], S[ii][c]);
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
      ns = wave_total(ns);
      nq = wave_total(cg == 0 ? nq : 0.f);
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
        TIn* op = static_cast<TIn*>(a.o) + (tok0 + t) * D + row0;
#pragma unroll
        for (int ii = 0; ii < R; ++ii) {
          const float ov = po[ii] * f;
          bad |= !isfinite(ov);
          Elem<TIn>::store(op + ii, ov);
        }
      }
      }  // kHasS
    }

    if (sidx + 1 < nstage) {
      st.store(stage + ((sidx + 1) & 1) * TT * NV * D, TT, NV, tid);
      if constexpr (!kHasA) ast.store(astage + ((sidx + 1) & 1) * TT * D, TT, 1, tid);
    }
    __syncthreads();
    if constexpr (kInv && NW > 1) {
      // alpha_hat of the stage's tokens, wave w taking tokens w, w + NW, ...:
      // the clamped coefficient, or for the residual update the unit vector
      // along A k_hat with k_hat = k / |k|.  The rows and this stage's k stay
      // in place until the next stage's first barrier (the buffers alternate
      // by stage), which every wave reaches only after these reads.
      constexpr int PL = D / 64;   // values per lane
      for (int tt = w; tt < tcount; tt += NW) {
        const float* arow = apend + ((sidx & 1) * TT + tt) * D + PL * lane;
        const float* krow = sbuf + (tt * NV + row_k) * D + PL * lane;
        float av[PL], an = 0.f, kn = 0.f;
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          av[e] = arow[e];
          an = fmaf(av[e], av[e], an);
          kn = fmaf(krow[e], krow[e], kn);
        }
        an = wave_sum(an);
        float ascale = an > 1.f ? 1.f / sqrtf(an) : 1.f;
        if (a.residual) {
          const float kinv = 1.f / fmaxf(sqrtf(wave_sum(kn)), 1e-12f);
          ascale = kinv / fmaxf(kinv * sqrtf(an), 1e-12f);
        }
        float* dst = x.alpha_out + (tok0 + tb + tt) * D + PL * lane;
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          const float ah = av[e] * ascale;
          bad |= !isfinite(ah);
          dst[e] = ah;
        }
      }
    }
  }

  // ---- final state and statistics ---------------------------------------
  const bool write_a = kFull || (kInv && chunk == x.nchunks - 1);
  if constexpr (kHasA) add_to_diagonal<R, C, CG>(A, row0, cg, shift);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int m = 0; m < C / 4; ++m) {
      const int col = (m * CG + cg) * 4;
      if constexpr (kHasA) {
        if (write_a) {
          const float4 av = make_float4(A[i][4 * m], A[i][4 * m + 1], A[i][4 * m + 2], A[i][4 * m + 3]);
          *reinterpret_cast<float4*>(a.A_T + (chain * D + row) * D + col) = av;
#pragma unroll
          for (int c = 0; c < 4; ++c) bad |= !isfinite(A[i][4 * m + c]);
        }
      }
      if constexpr (kHasS) {
        const float4 sv = make_float4(S[i][4 * m], S[i][4 * m + 1], S[i][4 * m + 2], S[i][4 * m + 3]);
        *reinterpret_cast<float4*>(a.S_T + (chain * D + row) * D + col) = sv;
#pragma unroll
        for (int c = 0; c < 4; ++c) bad |= !isfinite(S[i][4 * m + c]);
      }
    }
    if constexpr (kHasS) {
      if (cg == 0) {
        a.n_T[chain * D + row] = n[i];
        bad |= !isfinite(n[i]);
      }
    }
  }
  if constexpr (kInv) {
    // Guard fires break the chunk-start inverses of later chunks: flag the
    // chain for the sequential fallback.  Non-finite values are recorded.
    // (Guard fires are the same in every wave; a non-finite value may show
    // in any wave's rows.)
    const bool wave_bad = __any(bad);
    int32_t* info = x.chain_info + chain * 4;
    if (tid == 0 && guard_fires > 0) {
      atomicAdd(info + kInfoGuard, guard_fires);
      atomicOr(info + kInfoFallback, 1);
    }
    if (lane == 0 && wave_bad) atomicOr(info + kInfoNonfinite, 1);
    return;
  }
  if (a.stats) {
    const bool wave_bad = __any(bad);
    __syncthreads();
    if (lane == 0) red[w * 4] = wave_bad ? 1.f : 0.f;
    __syncthreads();
    if (tid == 0) {
      bool any_bad = false;
      for (int ww = 0; ww < NW; ++ww) any_bad |= red[ww * 4] != 0.f;
      int32_t guards = guard_fires;
      // A chain restarted past token 0 keeps the earlier outputs of the
      // chunked passes (no guard fired and no cap applied there).
      if (kFull && x.only_if && tbeg > 0) any_bad |= x.only_if[chain * 4 + kInfoNonfinite] != 0;
      if constexpr (!kFull) {
        guards = x.chain_info ? x.chain_info[chain * 4 + 0] : 0;
        any_bad |= x.chain_info && x.chain_info[chain * 4 + 2] != 0;
      }
      int32_t* s = a.stats + chain * 4;
      s[0] = guards;
      s[1] = cap_fires;
      s[2] = any_bad ? 1 : 0;
      s[3] = first_cap;
    }
  }
}

template <typename TIn, int D, int NW, int CG, SeqMode MODE>
static hipError_t launch_seq(const ScanArgs& a, const SeqExtra& x, int chains, hipStream_t stream) {
  // The stages and vectors, then the blocked rank-r update's z rows and scalars.
  const size_t lds =
      seq_lds_bytes<TIn, D, NW>(MODE, a.r) + sizeof(float) * (4 * D + kBlkScalars * (NW * 64 / CG + 4)) +
      (MODE == SeqMode::kInverseOnly && NW > 1 ? sizeof(float) * 2 * seq_stage_tokens<TIn, D, NW>(MODE, a.r) * D : 0);
  const unsigned grid = MODE == SeqMode::kInverseOnly ? static_cast<unsigned>(chains * x.chunk_cnt)
                                                       : static_cast<unsigned>(chains);
  if constexpr (MODE == SeqMode::kFull) {
    if (a.residual) {
      hipLaunchKernelGGL((vla_scan_seq_kernel<TIn, D, NW, CG, MODE, true>), dim3(grid), dim3(64 * NW), lds,
                         stream, a, x);
      return hipGetLastError();
    }
  } else if constexpr (MODE == SeqMode::kStateOnly) {
    if (a.residual) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((vla_scan_seq_kernel<TIn, D, NW, CG, MODE, false>), dim3(grid), dim3(64 * NW), lds, stream,
                     a, x);
  return hipGetLastError();
}

// Workgroup shapes.  The full scan runs one wave per chain for d <= 64 (many
// chains fill the chip) and eight waves at d = 128 (two rows per lane; four
// waves took 8 % longer on 128 chains of 8192 tokens); short calls see below.  The state-only chain of
// the time-parallel schedule has few chains and spreads each one over a
// whole compute unit.
// Below this many tokens per call (decode-like calls, where the state's trip
// through HBM dominates) the full scan spreads a chain over more waves, so
// each wave holds fewer rows of A and S and more waves share a SIMD, which
// overlaps one chain's state loads with another's arithmetic.
constexpr int kShortCallTokens = 16;

template <typename TIn, SeqMode MODE>
static hipError_t dispatch_seq(const ScanArgs& a, const SeqExtra& x, int d, int chains, hipStream_t stream) {
  if constexpr (MODE == SeqMode::kFull) {
    if (a.T <= kShortCallTokens) {
      switch (d) {
        case 32: return launch_seq<TIn, 32, 2, 4, MODE>(a, x, chains, stream);
        case 64: return launch_seq<TIn, 64, 4, 4, MODE>(a, x, chains, stream);
        default: break;
      }
    }
    switch (d) {
      case 16: return launch_seq<TIn, 16, 1, 4, MODE>(a, x, chains, stream);
      case 32: return launch_seq<TIn, 32, 1, 4, MODE>(a, x, chains, stream);
      case 64: return launch_seq<TIn, 64, 1, 4, MODE>(a, x, chains, stream);
      case 128: return launch_seq<TIn, 128, 8, 8, MODE>(a, x, chains, stream);
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (MODE == SeqMode::kStateOnly) {
    switch (d) {
      case 64: return launch_seq<TIn, 64, 4, 4, MODE>(a, x, chains, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (d) {
      case 64: return launch_seq<TIn, 64, 1, 4, MODE>(a, x, chains, stream);
      default: return hipErrorInvalidValue;   // d = 128 runs the blocked pass (inverse_wy128.hip)
    }
  }
}

// One-token calls at d = 64 (decode.hip).
hipError_t launch_decode(const ScanArgs& a, bool bf16, int chains, hipStream_t stream);
hipError_t launch_scan_split(const ScanArgs& a, int d, bool bf16, int chains, hipStream_t stream);

hipError_t launch_scan_sequential(const ScanArgs& a, int d, bool bf16, int chains, const int32_t* only_if,
                                  hipStream_t stream) {
  if (a.T == 1 && d == 64 && only_if == nullptr) return launch_decode(a, bf16, chains, stream);
  // Longer runs at d <= 64: the inverse and state recurrences on two waves.
  if (a.T > kShortCallTokens && d <= 64 && only_if == nullptr) return launch_scan_split(a, d, bf16, chains, stream);
  SeqExtra x{};
  x.only_if = only_if;
  return bf16 ? dispatch_seq<uint16_t, SeqMode::kFull>(a, x, d, chains, stream)
              : dispatch_seq<float, SeqMode::kFull>(a, x, d, chains, stream);
}

hipError_t launch_scan_inverse_chunks(const ScanArgs& a, const float* a_start, float* alpha_out,
                                     int32_t* chain_info, int chunk_len, int nchunks, int chunk_lo, int chunk_cnt,
                                     int d, bool bf16, int chains, hipStream_t stream) {
  if (chunk_cnt <= 0) return hipSuccess;
  SeqExtra x{};
  x.a_start = a_start;
  x.alpha_out = alpha_out;
  x.chain_info = chain_info;
  x.chunk_len = chunk_len;
  x.nchunks = nchunks;
  x.chunk_lo = chunk_lo;
  x.chunk_cnt = chunk_cnt;
  return bf16 ? dispatch_seq<uint16_t, SeqMode::kInverseOnly>(a, x, d, chains, stream)
              : dispatch_seq<float, SeqMode::kInverseOnly>(a, x, d, chains, stream);
}

}  // namespace vla
