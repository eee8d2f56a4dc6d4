// Inverse pass of the time-parallel schedule in blocked form (d = 64, one
// direction per token, bf16 or fp32 storage), on the gfx950 matrix cores.
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
// k enter exactly: as they are with bf16 storage, as three-term splits (which
// represent an fp32 value exactly) with fp32 storage.  The LDL^T elimination of I + C, carried along on E =
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

// This lane's index, recomputed where it is used (volatile: the compiler may
// not keep one copy live across the block loop, where it would spill).
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

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

// The eight fp32 values of a 16-feature operand fragment (two 16-byte
// pieces) as a three-term split.
__device__ __forceinline__ Split3 split_pieces(const float4& a, const float4& b) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return split3(v);
}

// F32: u and k stored as fp32 (else bf16).
template <bool UNIT_GATE, bool F32>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
vla_inverse_wy_kernel(const void* __restrict__ kx, const void* __restrict__ ux,
                      const float* __restrict__ a_start, float* __restrict__ alpha_out, float* __restrict__ A_T,
                      int32_t* __restrict__ chain_info, int T, int L, int nchunks, int chunk_lo, int chunk_cnt,
                      float eps, int nudge_period, int nudge_phase0) {
  __shared__ float4 sColQ[2][16];    // pivot columns k .. k + 3 of I + C: [lane half][slot], component = column
  __shared__ float4 sRowQ[kM][3];    // pivot rows k .. k + 3 of (I + C, E, T) at column t
  __shared__ __align__(16) float sDinv[kM];     // 1 / pivot
  constexpr int kEB = F32 ? 4 : 2;        // bytes per stored element
  constexpr int kPieces = F32 ? 2 : 1;    // 16-byte pieces per lane and k step
  __shared__ float4 sTok[2][4][kPieces][kD];   // the block's u and k operands: [u / k][k step][piece][lane]
  __shared__ float sKn[F32 && UNIT_GATE ? kD : 1];   // per lane: its half of |k|^2 (fp32 storage)

  const int64_t chain = blockIdx.x / chunk_cnt;
  const int chunk = chunk_lo + static_cast<int>(blockIdx.x % chunk_cnt);
  const int tbeg = chunk * L, tend = min(T, tbeg + L);
  const int lane0 = threadIdx.x, c0 = lane0 & 31, h0 = lane0 >> 5;   // (before the block loop only)

  // ---- A_b: tile (F, I) slot s = A[feat(32F + acc_row(s, h))][feat(32I + c)].
  // Slot s = 4 q + e sits at row 32F + 16 (q >> 1) + 8 h + 4 (q & 1) + e: a
  // per-lane byte offset plus a constant one, passed as the buffer access's
  // scalar offset so no per-element address stays live.
  const int a_voff0 = (8 * h0 * kD + feat(c0)) * 4;
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
          Acc[F][I][s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, a_voff0, a_soff(F, I, s), 0));
  }

  // Token rows go from HBM straight into LDS (buffer-to-LDS copies, no
  // registers held while they fly): lane (c, h) takes features 16 kappa +
  // 8 h .. + 7 of token c of the block for k step kappa (fp32: in two
  // 16-byte pieces).  The buffers end at
  // the chunk's last token, so rows past it read as zero.
  // Both buffers start at the chunk's first token, so their extents and
  // offsets stay below one chunk (at most 512 tokens) whatever T is.
  const int64_t row0 = chain * T + tbeg;
  const auto ru = make_rsrc(static_cast<const char*>(ux) + row0 * kD * kEB, (tend - tbeg) * kD * kEB);
  const auto rk = make_rsrc(static_cast<const char*>(kx) + row0 * kD * kEB, (tend - tbeg) * kD * kEB);
  auto copy_tokens = [&](int tb) {
    const int ln = fresh_lane();
    const int vo = ((tb - tbeg + (ln & 31)) * kD + 8 * (ln >> 5)) * kEB;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp)
#pragma unroll
      for (int pc = 0; pc < kPieces; ++pc) {
        const int off = vo + 16 * kEB * kp + 16 * pc;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void*)&sTok[0][kp][pc][0], 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)&sTok[1][kp][pc][0], 16, off, 0, 0, 0);
      }
  };

  const bool nudge_last = nudge_period > 0 && tend > tbeg && (nudge_phase0 + tend - 1) % nudge_period == 0;
  int guard = 0;
  bool bad = false;
  copy_tokens(tbeg);

  for (int tb = tbeg; tb < tend; tb += kM) {
    // Lane indices laundered per block: values derived from them are then
    // recomputed in each block instead of being hoisted and kept live.
    const int ln = fresh_lane();
    int c = ln & 31, h = ln >> 5;
    asm volatile("" : "+v"(c), "+v"(h));
    const int lane = c + 32 * h;
    // This wave's copies of the block's rows have landed (the compiler does
    // not order LDS reads after buffer-to-LDS copies by itself).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // bf16: the operands stay in registers for the block.  fp32: they are
    // split from LDS where they are used (the next block's copy starts only
    // after the last such use; the last block's rows stay for the nudge).
    uint4 uf[4], kf[4];
    if constexpr (!F32) {
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        const float4 a = sTok[0][kp][0][lane], b = sTok[1][kp][0][lane];
        uf[kp] = make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
        kf[kp] = make_uint4(__float_as_uint(b.x), __float_as_uint(b.y), __float_as_uint(b.z), __float_as_uint(b.w));
      }
    } else if constexpr (UNIT_GATE) {
      // The gate's |k|^2 before the rows are overwritten, kept in LDS.
      float kn = 0.f;
#pragma unroll
      for (int kp = 0; kp < 4; ++kp)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const float4 b = sTok[1][kp][pc][lane];
          kn = fmaf(b.x, b.x, kn); kn = fmaf(b.y, b.y, kn); kn = fmaf(b.z, b.z, kn); kn = fmaf(b.w, b.w, kn);
        }
      sKn[lane] = kn;
    }
    auto u_op = [&](int kp) {
      if constexpr (F32)
        return split_pieces(sTok[0][kp][0][lane], sTok[0][kp][1][lane]);
      else
        return __builtin_bit_cast(bf16x8, uf[kp]);
    };
    auto k_op = [&](int kp) {
      if constexpr (F32)
        return split_pieces(sTok[1][kp][0][lane], sTok[1][kp][1][lane]);
      else
        return __builtin_bit_cast(bf16x8, kf[kp]);
    };
    // ---- X_U = A U, X_K = A K (rows: basis features, columns: tokens) and
    // X_U^T (rows: tokens, columns: basis features).
    f32x16 XU[2] = {zero16(), zero16()}, XK[2] = {zero16(), zero16()}, XUT[2] = {zero16(), zero16()};
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int kp = 2 * F + g;
        const auto ub = u_op(kp), kb = k_op(kp);
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
        const auto ub = u_op(2 * I + g);
        Cm = mma_split(ub, split_slots(XU[I], g), Cm);
        Em = mma_split(ub, split_slots(XK[I], g), Em);
        sched_fence();
      }

    // The next block's rows start their copy (this block's stay in
    // registers; the last block keeps them for the nudge).
    if (tb + kM < tend) {
      lds_order();
      // fp32: this block's row reads have returned before the rows are overwritten.
      if constexpr (F32) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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
    // Four pivots per LDS round trip, k = 4 j: the Schur complement of the
    // pivot block P = S[K][K], K = k .. k + 3, S the current I + C.  With
    // P = L_P U_P (unit lower L_P; U_P's diagonal holds the four pivots),
    // column c of each of S, E and T (X below) becomes, for rows i past K,
    //   X[i][c] - S[i][K] w,   w = P^{-1} X[K][c],
    // and, in the rows of K, y = L_P^{-1} X[K][c] (what the one-at-a-time
    // elimination leaves there).  Lanes k .. k + 3 hold the columns S[.][K]
    // and publish them slot by slot; the rows X[K][c] sit in slots
    // 4 (k >> 3) .. + 3 of lane half (k >> 2) & 1.  Reading the columns a
    // slot at a time keeps them out of registers.
#pragma unroll
    for (int k = 0; k < kM; k += 4) {
      const int hk = (k >> 2) & 1, sq = 4 * (k >> 3);
      lds_order();   // the previous block of pivots has read the buffers
      if (c >= k && c < k + 4) {
        float* col = reinterpret_cast<float*>(&sColQ[h][0]) + (c - k);
#pragma unroll
        for (int s = 0; s < 16; ++s) col[4 * s] = cm[s];
      }
      if (h == hk) {
        sRowQ[c][0] = make_float4(cm[sq], cm[sq + 1], cm[sq + 2], cm[sq + 3]);
        sRowQ[c][1] = make_float4(em[sq], em[sq + 1], em[sq + 2], em[sq + 3]);
        sRowQ[c][2] = make_float4(tm[sq], tm[sq + 1], tm[sq + 2], tm[sq + 3]);
      }
      lds_order();
      // P[a][b] = S[k + a][k + b]: slot sq + a of half hk, component b.
      float P[4][4];
#pragma unroll
      for (int a2 = 0; a2 < 4; ++a2) {
        const float4 v = sColQ[hk][sq + a2];
        P[a2][0] = v.x; P[a2][1] = v.y; P[a2][2] = v.z; P[a2][3] = v.w;
      }
      auto rcp = [](float x) {
        float r = __builtin_amdgcn_rcpf(x);
        return fmaf(fmaf(-x, r, 1.f), r, r);
      };
      // P = L_P U_P, column by column.
      const float i0 = rcp(P[0][0]);
      const float l10 = P[1][0] * i0, l20 = P[2][0] * i0, l30 = P[3][0] * i0;
      const float p11 = fmaf(-l10, P[0][1], P[1][1]), p12 = fmaf(-l10, P[0][2], P[1][2]),
                  p13 = fmaf(-l10, P[0][3], P[1][3]);
      const float p21 = fmaf(-l20, P[0][1], P[2][1]), p22 = fmaf(-l20, P[0][2], P[2][2]),
                  p23 = fmaf(-l20, P[0][3], P[2][3]);
      const float p31 = fmaf(-l30, P[0][1], P[3][1]), p32 = fmaf(-l30, P[0][2], P[3][2]),
                  p33 = fmaf(-l30, P[0][3], P[3][3]);
      const float i1 = rcp(p11);
      const float l21 = p21 * i1, l31 = p31 * i1;
      const float q22 = fmaf(-l21, p12, p22), q23 = fmaf(-l21, p13, p23);
      const float q32 = fmaf(-l31, p12, p32), q33 = fmaf(-l31, p13, p33);
      const float i2 = rcp(q22);
      const float l32 = q32 * i2;
      const float u33 = fmaf(-l32, q23, q33);
      const float i3 = rcp(u33);
      guard += (fabsf(P[0][0]) < eps ? 1 : 0) + (fabsf(p11) < eps ? 1 : 0) + (fabsf(q22) < eps ? 1 : 0) +
               (fabsf(u33) < eps ? 1 : 0);
      asm volatile("" : "+v"(guard));
      if (lane == 0) *reinterpret_cast<float4*>(sDinv + k) = make_float4(i0, i1, i2, i3);
      // y = L_P^{-1} X[K][c], w = U_P^{-1} y, for X = S, E, T.
      float ys[3][4], ws[3][4];
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const float4 rv = sRowQ[c][m];
        const float y0 = rv.x;
        const float y1 = fmaf(-l10, y0, rv.y);
        const float y2 = fmaf(-l21, y1, fmaf(-l20, y0, rv.z));
        const float y3 = fmaf(-l32, y2, fmaf(-l31, y1, fmaf(-l30, y0, rv.w)));
        const float w3 = y3 * i3;
        const float w2 = fmaf(-q23, w3, y2) * i2;
        const float w1 = fmaf(-p13, w3, fmaf(-p12, w2, y1)) * i1;
        const float w0 = fmaf(-P[0][3], w3, fmaf(-P[0][2], w2, fmaf(-P[0][1], w1, y0))) * i0;
        ys[m][0] = y0; ys[m][1] = y1; ys[m][2] = y2; ys[m][3] = y3;
        ws[m][0] = w0; ws[m][1] = w1; ws[m][2] = w2; ws[m][3] = w3;
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int g = s >> 2;   // rows 8 g + 4 h + (s & 3)
        if (8 * g + 7 < k) continue;   // rows before K in both halves: done
        const float4 nv = sColQ[h][s];
        float* xs[3] = {&cm[s], &em[s], &tm[s]};
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          const float upd =
              fmaf(-nv.w, ws[m][3], fmaf(-nv.z, ws[m][2], fmaf(-nv.y, ws[m][1], fmaf(-nv.x, ws[m][0], *xs[m]))));
          if (g == (k >> 3)) {
            // The block of K: its rows in half hk, the rows past it (hk = 0)
            // or before it (hk = 1) in the other half.
            *xs[m] = h == hk ? ys[m][s & 3] : (hk == 0 ? upd : *xs[m]);
          } else {
            *xs[m] = upd;
          }
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
        for (int s = 0; s < 16; ++s) {
          float kv;
          if constexpr (F32)
            kv = reinterpret_cast<const float*>(&sTok[1][2 * I + (s >> 3)][(s & 7) >> 2][lane])[s & 3];
          else
            kv = frag_elem(kf[2 * I + (s >> 3)], s & 7);
          XK[I][s] = fmaf(eps, kv, XK[I][s]);
        }
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
      if constexpr (F32) {
        kn = sKn[lane];
      } else {
#pragma unroll
        for (int kp = 0; kp < 4; ++kp)
#pragma unroll
          for (int e = 0; e < 8; ++e) kn = fmaf(frag_elem(kf[kp], e), frag_elem(kf[kp], e), kn);
      }
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
  const int le = fresh_lane(), ce = le & 31, he = le >> 5;
  if (nudge_last) {
#pragma unroll
    for (int F = 0; F < 2; ++F)
#pragma unroll
      for (int s = 0; s < 16; ++s) Acc[F][F][s] += acc_row(s, he) == ce ? eps : 0.f;
  }
  if (chunk == nchunks - 1) {
    const auto rt = make_rsrc(A_T + chain * kD * kD, kD * kD * 4);
    const int a_voff = (8 * he * kD + feat(ce)) * 4;
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
  if (le == 0) {
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
                             int chunk_len, int nchunks, int chunk_lo, int chunk_cnt, bool bf16, int chains,
                             hipStream_t stream) {
  if (chunk_cnt <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(chains * chunk_cnt));
  auto kernel = a.residual ? (bf16 ? vla_inverse_wy_kernel<true, false> : vla_inverse_wy_kernel<true, true>)
                           : (bf16 ? vla_inverse_wy_kernel<false, false> : vla_inverse_wy_kernel<false, true>);
  hipLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, a.k, a.u, a_start, alpha_out, a.A_T, chain_info, a.T,
                     chunk_len, nchunks, chunk_lo, chunk_cnt, a.eps, a.nudge_period, a.nudge_phase0);
  return hipGetLastError();
}

}  // namespace vla
