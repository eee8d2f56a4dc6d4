// Inverse pass of the time-parallel schedule in blocked form at d = 128 (bf16
// storage, any rank r <= 4), on the gfx950 matrix cores.
//
// Method ("Mathematical Primitives", sections 2-3: rank-1 Sherman-Morrison
// tracking of A = M^{-1}, r sequential updates per token; section 4:
// alpha_t = A_t k_t; "Variational Linear Attention (VLA)" README, v3 notes:
// alpha_hat = alpha / max(|alpha|, 1)).  As in the d = 64 blocked pass
// (inverse_wy.hip), a block of m = r B directions u_j (B tokens, r each, in
// token order) starting from A_b composes exactly (Woodbury): with
// C = U^T A_b U and I + C = L D L^T,
//   delta_j = D_jj,
//   alpha_t = A_b k_t - X_U G[:, t],   G = L^{-T} D^{-1} ((L^{-1} U^T A_b K) o M),
//   M_jt = [j <= r t + r - 1]  (the directions of token t and the ones before),
//   A_{b+1} = A_b - X_U W X_U^T,  W = (I + C)^{-1},  X_U = A_b U.
// A guard fire (|delta| < eps) flags the chain for the sequential fallback.
//
// Four waves per chunk; B = 32 / r tokens per block (m <= 32 directions, one
// 32-wide matrix-core tile).  Wave w holds the column slab of A_b with
// feature block w, four 32 x 32 accumulator tiles (F, w), F = 0..3, in the
// permuted feature basis of the d = 64 kernel (bits 2 and 3 of a feature
// index swapped): A_b is symmetric, so a tile read as the A operand is the
// block it transposes to, and u and k rows enter as plain 16-byte pieces.
// Per block:
//   1. X_U and X_K for the wave's feature block (products over all four of
//      its tiles), and its share of C = U^T X_U and E = U^T X_K;
//   2. the LDL^T elimination of I + C (the d = 64 kernel's, two pivots per
//      LDS round trip) on three waves in step, one barrier per pivot pair:
//      wave 0 carries I + C, wave 1 E and wave 2 the identity (giving L^{-1}
//      E and L^{-1}); then wave 2 forms W and wave 1 G; every wave
//      transposes its X_U tile through LDS into X_U^T;
//   3. P^T = W X_U^T and alpha = X_K - X_U G per feature block;
//   4. A_b -= P^T X_U^T with every wave's P^T tile read from LDS, and
//      alpha_hat written once the per-token norms are summed over the waves.
// Tiles that every wave multiplies (W, G, P^T) cross LDS as three-term
// splits made once by the wave that produced them.
// Products with fp32 operands use three-term bf16 splits (fp32-grade).
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_mfma.h"
#include "vla_seq.h"
#include "vla_wide.h"

namespace vla {

namespace {

constexpr int kD = 128;
constexpr int kM = 32;        // directions per block (one tile)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXtLd = 36;     // row stride (floats) of the X_U transpose staging

// Feature held at basis index b: bits 2 and 3 swapped (an involution).
__host__ __device__ constexpr int feat(int b) { return (b & ~12) | ((b & 4) << 1) | ((b & 8) >> 1); }

__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }
// Workgroup barrier after this wave's LDS operations (global loads may stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

typedef __attribute__((address_space(3))) void lds_void;

// bf16 element e (0..7) of a 16-byte operand, as fp32.
__device__ __forceinline__ float frag_elem(const uint4& f, int e) {
  const uint32_t w = e < 2 ? f.x : e < 4 ? f.y : e < 6 ? f.z : f.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ uint4 as_u4(float4 a) {
  return make_uint4(__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w));
}

// An accumulator tile stored per lane (16 values), and read back: slots
// 4 i .. 4 i + 3 of every lane form one 1 KiB row (lane-consecutive 16-byte
// pieces, so the accesses do not collide on LDS banks).
__device__ __forceinline__ void put_tile(float* p, const f32x16& x, int lane) {
  float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[64 * i + lane] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}
__device__ __forceinline__ f32x16 get_tile(const float* p, int lane) {
  const float4* q = reinterpret_cast<const float4*>(p);
  f32x16 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = q[64 * i + lane];
    x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
  }
  return x;
}

// A tile's three-term split as MFMA operands, [k step g][term][lane]: each
// tile is split once, by the wave that produced it, and every wave reads the
// terms (16 lane-consecutive bytes per read).
typedef uint4 SplitTile[2][3][64];

__device__ __forceinline__ void put_split(SplitTile& p, const f32x16& x, float scale, int lane) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const Split3 t = split_slots(x, g, scale);
    p[g][0][lane] = __builtin_bit_cast(uint4, t.t1);
    p[g][1][lane] = __builtin_bit_cast(uint4, t.t2);
    p[g][2][lane] = __builtin_bit_cast(uint4, t.t3);
  }
}
__device__ __forceinline__ Split3 get_split(const SplitTile& p, int g, int lane) {
  Split3 t;
  t.t1 = __builtin_bit_cast(bf16x8, p[g][0][lane]);
  t.t2 = __builtin_bit_cast(bf16x8, p[g][1][lane]);
  t.t3 = __builtin_bit_cast(bf16x8, p[g][2][lane]);
  return t;
}

struct Lds128 {
  float4 tok[2][8][64];              // [u / k][k step kp][lane (c, h)]: features 16 kp + 8 h .. of direction / key c
  union {
    float part[2][kWaves - 1][64 * 16];   // phases 1-2: waves 1..3's shares of C and E
    SplitTile wg[2];                      // phases 2-3: W and -G from wave 0 (after it has read the shares)
  } pw;
  union {
    float xt[32 * kXtLd];             // X_U transpose staging
    SplitTile pt;                     // then -P^T of the wave's feature block
  } xp[kWaves];
  float nrm[kWaves][32];              // per-token |alpha|^2 over each wave's features
  float4 sCol[2][2][2][4];            // elimination, by pivot pair parity: columns k, k + 1 of I + C
  float2 sRow[2][3][kM];              // rows k, k + 1 of I + C, E and T at column c
  float sDinv[kM];                    // 1 / pivot
};

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
vla_inverse_wy128_kernel(const uint16_t* __restrict__ kx, const uint16_t* __restrict__ ux,
                         const float* __restrict__ a_start, float* __restrict__ alpha_out, float* __restrict__ A_T,
                         int32_t* __restrict__ chain_info, int T, int r, int L, int nchunks, int cm, int inv_lo,
                         int inv_cnt, float eps, int nudge_period, int nudge_phase0) {
  __shared__ __attribute__((aligned(16))) Lds128 sm;
  // The workgroup's span: cm consecutive chunks of L tokens from chunk0
  // (fewer at the end of the chain), starting from chunk0's start inverse.
  const int64_t chain = blockIdx.x / inv_cnt;
  const int chunk0 = (inv_lo + static_cast<int>(blockIdx.x % inv_cnt)) * cm;
  const int tbeg = chunk0 * L, tend = min(T, (chunk0 + cm) * L);
  const int tid = threadIdx.x, lane0 = tid & 63, c0 = lane0 & 31, h0 = lane0 >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = kM / r;          // tokens per block

  // ---- A_b: tile F slot s = A[feat(32 F + acc_row(s, h))][feat(32 w + c)].
  // Slot s = 4 q + e sits at row 32 F + 16 (q >> 1) + 8 h + 4 (q & 1) + e.
  const int a_voff = (8 * h0 * kD + feat(c0)) * 4;
  auto a_soff = [&](int F, int s) {
    const int q = s >> 2, e = s & 3;
    return ((32 * F + 16 * (q >> 1) + 4 * (q & 1) + e) * kD + 32 * w) * 4;
  };
  f32x16 Acc[4];
  {
    const auto ra = make_rsrc(a_start + (chain * nchunks + chunk0) * kD * kD, kD * kD * 4);
#pragma unroll
    for (int F = 0; F < 4; ++F)
#pragma unroll
      for (int s = 0; s < 16; ++s)
        Acc[F][s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, a_voff, a_soff(F, s), 0));
  }

  // Token rows go from HBM straight into LDS: wave w copies k steps 2 w and
  // 2 w + 1 of the block's u and k rows; lane (c, h) takes features
  // 16 kp + 8 h .. + 7 of direction c (u) and of token c (k).  Lanes with no
  // direction or token in the block (the last block of a chunk may be short)
  // read past the end of the buffers, so their rows are zero.
  const int64_t row0 = chain * T + tbeg;
  const int ubytes = (tend - tbeg) * r * kD * 2, kbytes = (tend - tbeg) * kD * 2;
  const auto ru = make_rsrc(ux + row0 * r * kD, ubytes);
  const auto rk = make_rsrc(kx + row0 * kD, kbytes);
  auto copy_tokens = [&](int tb, int cnt) {
    const int ou = c0 < cnt * r ? (((tb - tbeg) * r + c0) * kD + 8 * h0) * 2 : ubytes;
    const int ok = c0 < cnt ? ((tb - tbeg + c0) * kD + 8 * h0) * 2 : kbytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kp = 2 * w + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void*)&sm.tok[0][kp][0], 16, ou + 32 * kp, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)&sm.tok[1][kp][0], 16, ok + 32 * kp, 0, 0, 0);
    }
  };

  int guard = 0;
  bool bad = false;
  // Blocks run chunk by chunk: a chunk's last block may be short, and the
  // nudge, when it falls on a chunk's last token (no nudge falls inside a
  // chunk), is applied before the next chunk's first block.
  int sub_end = min(tend, tbeg + L);
  copy_tokens(tbeg, min(B, sub_end - tbeg));

  for (int tb = tbeg; tb < tend;) {
    const int tcount = min(B, sub_end - tb);
    const bool sub_last = tb + B >= sub_end;
    const bool last_block = sub_last && sub_end == tend;
    const bool nudged = sub_last && nudge_period > 0 && (nudge_phase0 + sub_end - 1) % nudge_period == 0;
    const int tb_next = sub_last ? sub_end : tb + B;
    const int sub_end_next = sub_last ? min(tend, sub_end + L) : sub_end;
    int c = c0, h = h0;
    asm volatile("" : "+v"(c), "+v"(h));
    const int lane = c + 32 * h;
    // Every wave's copies of the block's rows have landed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    // ---- 1. X_U = A U and X_K = A K on this wave's feature block (rows:
    // basis features 32 w.., columns: directions / tokens), and its shares
    // of C = U^T X_U and E = U^T X_K.
    f32x16 XU = zero16(), XK = zero16();
#pragma unroll
    for (int F = 0; F < 4; ++F)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int kp = 2 * F + g;
        const bf16x8 ub = __builtin_bit_cast(bf16x8, as_u4(sm.tok[0][kp][lane]));
        const bf16x8 kb = __builtin_bit_cast(bf16x8, as_u4(sm.tok[1][kp][lane]));
        const Split3 af = split_slots(Acc[F], g);
        XU = mma_split(af, ub, XU);
        XK = mma_split(af, kb, XK);
        sched_fence();
      }
    f32x16 Cm = zero16(), Em = zero16();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bf16x8 ub = __builtin_bit_cast(bf16x8, as_u4(sm.tok[0][2 * w + g][lane]));
      Cm = mma_split(ub, split_slots(XU, g), Cm);
      Em = mma_split(ub, split_slots(XK, g), Em);
    }
    // Shares for the elimination: C to wave 0 (from waves 1..3), E to wave 1
    // (from waves 0, 2, 3).
    if (w > 0) put_tile(sm.pw.part[0][w - 1], Cm, lane);
    if (w != 1) put_tile(sm.pw.part[1][w == 0 ? 0 : w - 1], Em, lane);
    lds_barrier();

    // ---- 2. The elimination, on three waves: wave 0 carries I + C, wave 1
    // E and wave 2 T (the identity, becoming L^{-1}); each applies the same
    // pivots to its matrix.  Every wave: X_U^T through its LDS staging tile,
    // X_U^T[j][f] = X_U[f][j] (X_U is staged first, so it is not live through
    // the elimination).
    float* xt = sm.xp[w].xt;
#pragma unroll
    for (int s = 0; s < 16; ++s) xt[acc_row(s, h) * kXtLd + c] = XU[s];
    // Lane (c, h) holds column c of its matrix; pivot k sits in lane half
    // (k >> 2) & 1, slot 4 (k >> 3) + (k & 3).  C and E are summed over the
    // waves in a fixed order (wave 0's share first).
    float mt[16];
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < kWaves - 1; ++j) {
        const f32x16 pc = get_tile(sm.pw.part[0][j], lane);
#pragma unroll
        for (int s = 0; s < 16; ++s) Cm[s] += pc[s];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) mt[s] = Cm[s] + (acc_row(s, h) == c ? 1.f : 0.f);
    } else if (w == 1) {
      const f32x16 p0 = get_tile(sm.pw.part[1][0], lane);
#pragma unroll
      for (int s = 0; s < 16; ++s) Em[s] += p0[s];
#pragma unroll
      for (int j = 1; j < kWaves - 1; ++j) {
        const f32x16 pe = get_tile(sm.pw.part[1][j], lane);
#pragma unroll
        for (int s = 0; s < 16; ++s) Em[s] += pe[s];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) mt[s] = Em[s];
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) mt[s] = (w == 2 && acc_row(s, h) == c) ? 1.f : 0.f;
    }
    const float hf = static_cast<float>(h);
    const int ws = w < 3 ? w : 2;   // wave 3 follows the barriers only (its rows are not read)
    // Two pivots per LDS round trip: the lanes get columns k and k + 1 of
    // I + C and rows k and k + 1 of their own matrix as they stood before
    // pivot k, and apply pivot k to their copies of column and row k + 1
    // themselves.  Buffers alternate by pivot pair, so one barrier per pair
    // orders every wave's reads of a pair before the writes two pairs later.
#pragma unroll
    for (int k = 0; k < kM; k += 2) {
      const int hk = (k >> 2) & 1, sk = 4 * (k >> 3) + (k & 3), pp = (k >> 1) & 1;
      if (w == 0 && (c == k || c == k + 1)) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sm.sCol[pp][c - k][h][q] = make_float4(mt[4 * q], mt[4 * q + 1], mt[4 * q + 2], mt[4 * q + 3]);
      }
      if (w < 3 && h == hk) sm.sRow[pp][w][c] = make_float2(mt[sk], mt[sk + 1]);
      lds_barrier();
      float na[16], nb[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = sm.sCol[pp][0][h][q], u4 = sm.sCol[pp][1][h][q];
        na[4 * q] = v.x; na[4 * q + 1] = v.y; na[4 * q + 2] = v.z; na[4 * q + 3] = v.w;
        nb[4 * q] = u4.x; nb[4 * q + 1] = u4.y; nb[4 * q + 2] = u4.z; nb[4 * q + 3] = u4.w;
      }
      const float2 pa = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(sm.sCol[pp][0][hk]) + sk);
      const float2 pb = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(sm.sCol[pp][1][hk]) + sk);
      const float2 rw = sm.sRow[pp][ws][c];
      float ia = __builtin_amdgcn_rcpf(pa.x);
      ia = fmaf(fmaf(-pa.x, ia, 1.f), ia, ia);
      const float a0 = rw.x * ia;
      const float q0 = fmaf(-pa.y, a0, rw.y);
      const float gab = pb.x * ia;
      const float pk1 = fmaf(-pa.y, gab, pb.y);
      float ib = __builtin_amdgcn_rcpf(pk1);
      ib = fmaf(fmaf(-pk1, ib, 1.f), ib, ib);
      const float b0 = q0 * ib;
      if (w == 0) {
        guard += (fabsf(pa.x) < eps ? 1 : 0) + (fabsf(pk1) < eps ? 1 : 0);
        asm volatile("" : "+v"(guard));
        if (lane == 0) {
          sm.sDinv[k] = ia;
          sm.sDinv[k + 1] = ib;
        }
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int base = 8 * (s >> 2) + (s & 3);   // row of slot s is base + 4 h
        if (base + 4 <= k) continue;
        const float xa = base > k ? na[s] : na[s] * hf;
        mt[s] = fmaf(-xa, a0, mt[s]);
        if (base + 4 > k + 1) {
          const float nk = fmaf(-na[s], gab, nb[s]);
          const float xb = base > k + 1 ? nk : nk * hf;
          mt[s] = fmaf(-xb, b0, mt[s]);
        }
        asm volatile("" : "+v"(mt[s]));
      }
    }
    // W = T^T D^{-1} T on wave 2 and G = T^T D^{-1} (F o M) on wave 1, T =
    // L^{-1}, F = L^{-1} E, M_jt = [j <= r t + r - 1]; wave 2 passes T to
    // wave 1 through the space of E's shares (read before the first pivot).
    if (w == 2) {
      f32x16 tv;
#pragma unroll
      for (int s = 0; s < 16; ++s) tv[s] = mt[s];
      put_tile(sm.pw.part[1][0], tv, lane);
    }
    lds_barrier();   // T, and the last pivots of D^{-1}
    if (w == 1 || w == 2) {
      float dv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(sm.sDinv + 8 * q + 4 * h);
        dv[4 * q] = v.x; dv[4 * q + 1] = v.y; dv[4 * q + 2] = v.z; dv[4 * q + 3] = v.w;
      }
      f32x16 tmv;
      if (w == 1) {
        tmv = get_tile(sm.pw.part[1][0], lane);
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) tmv[s] = mt[s];
      }
      const int jlast = r * c + r - 1;
      f32x16 Xm = zero16();
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float td[8], xr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int s = 8 * g + e;
          td[e] = tmv[s] * dv[s];
          xr[e] = w == 2 ? tmv[s] : (acc_row(s, h) <= jlast ? mt[s] : 0.f);
        }
        Xm = mma_split(split3(td), split3(xr), Xm);
      }
      put_split(sm.pw.wg[w == 2 ? 0 : 1], Xm, w == 2 ? 1.f : -1.f, lane);
    }
    lds_order();
    f32x16 XT;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(xt + c * kXtLd + 8 * q + 4 * h);
      XT[4 * q] = v.x; XT[4 * q + 1] = v.y; XT[4 * q + 2] = v.z; XT[4 * q + 3] = v.w;
    }
    lds_barrier();

    // ---- 3. P^T = W X_U^T (directions x features) and alpha = X_K - X_U G.
    Split3 XS[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) XS[g] = split_slots(XT, g);
    f32x16 PT = zero16();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      PT = mma_split(get_split(sm.pw.wg[0], g, lane), XS[g], PT);
      XK = mma_split(XS[g], get_split(sm.pw.wg[1], g, lane), XK);
      sched_fence();
    }
    if (nudged && c == tcount - 1) {
      // The chunk's last token is nudged: alpha = (A + eps I) k.
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint4 kf = as_u4(sm.tok[1][2 * w + (s >> 3)][lane]);
        XK[s] = fmaf(eps, frag_elem(kf, s & 7), XK[s]);
      }
    }
    {
      float nrm = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) nrm = fmaf(XK[s], XK[s], nrm);
      nrm += __shfl_xor(nrm, 32);
      if (h == 0) sm.nrm[w][c] = nrm;
    }
    // The wave's -P^T tile, split, for every wave's update (over its own
    // staging tile: its transpose reads are done).
    put_split(sm.xp[w].pt, PT, -1.f, lane);
    lds_barrier();

    // The next block's rows (every read of this block's rows is done).
    if (!last_block) copy_tokens(tb_next, min(B, sub_end_next - tb_next));

    // ---- 4. A_{b+1} = A_b - P^T X_U^T, and alpha_hat of the block's tokens.
#pragma unroll
    for (int F = 0; F < 4; ++F) {
#pragma unroll
      for (int g = 0; g < 2; ++g) Acc[F] = mma_split(get_split(sm.xp[F].pt, g, lane), XS[g], Acc[F]);
      sched_fence();
    }
    if (c < tcount) {
      const float n2 = (sm.nrm[0][c] + sm.nrm[1][c]) + (sm.nrm[2][c] + sm.nrm[3][c]);
      const float ascale = n2 > 1.f ? 1.f / sqrtf(n2) : 1.f;
      float* dst = alpha_out + (chain * T + tb + c) * kD;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = make_float4(XK[4 * q] * ascale, XK[4 * q + 1] * ascale, XK[4 * q + 2] * ascale,
                                     XK[4 * q + 3] * ascale);
        bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
        *reinterpret_cast<float4*>(dst + feat(32 * w + 4 * (2 * q + h))) = v;
      }
    }
    // The chunk's end state after a nudge: A + eps I.
    if (nudged) {
#pragma unroll
      for (int F = 0; F < 4; ++F) {   // the diagonal tile (w, w); F stays a constant index
        if (F == w) {
#pragma unroll
          for (int s = 0; s < 16; ++s) Acc[F][s] += acc_row(s, h) == c ? eps : 0.f;
        }
      }
    }
    tb = tb_next;
    sub_end = sub_end_next;
  }

  // ---- A_T from the chain's last chunk.
  if (chunk0 + cm >= nchunks) {
    const auto rt = make_rsrc(A_T + chain * kD * kD, kD * kD * 4);
#pragma unroll
    for (int F = 0; F < 4; ++F)
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const float v = Acc[F][s];
        bad |= !isfinite(v);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rt, a_voff, a_soff(F, s), 0);
      }
  }
  const bool wave_bad = __any(bad);
  if (lane0 == 0) {
    int32_t* info = chain_info + chain * 4;
    if (guard > 0) {   // (only wave 0 counts pivots)
      atomicAdd(info + kInfoGuard, guard);
      atomicOr(info + kInfoFallback, 1);
    }
    if (wave_bad) atomicOr(info + kInfoNonfinite, 1);
  }
}

}  // namespace

hipError_t launch_inverse_wy128(const ScanArgs& a, const float* a_start, float* alpha_out, int32_t* chain_info,
                                int chunk_len, int nchunks, int cm, int inv_lo, int inv_cnt, int chains,
                                hipStream_t stream) {
  if (inv_cnt <= 0) return hipSuccess;
  if (a.residual || a.r < 1 || a.r > 4 || cm < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vla_inverse_wy128_kernel, dim3(static_cast<unsigned>(chains * inv_cnt)), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.u), a_start, alpha_out,
                     a.A_T, chain_info, a.T, a.r, chunk_len, nchunks, cm, inv_lo, inv_cnt, a.eps, a.nudge_period,
                     a.nudge_phase0);
  return hipGetLastError();
}

}  // namespace vla
