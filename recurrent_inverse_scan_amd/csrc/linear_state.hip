// State pass of the time-parallel schedule at d = 128 without the Frobenius
// cap (additive update, bf16 storage of q, k, v and o).
//
// Method ("Variational Linear Attention (VLA)" README, v3 notes; "Variational
// Linear Attention: Stable Associative Memory for Long-Context Transformers",
// technical summary 2.4): with the cap off, S_t = S_0 + sum_{s<=t} v_s
// alpha_hat_s^T and n_t = n_0 + sum_{s<=t} k_s are plain prefix sums of the
// coefficients the inverse pass produced, so the readout
// o_t = S_t q_t / (n_t . q_t + den_eps) splits over chunks of 256 tokens as
// chunked linear attention does:
//   S_t q_t   = S_c q_t + sum_{s in chunk, s <= t} v_s (alpha_hat_s . q_t)
//   n_t . q_t = n_c . q_t + sum_{s in chunk, s <= t} k_s . q_t
// with S_c and n_c the state at the chunk start.
//
// Kernels, in stream order:
//   vla_lin_sums_kernel     per chunk: sum v alpha_hat^T and sum k
//   vla_lin_prefix_kernel   per state element: exclusive prefix over the
//                           chunks, in place (the chunk starts S_c, n_c),
//                           and S_T, n_T
//   vla_lin_readout_kernel  per chunk: both terms above and o
//   vla_lin_stats_kernel    per chain: guard fires and the non-finite flag
// The products run on the bf16 matrix cores.  q, k and v are bf16 and enter
// exactly; alpha_hat, S_c and the fp32 scores alpha_hat . q enter as
// three-term bf16 splits, which represent them exactly, so every product is
// fp32-grade.
#include "vla_common.h"
#include "vla_kernels.h"
#include "vla_mfma.h"
#include "vla_seq.h"

namespace vla {

namespace {

constexpr int kD = 128;
constexpr int kLinThreads = 512;   // eight waves
constexpr int kTile = 32;          // tokens per LDS stage
constexpr int kLdT16 = kTile + 8;  // bf16 per transposed row ([column][token]): 80 bytes
constexpr int kLdT32 = kTile + 4;  // fp32 per transposed row: 144 bytes
constexpr int kLdR16 = kD + 8;     // bf16 per token row: 272 bytes

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
// Eight consecutive fp32 values from LDS as a three-term split.
__device__ __forceinline__ Split3 lds_split8(const float* p) {
  const float4 x0 = *reinterpret_cast<const float4*>(p);
  const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  return split3(v);
}
// A 16-byte global load, or zeros when !ok.  (Written as a branch: a select
// between the loaded value and a zero constant becomes a select of pointers,
// with the constant spilled to scratch and a flat load.)
__device__ __forceinline__ uint4 load16_or_zero(const void* p, bool ok) {
  uint4 x = make_uint4(0, 0, 0, 0);
  if (ok) x = *reinterpret_cast<const uint4*>(p);
  return x;
}
__device__ __forceinline__ uint16_t half16(uint4 x, int e) {
  const uint32_t w = e < 2 ? x.x : (e < 4 ? x.y : (e < 6 ? x.z : x.w));
  return static_cast<uint16_t>((e & 1) ? (w >> 16) : w);
}

// ---- chunk sums -----------------------------------------------------------
// dS_c = V^T alpha_hat over the chunk's tokens (128 x 128, contraction over
// tokens), dn_c = sum of k.  Wave w computes the 32 x 32 tiles (row block
// w / 2, column blocks 2 (w % 2) and 2 (w % 2) + 1).  The contraction runs
// over tokens, so both operands need eight consecutive tokens of one column
// per lane: v and alpha_hat pass through LDS transposed ([column][token]),
// 32 tokens a stage, the next stage loaded while the current one multiplies.
__global__ void __launch_bounds__(kLinThreads)
vla_lin_sums_kernel(LinPlan lp) {
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][kD * kLdT16];
  __shared__ __attribute__((aligned(16))) float sAt[2][kD * kLdT32];
  const int64_t chain = blockIdx.x / lp.ncs;
  const int cs = blockIdx.x % lp.ncs;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
  const int t0 = cs * kLinChunk;
  const int ntok = min(kLinChunk, lp.T - t0);
  const int ntile = (ntok + kTile - 1) / kTile;
  const int64_t row0 = chain * lp.T + t0;
  const uint16_t* V = static_cast<const uint16_t*>(lp.v) + row0 * kD;
  const uint16_t* K = static_cast<const uint16_t*>(lp.k) + row0 * kD;
  const float* Al = lp.alpha + row0 * kD;
  // Thread (token s of the stage, v and k columns 8 p .., alpha_hat columns
  // 4 p .. and 4 (p + 16) ..).
  const int s = tid & 31, p = tid >> 5;
  uint4 rv, rk, ra0, ra1;
  float ksum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto load = [&](int tile) {
    const int tl = tile * kTile + s;
    const bool ok = tl < ntok;
    const int64_t r = static_cast<int64_t>(tl) * kD;
    rv = load16_or_zero(V + r + 8 * p, ok);
    rk = load16_or_zero(K + r + 8 * p, ok);
    ra0 = load16_or_zero(Al + r + 4 * p, ok);
    ra1 = load16_or_zero(Al + r + 4 * (p + 16), ok);
  };
  auto store = [&](int buf) {
    uint16_t* vt = sVt[buf] + 8 * p * kLdT16 + s;
    float* at0 = sAt[buf] + 4 * p * kLdT32 + s;
    float* at1 = sAt[buf] + 4 * (p + 16) * kLdT32 + s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vt[e * kLdT16] = half16(rv, e);
      ksum[e] += bf16_to_f32(half16(rk, e));
    }
    at0[0] = __uint_as_float(ra0.x); at0[kLdT32] = __uint_as_float(ra0.y);
    at0[2 * kLdT32] = __uint_as_float(ra0.z); at0[3 * kLdT32] = __uint_as_float(ra0.w);
    at1[0] = __uint_as_float(ra1.x); at1[kLdT32] = __uint_as_float(ra1.y);
    at1[2 * kLdT32] = __uint_as_float(ra1.z); at1[3 * kLdT32] = __uint_as_float(ra1.w);
  };
  const int it = w >> 1, jt0 = 2 * (w & 1);
  f32x16 acc[2] = {zero16(), zero16()};
  if (ntile > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntile; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntile) load(tile + 1);
#pragma unroll
    for (int kk = 0; kk < kTile / 16; ++kk) {
      const int off = 16 * kk + 8 * h;
      const bf16x8 a = lds_bf16x8(&sVt[buf][(32 * it + c32) * kLdT16 + off]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const Split3 bs = lds_split8(&sAt[buf][(32 * (jt0 + b) + c32) * kLdT32 + off]);
        acc[b] = mma_split(a, bs, acc[b]);
      }
    }
    // Buffer buf ^ 1 was last read in the previous stage, before its barrier.
    if (tile + 1 < ntile) store(buf ^ 1);
    __syncthreads();
  }
  float* dS = lp.dS + (chain * lp.ncs + cs) * kD * kD;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int sl = 0; sl < 16; ++sl) dS[(32 * it + acc_row(sl, h)) * kD + 32 * (jt0 + b) + c32] = acc[b][sl];
  // k sums: the 32 lanes of a half wave hold the same columns.
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float x = group_sum<16>(ksum[e]);
    x += __shfl_xor(x, 16, 64);
    ksum[e] = x;
  }
  if (c32 == 0) {
    float* dn = lp.dn + (chain * lp.ncs + cs) * kD + 8 * p;
    *reinterpret_cast<float4*>(dn) = make_float4(ksum[0], ksum[1], ksum[2], ksum[3]);
    *reinterpret_cast<float4*>(dn + 4) = make_float4(ksum[4], ksum[5], ksum[6], ksum[7]);
  }
}

// ---- prefix over chunks -----------------------------------------------------
// One thread per (chain, element of S or n): the chunk sums become the state
// at each chunk start (exclusive prefix from S_0, n_0), and the total is the
// final state.  Loads run eight chunks ahead of the running sum.
__global__ void __launch_bounds__(256)
vla_lin_prefix_kernel(LinPlan lp) {
  constexpr int E = kD * kD + kD;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(lp.chains) * E) return;
  const int64_t chain = idx / E;
  const int e = static_cast<int>(idx % E);
  const bool is_s = e < kD * kD;
  const int en = e - kD * kD;
  float* base = is_s ? lp.dS + chain * lp.ncs * kD * kD + e : lp.dn + chain * lp.ncs * kD + en;
  const int64_t stride = is_s ? kD * kD : kD;
  float acc = is_s ? lp.S_init[chain * kD * kD + e] : lp.n_init[chain * kD + en];
  for (int c0 = 0; c0 < lp.ncs; c0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = c0 + j < lp.ncs ? base[(c0 + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j < lp.ncs) {
        base[(c0 + j) * stride] = acc;
        acc += x[j];
      }
    }
  }
  if (is_s)
    lp.S_T[chain * kD * kD + e] = acc;
  else
    lp.n_T[chain * kD + en] = acc;
  if (!isfinite(acc)) atomicOr(lp.chain_info + chain * 4 + kInfoNonfinite, 1);
}

// ---- readout ----------------------------------------------------------------
// One workgroup per chunk.  Wave w owns 32 tokens (row tile rt; the pairing
// of tiles rt and 7 - rt on one SIMD evens out the causal work) and
// accumulates O[t][i] (four 32 x 32 tiles over i):
//   1. O = Q S_c^T: A operand q (eight consecutive columns of a token row,
//      held in registers for the whole chunk), B operand rows of S_c (LDS).
//   2. For each earlier or diagonal 32-token tile st of the chunk:
//      P^T = alpha_hat_st Q^T (scores, fp32), masked to s <= t on the
//      diagonal; O += P V_st with P^T's accumulator read as the A operand.
//      P^T's rows are permuted (row m holds token sigma(m), bits 2 and 3 of m
//      swapped) so that accumulator slots 8 kk .. 8 kk + 7 of lane l hold
//      tokens 16 kk + 8 (l >> 5) .. + 7 in order, the A operand layout.
//      The normaliser's in-chunk part sum_{s<=t} k_s . q_t comes from
//      K_st Q^T the same way, summed over s.
//   3. o = O / (n_c . q + in-chunk part + den_eps).
// Every stage of 32 tokens (alpha_hat rows, k rows, v transposed) goes
// through LDS once for all waves; the next is loaded while the current one
// multiplies.  The fp32 operands shared by the waves (alpha_hat, and S_c in
// two halves of 64 rows) are split into their three bf16 terms once, as
// they enter LDS, instead of by every wave that reads them.
constexpr int kPieces = kD / 8;     // 16-byte pieces (eight values) per row
constexpr int kPLd = kPieces + 1;   // padded: consecutive rows start one bank group apart

struct ReadoutStage {
  uint4 As[3][kTile][kPLd];      // alpha_hat rows: [term][token][piece]
  uint16_t K[kTile * kLdR16];    // k rows
  uint16_t Vt[kD * kLdT16];      // v columns
};

// Split terms of four consecutive values, each term four bf16 (8 bytes);
// the same terms as split3 gives for them.
__device__ __forceinline__ void split3_words4(const float4& x, uint2 (&t)[3]) {
#pragma clang fp contract(off)
  const float v[4] = {x.x, x.y, x.z, x.w};
  uint32_t a[4], r[4], c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = __float_as_uint(v[e]);
    const float rf = v[e] - __uint_as_float(a[e] & 0xffff0000u);
    r[e] = __float_as_uint(rf);
    c[e] = __float_as_uint(rf - __uint_as_float(r[e] & 0xffff0000u));
  }
  t[0] = make_uint2(pack_hi16(a[0], a[1]), pack_hi16(a[2], a[3]));
  t[1] = make_uint2(pack_hi16(r[0], r[1]), pack_hi16(r[2], r[3]));
  t[2] = make_uint2(pack_hi16(c[0], c[1]), pack_hi16(c[2], c[3]));
}
__device__ __forceinline__ Split3 get_split(const uint4 (*p)[kPLd], int row, int piece, int stride) {
  Split3 t;
  t.t1 = __builtin_bit_cast(bf16x8, p[row][piece]);
  t.t2 = __builtin_bit_cast(bf16x8, p[stride + row][piece]);
  t.t3 = __builtin_bit_cast(bf16x8, p[2 * stride + row][piece]);
  return t;
}

__device__ __forceinline__ int sigma(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__global__ void __launch_bounds__(kLinThreads)
vla_lin_readout_kernel(LinPlan lp) {
  __shared__ __attribute__((aligned(16))) uint4 sSs[3][64][kPLd];   // half of S_c: [term][row][piece]
  __shared__ __attribute__((aligned(16))) ReadoutStage st[2];
  __shared__ float sDen[8][kTile];
  const int64_t chain = blockIdx.x / lp.ncs;
  const int cs = blockIdx.x % lp.ncs;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w < 4 ? w : 11 - w;
  const int t0 = cs * kLinChunk;
  const int ntok = min(kLinChunk, lp.T - t0);
  const int ntile = (ntok + kTile - 1) / kTile;
  const int64_t row0 = chain * lp.T + t0;
  const uint16_t* Q = static_cast<const uint16_t*>(lp.q) + row0 * kD;
  const uint16_t* K = static_cast<const uint16_t*>(lp.k) + row0 * kD;
  const uint16_t* V = static_cast<const uint16_t*>(lp.v) + row0 * kD;
  const float* Al = lp.alpha + row0 * kD;
  const float* Sc = lp.dS + (chain * lp.ncs + cs) * kD * kD;
  const float* nc = lp.dn + (chain * lp.ncs + cs) * kD;

  // This wave's q rows as operands: token 32 rt + c32, columns 16 kk + 8 h ...
  const int tq = kTile * rt + c32;
  const bool tq_ok = tq < ntok;
  bf16x8 qop[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qop[kk] = __builtin_bit_cast(bf16x8, load16_or_zero(Q + static_cast<int64_t>(tq) * kD + 16 * kk + 8 * h, tq_ok));

  // Stage loads: alpha_hat pieces (token tid / 32 + 16 j, columns 4 (tid % 32) ..),
  // k pieces (token tid / 16, columns 8 (tid % 16) ..), v pieces (token
  // tid % 32, columns 8 (tid / 32) .., stored transposed).
  uint4 ra0, ra1, rk, rv;
  auto load = [&](int tile) {
    const int tb = tile * kTile;
    const int ta = tb + (tid >> 5);
    ra0 = load16_or_zero(Al + static_cast<int64_t>(ta) * kD + 4 * (tid & 31), ta < ntok);
    ra1 = load16_or_zero(Al + static_cast<int64_t>(ta + 16) * kD + 4 * (tid & 31), ta + 16 < ntok);
    const int tk = tb + (tid >> 4);
    rk = load16_or_zero(K + static_cast<int64_t>(tk) * kD + 8 * (tid & 15), tk < ntok);
    const int tv = tb + (tid & 31);
    rv = load16_or_zero(V + static_cast<int64_t>(tv) * kD + 8 * (tid >> 5), tv < ntok);
  };
  auto store = [&](ReadoutStage& sg) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint2 tw[3];
      const uint4 ra = j ? ra1 : ra0;
      split3_words4(make_float4(__uint_as_float(ra.x), __uint_as_float(ra.y), __uint_as_float(ra.z),
                                __uint_as_float(ra.w)), tw);
#pragma unroll
      for (int tm = 0; tm < 3; ++tm)
        reinterpret_cast<uint2*>(&sg.As[tm][(tid >> 5) + 16 * j][(tid & 31) >> 1])[tid & 1] = tw[tm];
    }
    *reinterpret_cast<uint4*>(&sg.K[(tid >> 4) * kLdR16 + 8 * (tid & 15)]) = rk;
#pragma unroll
    for (int e = 0; e < 8; ++e) sg.Vt[(8 * (tid >> 5) + e) * kLdT16 + (tid & 31)] = half16(rv, e);
  };

  // S_c by halves of 64 rows: each thread splits two pieces of eight values
  // (row pc / 16, piece pc % 16); the second half's values are loaded while
  // the first half multiplies.
  float4 sx[2][2];
  auto load_half = [&](int hf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pc = tid + kLinThreads * j;
      const float* src = Sc + (64 * hf + (pc >> 4)) * kD + 8 * (pc & 15);
      sx[j][0] = *reinterpret_cast<const float4*>(src);
      sx[j][1] = *reinterpret_cast<const float4*>(src + 4);
    }
  };
  auto store_half = [&]() {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pc = tid + kLinThreads * j;
      const float v[8] = {sx[j][0].x, sx[j][0].y, sx[j][0].z, sx[j][0].w,
                          sx[j][1].x, sx[j][1].y, sx[j][1].z, sx[j][1].w};
      const Split3 t = split3(v);
      sSs[0][pc >> 4][pc & 15] = __builtin_bit_cast(uint4, t.t1);
      sSs[1][pc >> 4][pc & 15] = __builtin_bit_cast(uint4, t.t2);
      sSs[2][pc >> 4][pc & 15] = __builtin_bit_cast(uint4, t.t3);
    }
  };
  load_half(0);
  if (ntile > 0) load(0);
  store_half();
  load_half(1);
  if (ntile > 0) store(st[0]);
  __syncthreads();

  // 1. O = Q S_c^T, rows i of S_c (column tiles ib of O) by halves.
  f32x16 O[4] = {zero16(), zero16(), zero16(), zero16()};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (hf == 1) {
      __syncthreads();   // every wave is done with the first half
      store_half();
      __syncthreads();
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int ib = 2 * hf; ib < 2 * hf + 2; ++ib)
        O[ib] = mma_split(qop[kk], get_split(sSs[0], 32 * (ib - 2 * hf) + c32, 2 * kk + h, 64), O[ib]);
  }

  // n_c . q_t for this lane's token, over its columns (completed across the
  // lane halves below).
  float nq = 0.f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const uint4 qv = __builtin_bit_cast(uint4, qop[kk]);
    const float4 n0 = *reinterpret_cast<const float4*>(nc + 16 * kk + 8 * h);
    const float4 n1 = *reinterpret_cast<const float4*>(nc + 16 * kk + 8 * h + 4);
    const float nv[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) nq = fmaf(nv[e], bf16_to_f32(half16(qv, e)), nq);
  }

  // 2. The chunk's own tokens, one stage at a time.
  const int sm = sigma(c32);
  for (int tile = 0; tile < ntile; ++tile) {
    const ReadoutStage& sg = st[tile & 1];
    if (tile + 1 < ntile) load(tile + 1);
    if (tile <= rt) {   // wave-uniform
      f32x16 P = zero16(), Pk = zero16();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        P = mma_split(get_split(sg.As[0], sm, 2 * kk + h, kTile), qop[kk], P);
        Pk = mfma_bf16(lds_bf16x8(&sg.K[c32 * kLdR16 + 16 * kk + 8 * h]), qop[kk], Pk);
      }
      if (tile == rt) {   // causal mask on the diagonal tile: token s > token t
#pragma unroll
        for (int sl = 0; sl < 16; ++sl) {
          const int m = acc_row(sl, h);
          if (sigma(m) > c32) P[sl] = 0.f;
          if (m > c32) Pk[sl] = 0.f;
        }
      }
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) nq += Pk[sl];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Split3 pa = split_slots(P, kk);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          O[ib] = mma_split(pa, lds_bf16x8(&sg.Vt[(32 * ib + c32) * kLdT16 + 16 * kk + 8 * h]), O[ib]);
      }
    }
    if (tile + 1 < ntile) store(st[(tile + 1) & 1]);
    __syncthreads();
  }

  // 3. Normalise and store.  Lane l's denominator belongs to token c32; the
  // accumulator rows are other tokens, so it goes through LDS.
  nq += __shfl_xor(nq, 32, 64);
  if (h == 0) sDen[w][c32] = 1.f / (nq + lp.den_eps);
  __syncthreads();
  bool bad = false;
  uint16_t* o = static_cast<uint16_t*>(lp.o) + row0 * kD;
#pragma unroll
  for (int sl = 0; sl < 16; ++sl) {
    const int m = acc_row(sl, h);
    const int t = kTile * rt + m;
    const float f = sDen[w][m];
    if (t < ntok) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const float ov = O[ib][sl] * f;
        bad |= !isfinite(ov);
        o[static_cast<int64_t>(t) * kD + 32 * ib + c32] = f32_to_bf16(ov);
      }
    }
  }
  if (__any(bad) && lane == 0) atomicOr(lp.chain_info + chain * 4 + kInfoNonfinite, 1);
}

__global__ void __launch_bounds__(256)
vla_lin_stats_kernel(const int32_t* __restrict__ chain_info, int32_t* __restrict__ stats, int chains) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= chains) return;
  stats[c * 4 + 0] = chain_info[c * 4 + kInfoGuard];
  stats[c * 4 + 1] = 0;
  stats[c * 4 + 2] = chain_info[c * 4 + kInfoNonfinite] ? 1 : 0;
  stats[c * 4 + 3] = -1;
}

}  // namespace

hipError_t launch_linear_state(const LinPlan& lp, hipStream_t stream) {
  if (lp.chains <= 0 || lp.ncs <= 0) return hipSuccess;
  const unsigned units = static_cast<unsigned>(lp.chains * lp.ncs);
  hipLaunchKernelGGL(vla_lin_sums_kernel, dim3(units), dim3(kLinThreads), 0, stream, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(lp.chains) * (kD * kD + kD);
  hipLaunchKernelGGL(vla_lin_prefix_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, lp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vla_lin_readout_kernel, dim3(units), dim3(kLinThreads), 0, stream, lp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (lp.stats) {
    hipLaunchKernelGGL(vla_lin_stats_kernel, dim3((lp.chains + 255) / 256), dim3(256), 0, stream, lp.chain_info,
                       lp.stats, lp.chains);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace vla
