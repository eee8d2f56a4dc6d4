// Penalty-direction projection u_{row,i} = normalize(W_u[i] k_raw[row]) on the
// gfx950 matrix cores.
//
// Source: "Variational Linear Attention (VLA)" README, v3 notes item 2
// (u_t = normalize(W_u k_t^raw)); normalize(x) = x / max(|x|_2, 1e-12).
//
// As a GEMM: Out[rows, r*d] = K_raw[rows, d] . W^T with W = W_u viewed as
// [r*d, d]; K = d is short, so the kernel is bound by streaming k_raw in and
// u out of HBM.  A wave computes tiles of 32 rows x d columns of one direction
// with 32x32 MFMA tiles (bf16: 32x32x16, fp32: 32x32x2, both accumulating in
// fp32) and normalises them in the epilogue, after the tile has gone through
// the wave's LDS into pieces of whole rows (see finish_tile).  The bf16
// kernel holds one direction's W in registers over a run of row tiles; the
// fp32 kernel (small workloads) keeps its k_raw rows across the r directions.
//
// MFMA 32x32 accumulator layout: lane l holds column l % 32 of the tile and,
// in accumulator slot a, row 8*(a/4) + 4*(l/32) + a%4.  Operand A holds row
// l % 32 and operand B column l % 32; both take the same k slice per lane, so
// the k assignment inside a lane only has to agree between A and B.
#include "vla_common.h"
#include "vla_kernels.h"

namespace vla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProjWaves = 4;

// LDS row stride (floats) of a wave's 32 x D staging tile.
template <int D>
constexpr int stage_ld() { return D + 4; }

// Normalises the wave's 32 rows of direction i, staged raw in the wave's LDS
// tile, and writes them: each lane takes pieces of eight consecutive values of
// a row (the lanes of one row are D/8 consecutive lanes), so a row's sum of
// squares is one short DPP group sum and each lane normalises and stores
// whole 16-byte (bf16) or 32-byte (fp32) pieces.  (Normalising in the
// accumulator layout took a 32-lane reduction per accumulator slot, 16 per
// tile.)
template <int D, typename Store>
__device__ __forceinline__ void normalize_rows(int lane, const float* tile, Store&& store) {
  asm volatile("" ::: "memory");   // one wave's LDS operations complete in order
  constexpr int LD = stage_ld<D>();
  constexpr int PPR = D / 8;       // pieces of eight values per row
  static_assert((32 * PPR) % 64 == 0 && 64 % PPR == 0, "whole rows per lane group");
#pragma unroll
  for (int it = 0; it < 32 * PPR / 64; ++it) {
    const int c = lane + 64 * it;
    const int rl = c / PPR, pc = c % PPR;
    const float4 x0 = *reinterpret_cast<const float4*>(tile + rl * LD + pc * 8);
    const float4 x1 = *reinterpret_cast<const float4*>(tile + rl * LD + pc * 8 + 4);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
    ss = group_sum<PPR>(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= inv;
    store(rl, pc, v);
  }
  asm volatile("" ::: "memory");   // the reads finish before the next tile's writes
}

// Eight output values as 16 (bf16) or 32 (fp32) bytes.
template <typename TOut>
__device__ __forceinline__ void put8(TOut* dst, const float (&v)[8]) {
  if constexpr (sizeof(TOut) == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
}
template <typename TOut>
__device__ __forceinline__ void buf_put8(__amdgpu_buffer_rsrc_t rs, int off, const float (&v)[8]) {
  if constexpr (sizeof(TOut) == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                 __float_as_uint(v[3])}, rs, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                                 __float_as_uint(v[7])}, rs, off + 16, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                 pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])}, rs, off, 0, 0);
  }
}

// Column block nb of the raw tile into the wave's LDS staging tile.
template <int D>
__device__ __forceinline__ void stage_block(const f32x16& acc, int nb, int lane, float* tile) {
  constexpr int LD = stage_ld<D>();
  const int col = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int s = 0; s < 16; ++s) tile[(8 * (s / 4) + 4 * hi + (s % 4)) * LD + nb * 32 + col] = acc[s];
}

// The whole raw tile (D / 32 accumulator blocks) staged, normalised and stored.
template <int D, typename TOut>
__device__ __forceinline__ void finish_tile(f32x16 (&acc)[D / 32], int64_t row_base, int64_t rows, int r,
                                            int i, int lane, TOut* u, float* tile) {
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) stage_block<D>(acc[nb], nb, lane, tile);
  normalize_rows<D>(lane, tile, [&](int rl, int pc, const float (&v)[8]) {
    const int64_t row = row_base + rl;
    if (row < rows) put8<TOut>(u + (row * r + i) * D + pc * 8, v);
  });
}

// Consecutive 32-row tiles per wave of the bf16 kernel (its W slice is loaded
// once per run of tiles).
template <int D>
constexpr int proj_tiles_per_wave() { return D >= 128 ? 16 : 8; }

// bf16 inputs: v_mfma_f32_32x32x16_bf16, 8 bf16 of k per lane per tile.  Each
// wave owns one direction i and a run of consecutive 32-row tiles, and keeps
// W_i (D x D, as B operands) in its registers for the whole run: W is read
// once per run rather than once per tile (at d = 128, r = 4 the per-tile
// reloads came to 128 KiB of cache reads per 32 rows, several times the
// kernel's HBM bytes).  Consecutive waves take the r directions of the same
// rows, so a workgroup's k_raw rows are shared through the cache.  The next
// tile's k_raw rows are loaded while the current tile is normalised and stored.
template <int D, typename TOut>
__global__ void __launch_bounds__(64 * kProjWaves) __attribute__((amdgpu_waves_per_eu(2)))
project_u_bf16_kernel(int64_t rows, int r, int64_t nruns, const uint16_t* __restrict__ W,
                      const uint16_t* __restrict__ kraw, TOut* __restrict__ u) {
  constexpr int KB = D / 16, NB = D / 32, TPW = proj_tiles_per_wave<D>();
  constexpr int NP = NB >= 2 ? 2 : 1;   // column blocks per accumulation round
  __shared__ float tiles[kProjWaves][32 * stage_ld<D>()];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kProjWaves + w;
  const int64_t run = g / r;
  const int i = static_cast<int>(g - run * r);
  // Waves past the last run have nothing to do (the kernel has no workgroup
  // barrier: each wave stages through its own LDS tile).
  if (run >= nruns) return;
  const int koff = 8 * (lane >> 5);

  bf16x8 b[NB][KB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint16_t* wrow = W + (static_cast<int64_t>(i) * D + nb * 32 + (lane & 31)) * D + koff;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) b[nb][kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wrow + kb * 16));
  }
  // The run's rows through buffer resources over just those rows: loads past
  // the last row read zeros and stores there are dropped, so the loop has no
  // branches and its waits count only the k_raw loads it needs (stores also
  // count toward vmcnt here).
  const int64_t row0 = run * TPW * 32;
  const int64_t nrow = rows - row0 < TPW * 32 ? rows - row0 : TPW * 32;
  const int ntl = static_cast<int>((nrow + 31) / 32);
  const auto rk = make_rsrc(kraw + row0 * D, static_cast<int>(nrow * D * 2));
  const auto ru = make_rsrc(u + (row0 * r + i) * D, static_cast<int>(((nrow - 1) * r + 1) * D * sizeof(TOut)));
  bf16x8 a[KB];
  auto load_a = [&](int tl) {
    const int off = ((tl * 32 + (lane & 31)) * D + koff) * 2;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) a[kb] = __builtin_bit_cast(bf16x8, buf_load16(rk, off + 32 * kb));
  };
  load_a(0);
  for (int tl = 0; tl < ntl; ++tl) {
    // Two column blocks at a time (two independent accumulation chains),
    // staged as soon as they are done: two accumulator tiles live beside W_i.
#pragma unroll
    for (int nb = 0; nb < NB; nb += NP) {
      f32x16 acc[NP];
#pragma unroll
      for (int j = 0; j < NP; ++j)
        acc[j] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < NP; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], b[nb + j][kb], acc[j], 0, 0, 0);
      if (nb + NP == NB) load_a(tl + 1);   // past the run: zeros, unused
#pragma unroll
      for (int j = 0; j < NP; ++j) stage_block<D>(acc[j], nb + j, lane, tiles[w]);
    }
    normalize_rows<D>(lane, tiles[w], [&](int rl, int pc, const float (&v)[8]) {
      buf_put8<TOut>(ru, (((tl * 32 + rl) * r) * D + pc * 8) * static_cast<int>(sizeof(TOut)), v);
    });
  }
}

// fp32 inputs: v_mfma_f32_32x32x2_f32, one float of k per lane per tile.
template <int D, typename TOut>
__global__ void __launch_bounds__(64 * kProjWaves)
project_u_f32_kernel(int64_t rows, int r, const float* __restrict__ W, const float* __restrict__ kraw,
                     TOut* __restrict__ u) {
  constexpr int KB = D / 2;
  __shared__ float tiles[kProjWaves][32 * stage_ld<D>()];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row_base = (static_cast<int64_t>(blockIdx.x) * kProjWaves + w) * 32;
  const int64_t arow = row_base + (lane & 31);
  const int koff = lane >> 5;

  float a[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) a[kb] = (arow < rows) ? kraw[arow * D + 2 * kb + koff] : 0.f;
  for (int i = 0; i < r; ++i) {
    f32x16 acc[D / 32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      acc[nb] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float* wrow = W + (static_cast<int64_t>(i) * D + nb * 32 + (lane & 31)) * D + koff;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[kb], wrow[2 * kb], acc[nb], 0, 0, 0);
    }
    finish_tile<D, TOut>(acc, row_base, rows, r, i, lane, u, tiles[w]);
  }
}

// d = 16 is narrower than one 32-column tile: plain fp32 FMAs, one row per
// thread (the tiny head size only appears in small parity workloads).
template <typename TIn, typename TOut>
__global__ void __launch_bounds__(256)
project_u_d16_kernel(int64_t rows, int r, const TIn* __restrict__ W, const TIn* __restrict__ kraw,
                     TOut* __restrict__ u) {
  constexpr int D = 16;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= rows) return;
  float kv[D];
#pragma unroll
  for (int m = 0; m < D; ++m) kv[m] = Elem<TIn>::load(kraw + row * D + m);
  for (int i = 0; i < r; ++i) {
    float x[D];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < D; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < D; ++m) acc = fmaf(Elem<TIn>::load(W + (i * D + j) * D + m), kv[m], acc);
      x[j] = acc;
      ss = fmaf(acc, acc, ss);
    }
    const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int j = 0; j < D; ++j) Elem<TOut>::store(u + (row * r + i) * D + j, x[j] * inv);
  }
}

template <typename TIn, typename TOut, int D>
hipError_t launch_proj(int64_t rows, int r, const void* W, const void* kraw, void* u, hipStream_t s) {
  if constexpr (D == 16) {
    const unsigned grid = static_cast<unsigned>((rows + 255) / 256);
    hipLaunchKernelGGL((project_u_d16_kernel<TIn, TOut>), dim3(grid), dim3(256), 0, s, rows, r,
                       static_cast<const TIn*>(W), static_cast<const TIn*>(kraw), static_cast<TOut*>(u));
  } else {
    if constexpr (sizeof(TIn) == 2) {
      constexpr int TPW = proj_tiles_per_wave<D>();
      const int64_t nruns = ((rows + 31) / 32 + TPW - 1) / TPW;
      const unsigned grid = static_cast<unsigned>((nruns * r + kProjWaves - 1) / kProjWaves);
      hipLaunchKernelGGL((project_u_bf16_kernel<D, TOut>), dim3(grid), dim3(64 * kProjWaves), 0, s, rows, r, nruns,
                         static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(kraw), static_cast<TOut*>(u));
    } else {
      const unsigned grid = static_cast<unsigned>((rows + 32 * kProjWaves - 1) / (32 * kProjWaves));
      hipLaunchKernelGGL((project_u_f32_kernel<D, TOut>), dim3(grid), dim3(64 * kProjWaves), 0, s, rows, r,
                         static_cast<const float*>(W), static_cast<const float*>(kraw), static_cast<TOut*>(u));
    }
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t dispatch_proj(int64_t rows, int d, int r, const void* W, const void* kraw, void* u, hipStream_t s) {
  switch (d) {
    case 16: return launch_proj<TIn, TOut, 16>(rows, r, W, kraw, u, s);
    case 32: return launch_proj<TIn, TOut, 32>(rows, r, W, kraw, u, s);
    case 64: return launch_proj<TIn, TOut, 64>(rows, r, W, kraw, u, s);
    case 128: return launch_proj<TIn, TOut, 128>(rows, r, W, kraw, u, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_project_u(int64_t rows, int d, int r, bool in_bf16, bool out_bf16, const void* W,
                            const void* kraw, void* u, hipStream_t s) {
  if (in_bf16) {
    return out_bf16 ? dispatch_proj<uint16_t, uint16_t>(rows, d, r, W, kraw, u, s)
                    : dispatch_proj<uint16_t, float>(rows, d, r, W, kraw, u, s);
  }
  return out_bf16 ? dispatch_proj<float, uint16_t>(rows, d, r, W, kraw, u, s)
                  : dispatch_proj<float, float>(rows, d, r, W, kraw, u, s);
}

}  // namespace vla
