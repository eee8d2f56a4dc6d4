// Shared device helpers for the VLA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

// ---- bfloat16 storage: raw 16-bit patterns ---------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two values rounded to bf16 (nearest, ties to even; NaN stays NaN) and
// packed, a in the low half: one v_cvt_pk_bf16_f32.
typedef float vla_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 vla_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((vla_f32x2{a, b}), vla_bf16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// ---- cross-lane reductions (DPP within rows of 16 lanes) -------------------
__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int CTRL>
__device__ __forceinline__ float dpp_read(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16

// Sum over groups of G consecutive lanes (G = 4, 8 or 16); every lane of a
// group receives the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G >= 2) x += dpp_read<kQuadSwap1>(x);
  if constexpr (G >= 4) x += dpp_read<kQuadSwap2>(x);
  if constexpr (G >= 8) x += dpp_read<kRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_read<kRowMirror>(x);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane i gets x_0 + ... + x_i):
// Hillis-Steele inside rows of 16 lanes with DPP row shifts, then the row
// totals carried across rows with the gfx9 row broadcasts (lane 15 of each
// row into rows 1 and 3, then lane 31 into rows 2 and 3).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
__device__ __forceinline__ float wave_incl_scan(float x, int /*lane*/) {
  x += dpp_read<kRowShr1>(x);
  x += dpp_read<kRowShr2>(x);
  x += dpp_read<kRowShr4>(x);
  x += dpp_read<kRowShr8>(x);
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast15, 0xA, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast31, 0xC, 0xF, false));
  return x;
}

// Sum over the whole wave; the result is wave-uniform and identical on every
// wave that reduces the same values (fixed order).
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

// ---- raw buffer access -----------------------------------------------------
// A buffer resource (gfx9 layout: 32-bit dwords, no swizzle, no stride) over
// `bytes` bytes at a wave-uniform base.  Each access takes a per-lane byte
// offset, so unrolled loops keep one offset register plus immediates instead
// of one 64-bit address per access.  Loads at or past `bytes` return zero and
// stores there are dropped.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float buf_load_elem(__amdgpu_buffer_rsrc_t r, int off, const float*) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_elem(__amdgpu_buffer_rsrc_t r, int off, const uint16_t*) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, int off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}

}  // namespace vla
