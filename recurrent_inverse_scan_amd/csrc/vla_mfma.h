// Matrix-core helpers shared by the gfx950 kernels: the 32x32x16 bf16 MFMA,
// its register layouts, and fp32 operands split into three bf16 terms so the
// bf16 matrix cores deliver fp32-grade products.
//
// v_mfma_f32_32x32x16_bf16, wave64, D = A B + C with A 32x16, B 16x32:
//   A operand  lane l holds A[l & 31][8 (l >> 5) + e],  e = 0..7
//   B operand  lane l holds B[8 (l >> 5) + e][l & 31]
//   C / D      lane l holds D[8 (s >> 2) + 4 (l >> 5) + (s & 3)][l & 31], s = 0..15
// The contraction index may be permuted freely as long as both operands use
// the same permutation; that lets an accumulator tile serve directly as the
// B operand (contracting over its rows) or, read as the A operand, as its
// own transpose.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 zero16() {
  return f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator slot s in lane half h (see the layout above).
__host__ __device__ constexpr int acc_row(int s, int h) { return 8 * (s >> 2) + 4 * h + (s & 3); }

// x = t1 + t2 + t3 exactly, each term a bf16: t1 is x with the low 16 bits
// of its encoding cleared, r = x - t1 (exact: the low 16 significand bits),
// t2 is r cleared the same way and t3 = r - t2 holds at most 8 significant
// bits, so it is a bf16 as well.  Each term is the upper half of an fp32
// encoding; byte permutes pack two of them per word.
struct Split3 {
  bf16x8 t1, t2, t3;
};
__device__ __forceinline__ uint32_t pack_hi16(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}
__device__ __forceinline__ Split3 split3(const float (&x)[8]) {
#pragma clang fp contract(off)   // x is what the caller rounded, not an exact product
  uint32_t a[8], r[8], c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __float_as_uint(x[e]);
    const float rf = x[e] - __uint_as_float(a[e] & 0xffff0000u);
    r[e] = __float_as_uint(rf);
    c[e] = __float_as_uint(rf - __uint_as_float(r[e] & 0xffff0000u));
  }
  Split3 s;
  s.t1 = __builtin_bit_cast(bf16x8, make_uint4(pack_hi16(a[0], a[1]), pack_hi16(a[2], a[3]), pack_hi16(a[4], a[5]),
                                               pack_hi16(a[6], a[7])));
  s.t2 = __builtin_bit_cast(bf16x8, make_uint4(pack_hi16(r[0], r[1]), pack_hi16(r[2], r[3]), pack_hi16(r[4], r[5]),
                                               pack_hi16(r[6], r[7])));
  s.t3 = __builtin_bit_cast(bf16x8, make_uint4(pack_hi16(c[0], c[1]), pack_hi16(c[2], c[3]), pack_hi16(c[4], c[5]),
                                               pack_hi16(c[6], c[7])));
  return s;
}

// Slots 8 g .. 8 g + 7 of an accumulator tile (one k step of 16 of its rows),
// optionally scaled, as a three-term split.
__device__ __forceinline__ Split3 split_slots(const f32x16& x, int g, float scale = 1.f) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[8 * g + e] * scale;
  return split3(v);
}

// acc += A B with A and B given as three-term splits (terms of order >= 3 dropped).
__device__ __forceinline__ f32x16 mma_split(const Split3& a, const Split3& b, f32x16 acc) {
  acc = mfma_bf16(a.t2, b.t2, acc);
  acc = mfma_bf16(a.t3, b.t1, acc);
  acc = mfma_bf16(a.t1, b.t3, acc);
  acc = mfma_bf16(a.t2, b.t1, acc);
  acc = mfma_bf16(a.t1, b.t2, acc);
  return mfma_bf16(a.t1, b.t1, acc);
}
// acc += A B with A exact in bf16.
__device__ __forceinline__ f32x16 mma_split(bf16x8 a, const Split3& b, f32x16 acc) {
  acc = mfma_bf16(a, b.t3, acc);
  acc = mfma_bf16(a, b.t2, acc);
  return mfma_bf16(a, b.t1, acc);
}
// acc += A B with B exact in bf16.
__device__ __forceinline__ f32x16 mma_split(const Split3& a, bf16x8 b, f32x16 acc) {
  acc = mfma_bf16(a.t3, b, acc);
  acc = mfma_bf16(a.t2, b, acc);
  return mfma_bf16(a.t1, b, acc);
}
// acc += A B with both operands exact in bf16.
__device__ __forceinline__ f32x16 mma_split(bf16x8 a, bf16x8 b, f32x16 acc) { return mfma_bf16(a, b, acc); }

}  // namespace vla
