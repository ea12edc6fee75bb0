// Device-side helpers shared by the gfx950 kernels of the pair-attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// 32x32x16 bf16 MFMA, fp32 accumulate: D = A(32x16) * B(16x32) + C.
// Lane l holds row/column (l % 32) of A/B and eight consecutive K-slots of
// half (l / 32); both operands use the same K-slot order, so any consistent
// assignment of the K index to (half, slot) gives the same product.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Same shape with fp16 operands (same issue rate on gfx950, 3 more mantissa bits).
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register j of a lane in half g
// (the column is lane % 32): four consecutive rows per group of four
// registers, groups 8 rows apart, the second half offset by 4.
__device__ __forceinline__ constexpr int acc_row(int j, int g) { return (j >> 2) * 8 + g * 4 + (j & 3); }

__device__ __forceinline__ bf16x8 ld16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f16x8 ld16(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ void st8(bf16* p, const bf16x4& v) { *reinterpret_cast<bf16x4*>(p) = v; }
__device__ __forceinline__ void st8(f16* p, const f16x4& v) { *reinterpret_cast<f16x4*>(p) = v; }

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }   // round to nearest even
__device__ __forceinline__ f16 f2h(float v) { return (f16)v; }       // round to nearest even
// fp16 conversion that saturates at the largest finite fp16 instead of overflowing
__device__ __forceinline__ f16 f2h_sat(float v) { return (f16)__builtin_fminf(__builtin_fmaxf(v, -65504.0f), 65504.0f); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over an aligned group of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace pa
