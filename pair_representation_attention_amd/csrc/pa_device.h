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

// ---------------------------------------------------------------------------
// Operand-ordered workspace layouts of the bf16 path.  Each 1 KB chunk is the
// register image of one MFMA operand for a wave (lane l owns bytes l*16..+16),
// so a wave copies a chunk with one contiguous 1 KB load.
//   rh = row * H + head;  nb = padded positions / 32
//   q: chunk (rh, pos/32, d/16): lane (pos%32) + 32*((d/8)%2), half d%8
//   k: same with lane pi(pos%32), pi = swap of bits 2 and 3 (the key order
//      that makes the S^T accumulator the K-slot order of the P operand)
//   v: chunk (rh, pos/32, (pos/16)%2): lane d + 32*((pos/8)%2), half pos%8
//   bias (fp16, the S^T accumulator image): chunk (h, q/32, k/32, u):
//      lane (q%32) + 32*g, half s, where for kk = k%32: u = kk/16,
//      g = (kk/8)%2, s = kk%8 -- accumulator register u*8+s of that lane
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int kperm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__device__ __forceinline__ int64_t q_off(int64_t rh, int nb, int pos, int d) {
  return ((((rh * nb + (pos >> 5)) * 2 + (d >> 4)) * 64 + (pos & 31) + 32 * ((d >> 3) & 1)) << 3) + (d & 7);
}
__device__ __forceinline__ int64_t k_off(int64_t rh, int nb, int pos, int d) {
  return ((((rh * nb + (pos >> 5)) * 2 + (d >> 4)) * 64 + kperm(pos & 31) + 32 * ((d >> 3) & 1)) << 3) + (d & 7);
}
__device__ __forceinline__ int64_t v_off(int64_t rh, int nb, int pos, int d) {
  return ((((rh * nb + (pos >> 5)) * 2 + ((pos >> 4) & 1)) * 64 + d + 32 * ((pos >> 3) & 1)) << 3) + (pos & 7);
}
__device__ __forceinline__ int64_t b16_off(int h, int nb, int q, int k) {
  const int kk = k & 31;
  return (((((int64_t)h * nb + (q >> 5)) * nb + (k >> 5)) * 2 + (kk >> 4)) * 64 + (q & 31) + 32 * ((kk >> 3) & 1)) * 8 +
         (kk & 7);
}
// start of chunk `c` of block (a, b): element offsets for the 16-byte-per-lane reads
__device__ __forceinline__ int64_t qkv_chunk(int64_t rh, int nb, int blk, int c) { return ((rh * nb + blk) * 2 + c) * 512; }
__device__ __forceinline__ int64_t b16_chunk(int h, int nb, int qb, int kb, int c) {
  return ((((int64_t)h * nb + qb) * nb + kb) * 2 + c) * 512;
}

// Sum over an aligned group of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace pa
