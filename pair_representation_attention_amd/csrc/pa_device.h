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
__device__ __forceinline__ void st16(f16* p, const f16x8& v) { *reinterpret_cast<f16x8*>(p) = v; }

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
// Along the contraction index x of an operand (head channel d for q, k and
// the gate; key for v and the bias), x = 16t + 8*(e/4) + 4*hg + e%4 sits in
// chunk t, lane half hg, half-word e.  This is the order in which a 32x32
// accumulator holds its rows (register 8t+e of lane half hg is row
// (2t + e/4)*8 + 4*hg + e%4), so
//   * the projection's accumulators, read in register order, are whole
//     16-byte lane slots (each chunk is written as one contiguous 1 KB), and
//   * with keys in natural order in K, the S^T accumulator of Q.K^T is
//     already the K-slot order of the P operand of P.V.
//   q, k, gate: chunk (rh, pos/32, t(d)):   lane (pos%32) + 32*hg(d),  half e(d)
//   v:          chunk (rh, pos/32, t(pos%32)): lane d + 32*hg(pos%32), half e(pos%32)
//   bias (fp16, the S^T accumulator image): chunk (h, q/32, k/32, t(k%32)):
//               lane (q%32) + 32*hg(k%32), half e(k%32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ constexpr int slot_t(int x) { return (x >> 4) & 1; }
__device__ __forceinline__ constexpr int slot_hg(int x) { return (x >> 2) & 1; }
__device__ __forceinline__ constexpr int slot_e(int x) { return (((x >> 3) & 1) << 2) | (x & 3); }
// the index x held by half-word e of lane half hg in chunk t
__device__ __forceinline__ constexpr int slot_x(int t, int hg, int e) { return 16 * t + 8 * (e >> 2) + 4 * hg + (e & 3); }

__device__ __forceinline__ int64_t q_off(int64_t rh, int nb, int pos, int d) {
  return ((((rh * nb + (pos >> 5)) * 2 + slot_t(d)) * 64 + (pos & 31) + 32 * slot_hg(d)) << 3) + slot_e(d);
}
__device__ __forceinline__ int64_t k_off(int64_t rh, int nb, int pos, int d) { return q_off(rh, nb, pos, d); }
__device__ __forceinline__ int64_t v_off(int64_t rh, int nb, int pos, int d) {
  const int x = pos & 31;
  return ((((rh * nb + (pos >> 5)) * 2 + slot_t(x)) * 64 + d + 32 * slot_hg(x)) << 3) + slot_e(x);
}
// bias of nbq query blocks by nbk key blocks (both nb for the square bias)
__device__ __forceinline__ int64_t b16_off(int h, int nbq, int nbk, int q, int k) {
  const int x = k & 31;
  return (((((int64_t)h * nbq + (q >> 5)) * nbk + (k >> 5)) * 2 + slot_t(x)) * 64 + (q & 31) + 32 * slot_hg(x)) * 8 +
         slot_e(x);
}
// start of chunk `c` of block (a, b): element offsets for the 16-byte-per-lane reads
__device__ __forceinline__ int64_t qkv_chunk(int64_t rh, int nb, int blk, int c) { return ((rh * nb + blk) * 2 + c) * 512; }
__device__ __forceinline__ int64_t b16_chunk(int h, int nbq, int nbk, int qb, int kb, int c) {
  return ((((int64_t)h * nbq + qb) * nbk + kb) * 2 + c) * 512;
}

// Sum over an aligned group of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace pa
