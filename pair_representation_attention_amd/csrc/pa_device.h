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
// 16-byte global stores of data that only a later kernel reads, after more
// bytes than the caches hold have passed through them (projection planes,
// attention output rows): non-temporal, so the lines do not displace the
// cached K/V, bias and input lines on their way to HBM.
__device__ __forceinline__ void st16(f16* p, const f16x8& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f16x8*>(p));
}
__device__ __forceinline__ void st16(bf16* p, const bf16x8& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// every vector memory operation of this wave (loads, stores, LDS copies) done
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane, global -> LDS: global address sbase + voff (sbase a
// wave-uniform 64-bit base in scalar registers, voff this lane's byte
// offset), LDS address lds_addr + lane*16 (lds_addr wave-uniform).  Issued
// from inline asm so that the compiler neither tracks the copy (it would
// drain every copy in flight before each LDS read) nor orders it: the
// kernels that use it wait for their copies explicitly.  The copy has no
// register result and its address operands are read at issue; one wait
// state separates the M0 write from the copy that reads it.
__device__ __forceinline__ void g2lds16_sbase(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1" ::"v"(voff),
      "s"(sbase), "s"(lds_addr)
      : "memory");
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }   // round to nearest even
__device__ __forceinline__ f16 f2h(float v) { return (f16)v; }       // round to nearest even
// fp16 conversion that saturates at the largest finite fp16 instead of overflowing
__device__ __forceinline__ f16 f2h_sat(float v) { return (f16)__builtin_fminf(__builtin_fmaxf(v, -65504.0f), 65504.0f); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// sigmoid(x) = 1 / (1 + e^-x) with the hardware reciprocal (1 ulp) instead of
// an IEEE division (about ten instructions): exact to fp32 rounding for the
// gate, which is then rounded to fp16 (bf16 path) or used in fp32.  Large
// negative x gives rcp(inf) = 0, large positive x gives 1.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// The bf16 path packs the gate columns of the projection scaled by -log2(e)
// (and the q columns by log2(e)/sqrt(d), d = 32): for such a column,
// t = -x log2(e) and sigmoid(x) = 1 / (1 + 2^t).
__host__ __device__ constexpr float column_scale(int tensor) {
  return tensor == 0 ? 0.2550348616f : tensor == 3 ? -1.4426950409f : 1.0f;
}
__device__ __forceinline__ float sigmoid_from_log2(float t) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

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

// Index checks of the debug build (-DPA_DEBUG).  A failed check sets bit
// `bit` of this source file's flag word with a vector atomic and the kernel
// goes on, so a bad index is reported instead of trapping; the host takes
// (reads and clears) the words after a call (pairattn_debug_status).  Bits:
//   0 K/V copy source   1 bias copy source   2 LDS stage address
//   3 q / gate tile     4 projection store   5 pair-bias store
//   6 keep-bits word    7 staged output tile in LDS
//   8 projection operand slice copy source
// In the release build the checks compile to nothing.
#ifdef PA_DEBUG
static __device__ unsigned int pa_dbg_flags;
#define PA_DCHECK(cond, bit)                                                      \
  do {                                                                            \
    if (!(cond)) atomicOr(&pa_dbg_flags, 1u << (bit));                           \
  } while (0)
// this file's flag word, then cleared (host side)
static inline hipError_t pa_debug_take(unsigned int* out) {
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(pa_dbg_flags), sizeof(unsigned int));
  if (e != hipSuccess) return e;
  const unsigned int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(pa_dbg_flags), &zero, sizeof(unsigned int));
}
#else
#define PA_DCHECK(cond, bit) \
  do {                       \
  } while (0)
static inline hipError_t pa_debug_take(unsigned int* out) {
  *out = 0;
  return hipSuccess;
}
#endif

// Keep bits and key-block range of one row, by one wave:
//   bits[kb]: bit b = key kb*32+b is kept (key < P and mrow[key*ms_k] != 0,
//             or no mask); a ballot of the wave packs the words of two
//             blocks at once
//   range[0] = lo, the first block with a kept key (nkb if none);
//   range[1] = hi, one past the last such block (0 if none)
__device__ __forceinline__ void mask_bits_row(const uint8_t* __restrict__ mrow, int64_t ms_k,
                                              uint32_t* __restrict__ brow, int* __restrict__ range, int P,
                                              int nkb) {
  const int lane = threadIdx.x % kWave;
  int lo = nkb, hi = 0;
  for (int kb0 = 0; kb0 < nkb; kb0 += 2) {
    const int kb = kb0 + (lane >> 5);
    const int key = kb * 32 + (lane & 31);
    const bool keep = kb < nkb && key < P && (mrow == nullptr || mrow[(int64_t)key * ms_k] != 0);
    const uint64_t m = __ballot(keep);
    const uint32_t w0 = (uint32_t)m, w1 = (uint32_t)(m >> 32);
    PA_DCHECK(kb0 < nkb, 6);
    if (lane == 0) brow[kb0] = w0;
    if (lane == 32 && kb0 + 1 < nkb) brow[kb0 + 1] = w1;
    if (w0 != 0u) {
      lo = min(lo, kb0);
      hi = kb0 + 1;
    }
    if (w1 != 0u) {
      lo = min(lo, kb0 + 1);
      hi = kb0 + 2;
    }
  }
  if (lane == 0) {
    range[0] = lo;
    range[1] = hi;
  }
}

// beta . w_b[:, hh] (the pair-bias constant of head hh) by one wave: lane
// partial sums in channel order, then a butterfly over the 64 lanes; every
// lane returns the total.  One function for every place that forms it, so
// that all of them give the same bits.
__device__ __forceinline__ float pair_bias_const(const bf16* __restrict__ beta, const bf16* __restrict__ wb,
                                                 int c_in, int H, int hh) {
  const int lane = threadIdx.x % kWave;
  float acc = 0.0f;
  for (int k = lane; k < c_in; k += kWave) acc += bf2f(beta[k]) * bf2f(wb[(int64_t)k * H + hh]);
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  return acc;
}

// Sum over an aligned group of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace pa
