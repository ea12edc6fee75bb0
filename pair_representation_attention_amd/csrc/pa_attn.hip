// Flash-style pair-biased attention for gfx950 (bf16 interface, fp16 MFMA
// operands, fp32 softmax), with the gate and the output projection fused in.
//
// Problem ("row attention"): nrows independent rows of P positions; in row r
// query p attends over keys k of the same row with
//   logit = q[r,p].k[r,k] / sqrt(d) + bias[p][k]   (bias shared by all rows)
// keys masked per (row, key).  The caller's orientation (starting node,
// ending node, MSA rows) is folded into the workspace and the strides.
//
// Work decomposition
//   unit = 32 queries x 32 keys of one (row, head)
//   workgroup = 8 waves covering RWG rows x QWG query blocks x H heads
//     H = 4: RWG = 2, QWG = 4, wave = (head, query-block pair), 2 x 2 units per key block
//     H = 8: RWG = 1, QWG = 3, wave = head (all 3 query blocks), 1 x 3 units per key block
//   per key block and unit (S^T is keys x queries, log2 units):
//     S^T = K Q^T + C      two MFMAs; C = the fp16 bias tile widened to fp32
//                          by four 4x4x4 MFMAs (shared by the workgroup's rows)
//     p = exp2(S - m)      rounded to fp16 (the P operand); l += sum of p
//                          (four 4x4x4 MFMAs against ones on the pipelined
//                          sweep, fp16 dot products on the generic one)
//     O^T += V^T P^T       two MFMAs
//   Softmax shift m per (row, query): a first sweep uses m = 0 with no
//   per-unit test; afterwards every l must be finite (no fp16 weight
//   overflowed) and at least 1 on rows with a kept key (the largest weights
//   are normal fp16 numbers).  Where that fails anywhere in the workgroup,
//   it sweeps again choosing m on the row's first block with a kept key and
//   raising it (O and l rescaled) whenever a block sum passes 2^15.  Exact in
//   real arithmetic for any shift.
// Memory path: K/V tiles of the workgroup's rows (each shared by the two
// waves of a head) and the bias tiles of its query blocks are copied per key
// block with global_load_lds_dwordx4 into LDS rings (K/V three stages deep,
// bias two).  The workspace is stored in MFMA operand order (pa_device.h):
// every copy is a contiguous 1 KB read, every LDS read a conflict-free
// ds_read_b128, and the S^T accumulator (rows = keys in natural order) is
// already the K-slot order of the P operand.
// Bytes moved per unit: 4 KB K/V / 4 query blocks + 2 KB bias / 2 rows (H = 4),
// 4 KB K/V / 3 query blocks + 2 KB bias (H = 8).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// 16 bytes per lane, global -> LDS at lds_base + lane*16 (lds_base
// wave-uniform), issued from inline asm for the staging rings.  (The
// compiler tracks every LDS-DMA copy of its own builtin in one slot and would
// drain all copies in flight before each LDS read; the rings keep their
// order explicitly instead: a counted wait before the barrier of each key
// block, a full drain before the LDS is reused.)  The copy has no register
// result and its address operands are read at issue; one wait state
// separates the M0 write from the copy that reads it.
__device__ __forceinline__ void g2lds16_ring(const void* gsrc, char* lds_base) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_void_t*)lds_base;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off" ::"v"(gsrc),
      "s"(lds_addr)
      : "memory");
}

// (g2lds16_sbase of pa_device.h is the same copy from a wave-uniform 64-bit
// base in scalar registers plus a 32-bit per-lane byte offset, with no vector
// address arithmetic per copy.)

// s_waitcnt vmcnt(N) through the builtin (gfx9 immediate layout: vmcnt in
// bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] at their no-wait
// maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) (LDS reads and scalar loads), vmcnt and expcnt at their no-wait maxima
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

__device__ __forceinline__ f16x8 lds_f16x8(const char* p) { return *reinterpret_cast<const f16x8*>(p); }

typedef float f32x8 __attribute__((ext_vector_type(8)));

// v_mfma_f32_4x4x4_16b_f16: 16 independent 4x4x4 products.  Lane 4b+i holds
// row i of A_b and lane 4b+j column j of B_b (4 fp16 each, k = 0..3); output
// register i of lane 4b+j is D_b[i][j].  So with A = the lane's unit vector
// e_(lane%4) every lane gets its own four B values widened to fp32 (exact),
// and with A = ones every output register of a lane gets the fp32 sum of its
// own four B values.  Either way only 1/16 of the multiplier work of a 32x32
// product, on the matrix cores instead of the VALU.
__device__ __forceinline__ f32x4 mfma4(const f16x4& a, const f16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 lo4(const f16x8& v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ f16x4 hi4(const f16x8& v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

// The fp16 bias tile of a lane (the 16 values of its S^T accumulator slots)
// widened to the fp32 C operand of the logits product: four 4x4x4 products
// against the lane's unit vector `ident`.
__device__ __forceinline__ f32x16 widen_bias(const f16x8& b0, const f16x8& b1, const f16x4& ident) {
  const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x8 c01 = __builtin_shufflevector(mfma4(ident, lo4(b0), z4), mfma4(ident, hi4(b0), z4), 0, 1, 2, 3, 4, 5,
                                            6, 7);
  const f32x8 c23 = __builtin_shufflevector(mfma4(ident, lo4(b1), z4), mfma4(ident, hi4(b1), z4), 0, 1, 2, 3, 4, 5,
                                            6, 7);
  return __builtin_shufflevector(c01, c23, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// The same with accumulator inputs m (registers in the order of the S^T
// accumulator): every output is its bias value plus m, so -inf in m masks a
// key in the logits product that takes this as its C operand.
__device__ __forceinline__ f32x16 widen_bias_acc(const f16x8& b0, const f16x8& b1, const f16x4& ident,
                                                 const f32x16& m) {
  const f32x8 c01 = __builtin_shufflevector(mfma4(ident, lo4(b0), __builtin_shufflevector(m, m, 0, 1, 2, 3)),
                                            mfma4(ident, hi4(b0), __builtin_shufflevector(m, m, 4, 5, 6, 7)), 0, 1,
                                            2, 3, 4, 5, 6, 7);
  const f32x8 c23 = __builtin_shufflevector(mfma4(ident, lo4(b1), __builtin_shufflevector(m, m, 8, 9, 10, 11)),
                                            mfma4(ident, hi4(b1), __builtin_shufflevector(m, m, 12, 13, 14, 15)), 0,
                                            1, 2, 3, 4, 5, 6, 7);
  return __builtin_shufflevector(c01, c23, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// Lane mask of accumulator register j (key k0 = (j/4)*8 + j%4 in lane half 0,
// key k0 + 4 in lane half 1) from a block's keep bits: each half is bit k0
// (or k0 + 4) sign-extended to 32 bits, one scalar bit-field extract each.
// Volatile, so that the compiler computes each mask where it is used instead
// of keeping all 16 of a block alive in scalar registers across the units.
template <int K0>
__device__ __forceinline__ uint64_t key_lanes(uint32_t bits) {
  uint32_t lo, hi;
  // early-clobber outputs: the first is written before the second
  // instruction reads `bits`, so neither may share its register
  asm volatile("s_bfe_i32 %0, %2, %3\n\ts_bfe_i32 %1, %2, %4"
               : "=&s"(lo), "=&s"(hi)
               : "s"(bits), "i"(K0 | (1 << 16)), "i"((K0 + 4) | (1 << 16)));
  return ((uint64_t)hi << 32) | lo;
}
template <int J>
__device__ __forceinline__ float keep_reg(float s, uint32_t bits);

// s where bit `lane` of the wave-uniform mask is set, else -inf: one
// v_cndmask with the mask as its scalar condition.  (A compiler builtin, not
// inline asm, so that the wait states after the MFMA producing s are known.)
__device__ __forceinline__ float keep_or_neg_inf(float s, uint64_t lanes) {
  return __builtin_amdgcn_inverse_ballot_w64(lanes) ? s : -__builtin_inff();
}
// accumulator register J of a unit, -inf where its key is masked
template <int J>
__device__ __forceinline__ float keep_reg(float s, uint32_t bits) {
  return keep_or_neg_inf(s, key_lanes<(J >> 2) * 8 + (J & 3)>(bits));
}
// all 16 registers of a unit's S^T accumulator
__device__ __forceinline__ void keep_unit(f32x16& S, uint32_t bits) {
  S[0] = keep_reg<0>(S[0], bits);
  S[1] = keep_reg<1>(S[1], bits);
  S[2] = keep_reg<2>(S[2], bits);
  S[3] = keep_reg<3>(S[3], bits);
  S[4] = keep_reg<4>(S[4], bits);
  S[5] = keep_reg<5>(S[5], bits);
  S[6] = keep_reg<6>(S[6], bits);
  S[7] = keep_reg<7>(S[7], bits);
  S[8] = keep_reg<8>(S[8], bits);
  S[9] = keep_reg<9>(S[9], bits);
  S[10] = keep_reg<10>(S[10], bits);
  S[11] = keep_reg<11>(S[11], bits);
  S[12] = keep_reg<12>(S[12], bits);
  S[13] = keep_reg<13>(S[13], bits);
  S[14] = keep_reg<14>(S[14], bits);
  S[15] = keep_reg<15>(S[15], bits);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Sum of the 16 fp16 softmax weights of a lane (the values the P.V product
// uses), accumulated in fp32 by dot products with (1, 1).
__device__ __forceinline__ float sum16_f16(const f16x8& a, const f16x8& b) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
  float s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), one, 0.0f, false);
  float s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 0, 1), one, 0.0f, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), one, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 2, 3), one, s1, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), one, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 4, 5), one, s1, false);
  s0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), one, s0, false);
  s1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(b, b, 6, 7), one, s1, false);
  return s0 + s1;
}

template <int H>
struct AttnShape {
  // query blocks per wave: 3 at H = 8 (fewer workgroups, so fewer reloads of
  // K/V and of the 256-wide W_o per query; its 48 KB bias stages leave room
  // for a K/V ring two stages deep)
  static constexpr int QW = H == 8 ? 3 : 2;
  static constexpr int QG = 8 / H;                 // query-block groups per workgroup
  static constexpr int QWG = QW * QG;              // query blocks per workgroup
  // rows per workgroup (every wave does all): 2 at H = 4; 1 at H = 8, so
  // that a K/V stage is 32 KB and the ring three stages deep
  static constexpr int RWG = H == 4 ? 2 : 1;
  static constexpr int KV_TILE = 4096;             // K (2 chunks) + V (2 chunks) of one (row, head)
  static constexpr int B_TILE = 2048;              // fp16 bias tile (2 chunks) of one (query block, head)
  static constexpr int KV_STAGE = RWG * H * KV_TILE;   // 32 KB
  static constexpr int B_STAGE = QWG * H * B_TILE;     // 32 KB
  // K/V ring of NKV stages (NKV-1 key blocks ahead), bias ring of 2 (one
  // block ahead): 3 x 32 + 2 x 32 KB at H = 4, 2 x 32 + 2 x 48 KB at H = 8
  static constexpr int NKV = 3 * KV_STAGE + 2 * B_STAGE <= 160 * 1024 ? 3 : 2;
  static constexpr int LDS_KV = NKV * KV_STAGE;
  static constexpr int LDS_B = 2 * B_STAGE;
  static constexpr int N_KV_CH = RWG * H * 4;      // 1 KB copies per stage
  static constexpr int N_B_CH = QWG * H * 2;
  static constexpr int NCW = N_KV_CH / 8;          // K/V copies per wave and stage
  static constexpr int NCB = N_B_CH / 8;           // bias copies per wave and stage
  static_assert(N_KV_CH % 8 == 0 && N_B_CH % 8 == 0, "copies split evenly over the 8 waves");
  static_assert(LDS_KV + LDS_B <= 160 * 1024, "LDS");
  // Block kb needs bias stage kb (issued at the top of kb-1, before that
  // block's K/V copies) and K/V stage kb (issued NKV-1 blocks ago): the K/V
  // copies of block kb-1 may stay in flight when the ring is 3 deep.
  static constexpr int WAIT = NKV == 3 ? NCW : 0;
};

// MODE 0: one pass over all keys, gate and output projection into `out`.
// MODE 1: one shard of keys (nbq_in query blocks, Pk_in keys in nbk_in
//         blocks); the per-head output o = O / l and its log-sum-exp
//         lse = ln l + m ln 2 go to o_part [nrows][P][H*32] and lse_part
//         [nrows][H][P].  MODE 2: merged into the o_part / lse_part already
//         there (log-sum-exp weights).
template <int H, int C_OUT, bool HAS_MASK, int MODE>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(
    const f16* __restrict__ q_ws, const f16* __restrict__ k_ws, const f16* __restrict__ v_ws,
    const f16* __restrict__ g_ws, const f16* __restrict__ bias, const uint32_t* __restrict__ mask_bits,
    const int* __restrict__ mask_range, const f16* __restrict__ woT, const bf16* __restrict__ b_o, bf16* __restrict__ out, int64_t os_r,
    int64_t os_p, int nrows, int P, int Pp, int n_qg, int n_rg, int qgb, int nbq_in, int Pk_in, int nbk_in,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  static_assert(MODE >= 0 && MODE <= 2, "mode");
  static_assert(H == 4 || H == 8, "4 or 8 heads");
  using SH = AttnShape<H>;
  constexpr int HD = H * 32;
  constexpr int QW = SH::QW, RW = SH::RWG;
  __shared__ __attribute__((aligned(1024))) char kv_lds[SH::LDS_KV];
  __shared__ __attribute__((aligned(1024))) char b_lds[SH::LDS_B];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int h = wave % H;
  const int qgrp = wave / H;
  // A operands of the 4x4x4 products: this lane's unit vector, and ones
  f16x4 ident4, ones4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ident4[e] = (f16)(e == (lane & 3) ? 1.0f : 0.0f);
    ones4[e] = (f16)1.0f;
  }

  // XCD-aware tile order: consecutive workgroup ids are spread round-robin
  // over the 8 XCDs, so give each XCD a contiguous range of logical tiles,
  // and walk tiles in super-columns of QGB query groups (chosen by the host),
  // so the workgroups that run together on one XCD share rows (K/V) and
  // query groups (bias).
  int L = blockIdx.x;
  {
    const int n = gridDim.x, per = n / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
  }
  const int QGB = qgb;
  const int sc = L / (n_rg * QGB);
  const int sc_w = min(QGB, n_qg - sc * QGB);
  const int rem = L - sc * n_rg * QGB;
  const int rgi = rem / sc_w;
  const int qg = sc * QGB + rem % sc_w;
  const int r0 = rgi * RW;
  const int qb0_wg = qg * SH::QWG;           // first query block of the workgroup
  const int qb0 = qb0_wg + qgrp * QW;        // first query block of this wave

  // key blocks, query blocks and keys (all from Pp and P in the one-pass form)
  const int nkb = MODE == 0 ? Pp / 32 : nbk_in;
  const int nbq = MODE == 0 ? Pp / 32 : nbq_in;
  const int Pk = MODE == 0 ? P : Pk_in;

  int rows_c[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) rows_c[rr] = min(r0 + rr, nrows - 1);

  // ---- per-(row, query block) state ----
  f16x8 Q[RW][QW][2];
  f32x16 O[RW][QW];
  float m_sh[RW][QW], l_run[RW][QW];
  bool mset[RW], shifted[RW];   // wave-uniform: row has its shift / some lane has m != 0
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    mset[rr] = false;
    shifted[rr] = false;
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const int qblk = min(qb0 + qq, nbq - 1);
      const int64_t rh = (int64_t)rows_c[rr] * H + h;
      PA_DCHECK(qkv_chunk(rh, nbq, qblk, 1) + 512 <= (int64_t)nrows * H * nbq * 1024, 3);
      Q[rr][qq][0] = ld16(q_ws + qkv_chunk(rh, nbq, qblk, 0) + lane * 8);
      Q[rr][qq][1] = ld16(q_ws + qkv_chunk(rh, nbq, qblk, 1) + lane * 8);
      O[rr][qq] = f32x16{};
      m_sh[rr][qq] = 0.0f;
      l_run[rr][qq] = 0.0f;
    }
  }

  // ---- staging: K/V ring (NKV stages) and bias ring (2 stages) ----
  // Every 1 KB copy of this wave advances by 2 KB (one key block) per kb in
  // its source, so the sources of key block 0 and the LDS offsets are
  // computed once.  Blocks past the end are clamped to the last one
  // (in-bounds copies into a free stage), so that every block issues the
  // same number of copies and the counted wait holds.
  constexpr int NCW = SH::NCW, NCB = SH::NCB;
  const f16* kv_src[NCW];
  int kv_off[NCW];
  const f16* b_src[NCB];
  int b_off[NCB];
#pragma unroll
  for (int j = 0; j < NCW; ++j) {
    const int i = wave + 8 * j;
    const int t = i >> 2, c = i & 3;          // tile (row, head), chunk K0 K1 V0 V1
    const int rr = t / H, hh = t % H;
    const int64_t rh = (int64_t)rows_c[rr] * H + hh;
    kv_src[j] = (c < 2 ? k_ws : v_ws) + qkv_chunk(rh, nkb, 0, c & 1);
    kv_off[j] = t * SH::KV_TILE + c * 1024;
  }
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const int ib = wave + 8 * j;
    const int t = ib >> 1, c = ib & 1;        // tile (query block, head), chunk
    const int qb = min(qb0_wg + t / H, nbq - 1), hh = t % H;
    b_src[j] = bias + b16_chunk(hh, nbq, nkb, qb, 0, c);
    b_off[j] = t * SH::B_TILE + c * 1024;
  }
  constexpr int NU = RW * QW;   // units per wave and key block, query-block major
  // copies [j0, j1) of one stage
  auto stage_kv = [&](int kb, int j0, int j1) {
    const int kbc = min(kb, nkb - 1);
    char* base = kv_lds + (kb % SH::NKV) * SH::KV_STAGE;
#pragma unroll
    for (int j = 0; j < NCW; ++j)
      if (j >= j0 && j < j1) {
        PA_DCHECK((kv_src[j] - ((wave & 3) < 2 ? k_ws : v_ws)) + (int64_t)kbc * 1024 + 512 <=
                      (int64_t)nrows * H * nkb * 1024, 0);   // one 512-element chunk
        PA_DCHECK(kv_off[j] + 1024 <= SH::KV_STAGE, 2);
        g2lds16_ring(kv_src[j] + (int64_t)kbc * 1024 + lane * 8, base + kv_off[j]);
      }
  };
  auto stage_b = [&](int kb, int j0, int j1) {
    const int kbc = min(kb, nkb - 1);
    char* base = b_lds + (kb & 1) * SH::B_STAGE;
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      if (j >= j0 && j < j1) {
        PA_DCHECK((b_src[j] - bias) + (int64_t)kbc * 1024 + 512 <= (int64_t)H * nbq * nkb * 1024, 1);
        PA_DCHECK(b_off[j] + 1024 <= SH::B_STAGE, 2);
        g2lds16_ring(b_src[j] + (int64_t)kbc * 1024 + lane * 8, base + b_off[j]);
      }
  };
  // The copies of one block (bias stage kb+1, then K/V stage kb+NKV-1) are
  // spread over its units, so that the address unit works through them while
  // the waves compute instead of stalling the issue of every wave at once.
  constexpr int NCP = NCB + NCW;                 // copies per wave and block
  auto copies_for_unit = [&](int kb, int u) {
    const int c0 = u * NCP / NU, c1 = (u + 1) * NCP / NU;
    stage_b(kb + 1, c0, min(c1, NCB));
    stage_kv(kb + SH::NKV - 1, max(c0 - NCB, 0), c1 - NCB);
  };
  // keep bits: word (row, kb) of mask_bits holds bit b = key kb*32+b kept.
  // Without a mask only keys past P are dropped, which is computed; with
  // one the word is a scalar load (scalar loads do not count against the
  // copies' vector-memory counter).
  auto keep_bits = [&](int rr, int kb) -> uint32_t {
    if constexpr (HAS_MASK) {
      return mask_bits[(int64_t)rows_c[rr] * nkb + kb];
    } else {
      const int n = Pk - kb * 32;
      return n >= 32 ? 0xffffffffu : (n <= 0 ? 0u : ((1u << n) - 1u));
    }
  };

  // Q has landed before the generic sweep issues any copy: the compiler's
  // waits for it would otherwise sit inside the loop and drain the copies
  // too.  (The empty asm statements consume Q, so its loads cannot sink
  // below.)
  auto wait_q = [&]() {
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) asm volatile("" ::"v"(Q[rr][qq][0]), "v"(Q[rr][qq][1]));
    wait_vmcnt<0>();
  };
  bool row_has_key[RW];   // wave-uniform: some block of the row keeps a key

  // Epilogue operands: the gate tiles (layout of q; loaded during the last
  // key block of the pipelined sweep, so that their latency hides behind it)
  // and the W_o^T rows of this wave's output channel block (loaded before
  // the gated o tiles are formed).
  constexpr int CBN = C_OUT / 32;
  constexpr int KO = HD / 16;
  const int cb_w = wave % CBN;
  f16x8 Gt[RW][QW][2], Wo[KO];
  bf16x4 Bo[4];   // b_o of this lane's output channels cb_w*32 + jj*8 + g*4 + 0..3
  auto load_wo = [&]() {
#pragma unroll
    for (int t = 0; t < KO; ++t) Wo[t] = ld16(woT + (int64_t)(cb_w * 32 + lq) * HD + t * 16 + g * 8);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      Bo[jj] = b_o != nullptr ? *reinterpret_cast<const bf16x4*>(b_o + cb_w * 32 + jj * 8 + g * 4) : bf16x4{};
  };
  auto load_epi = [&]() {
    if constexpr (MODE == 0) {
#pragma unroll
      for (int rr = 0; rr < RW; ++rr)
#pragma unroll
        for (int qq = 0; qq < QW; ++qq) {
          const int64_t rh = (int64_t)rows_c[rr] * H + h;
          PA_DCHECK(qkv_chunk(rh, nbq, min(qb0 + qq, nbq - 1), 1) + 512 <= (int64_t)nrows * H * nbq * 1024, 3);
          const f16* gp = g_ws + qkv_chunk(rh, nbq, min(qb0 + qq, nbq - 1), 0) + lane * 8;
          Gt[rr][qq][0] = ld16(gp);
          Gt[rr][qq][1] = ld16(gp + 512);
        }
    }
  };

  // One sweep over all key blocks.
  //   FAST: p = exp2(S) with no shift and no per-unit test, so the units of
  //         a block form one basic block.  Valid when every sum l stays finite
  //         (no fp16 weight, nor in the pipelined sweeps an fp16 partial sum
  //         of four weights, overflowed) and is at least 1 for rows with a
  //         kept key (the largest weights are normal fp16 numbers); checked
  //         after the sweep, and the workgroup sweeps again with SAFE
  //         otherwise.
  //   SAFE: a per-(row, query) shift chosen on the row's first block with a
  //         kept key and raised whenever a block sum passes 2^15.
  auto sweep = [&](auto fastc) {
    constexpr bool FAST = decltype(fastc)::value;
    wait_q();
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      mset[rr] = FAST;
      shifted[rr] = false;
      row_has_key[rr] = false;
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        O[rr][qq] = f32x16{};
        m_sh[rr][qq] = 0.0f;
        l_run[rr][qq] = 0.0f;
      }
    }
    stage_b(0, 0, NCB);
  #pragma unroll
    for (int j = 0; j < SH::NKV - 1; ++j) stage_kv(j, 0, NCW);


    for (int kb = 0; kb < nkb; ++kb) {
      // Bias stage kb and K/V stage kb landed for all waves, stages kb-1 fully
      // read.  A bare barrier: __syncthreads' release fence would also wait
      // for the copies in flight for later blocks.  The empty asm statements
      // keep the compiler from moving LDS accesses across it.
      wait_vmcnt<SH::WAIT>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      uint32_t bits_cur[RW];
  #pragma unroll
      for (int rr = 0; rr < RW; ++rr) bits_cur[rr] = keep_bits(rr, kb);

      const char* st = kv_lds + (kb % SH::NKV) * SH::KV_STAGE;
      const char* bst = b_lds + (kb & 1) * SH::B_STAGE;
      f16x8 K[RW][2], V[RW][2];
  #pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const char* kv = st + (rr * H + h) * SH::KV_TILE + lane * 16;
        K[rr][0] = lds_f16x8(kv);
        K[rr][1] = lds_f16x8(kv + 1024);
        V[rr][0] = lds_f16x8(kv + 2048);
        V[rr][1] = lds_f16x8(kv + 3072);
      }
      f16x8 Bt[QW][2];
  #pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        const char* bt = bst + ((qgrp * QW + qq) * H + h) * SH::B_TILE + lane * 16;
        Bt[qq][0] = lds_f16x8(bt);
        Bt[qq][1] = lds_f16x8(bt + 1024);
      }
      auto bias_c = [&](int qq) -> f32x16 { return widen_bias(Bt[qq][0], Bt[qq][1], ident4); };
      auto qk = [&](int rr, int qq, const f32x16& C) -> f32x16 {
        const f32x16 S = mfma32(K[rr][0], Q[rr][qq][0], C);
        return mfma32(K[rr][1], Q[rr][qq][1], S);
      };
      bool keyed[RW], full[RW];
  #pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        keyed[rr] = false;                           // block holds a kept key of row rr
        full[rr] = bits_cur[rr] == 0xffffffffu;      // no masked key in this block
      }

      // The units of the block (MASKED: the keep bits are consulted).
      auto units = [&](auto maskedc) {
        constexpr bool MASKED = decltype(maskedc)::value;
        f32x16 Cb = bias_c(0);
        f32x16 Scur = qk(0, 0, Cb);
    #pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int qq = u / RW, rr = u % RW;
          // priority ladder over the units of a block, falling from 3 (as in
          // the pipelined sweep: the wave that is behind in the block wins
          // the issue arbitration)
          if (u == 0) __builtin_amdgcn_s_setprio(3);
          else if (u == 1) __builtin_amdgcn_s_setprio(NU >= 3 ? 2 : 0);
          else if (u == 2) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
          copies_for_unit(kb, u);
          f32x16 Snext;
          if (u + 1 < NU) {
            const int nq = (u + 1) / RW, nr = (u + 1) % RW;
            if (nr == 0) Cb = bias_c(nq);
            Snext = qk(nr, nq, Cb);
          }
          f32x16 S = Scur;
          if (MASKED && !full[rr]) {   // masked keys (or keys past P) get -inf
            // Register j holds key (j/4)*8 + g*4 + j%4: its keep bit depends only
            // on the lane half g, so the select's lane mask is built on the
            // scalar unit (no per-lane bit tests).
            keep_unit(S, bits_cur[rr]);
          }
          if (!FAST && shifted[rr]) {
    #pragma unroll
            for (int j = 0; j < 16; ++j) S[j] -= m_sh[rr][qq];
          }

          // fast path, unconditional so that it shares a basic block (and the
          // scheduler's interleaving) with the MFMAs issued around it
          f16x8 P0, P1;
    #pragma unroll
          for (int j = 0; j < 8; ++j) {
            P0[j] = f2h(fast_exp2(S[j]));
            P1[j] = f2h(fast_exp2(S[8 + j]));
          }
          float psum = sum16_f16(P0, P1);
          if (!FAST && (!mset[rr] || __ballot(!(psum <= 32768.0f)) != 0)) {
            // S is relative to the current shift; choose / raise the shift
            float bmax = S[0];
    #pragma unroll
            for (int j = 1; j < 16; ++j) bmax = fmaxf(bmax, S[j]);
            bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
            const bool any_key = __ballot(bmax > -__builtin_inff()) != 0;
            keyed[rr] = keyed[rr] || any_key;
            float d = 0.0f;
            if (any_key) {
              if (mset[rr]) {
                d = fmaxf(bmax, 0.0f);
                const float alpha = fast_exp2(-d);
    #pragma unroll
                for (int j = 0; j < 16; ++j) O[rr][qq][j] *= alpha;
                l_run[rr][qq] *= alpha;
              } else {
                d = (bmax >= -8.0f && bmax <= 8.0f) ? 0.0f : bmax;
              }
              m_sh[rr][qq] += d;
            }
    #pragma unroll
            for (int j = 0; j < 8; ++j) {
              P0[j] = f2h(fast_exp2(S[j] - d));
              P1[j] = f2h(fast_exp2(S[8 + j] - d));
            }
            psum = sum16_f16(P0, P1);
            shifted[rr] = shifted[rr] || __ballot(m_sh[rr][qq] != 0.0f) != 0;
          }
          l_run[rr][qq] += psum;
          O[rr][qq] = mfma32(V[rr][0], P0, O[rr][qq]);
          O[rr][qq] = mfma32(V[rr][1], P1, O[rr][qq]);
          if (u + 1 < NU) Scur = Snext;
        }
      };
      units(std::integral_constant<bool, true>{});
      // the first block with a kept key sets the reference maximum of the row
  #pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        mset[rr] = mset[rr] || keyed[rr];
        row_has_key[rr] = row_has_key[rr] || bits_cur[rr] != 0u;
      }
    }

  };

  auto cvt_bias = [&](const f16x8* b) -> f32x16 { return widen_bias(b[0], b[1], ident4); };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // softmax of S (one unit) with the next unit's logits (NEXT) and this
  // unit's P.V product issued between its exp2 groups.  The row sums: the
  // 16 fp16 weights of a lane are added in fp16 to four sums of four
  // (packed adds), which one 4x4x4 product with ones adds into lacc in fp32
  // (every element of lacc holds the lane's running sum).  A partial sum
  // that overflows fp16 makes l infinite, which the check after the fast
  // sweep sends to the shifted rerun.  MASKED: keys
  // whose bit in `bits` is clear get -inf first (register j holds key
  // (j/4)*8 + g*4 + j%4, so the select's lane mask is built on the scalar
  // unit).
  auto stream = [&](auto nextc, auto maskc, const f32x16& S_in, f32x16& Sn, const f16x8* kn, const f16x8* qn,
                    const f32x16& cn, const f16x8* v, f32x16& o, f32x4& lacc, uint32_t bits) {
    constexpr bool NEXT = decltype(nextc)::value;
    constexpr bool MASKED = decltype(maskc)::value;
    float e[16];
    f16x8 p0, p1;
    f32x16 S = S_in;
    if constexpr (MASKED) {
      if (bits != 0xffffffffu) keep_unit(S, bits);   // uniform: a block with every key kept skips the select
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = fast_exp2(S[j]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn[0], qn[0], cn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 4; j < 8; ++j) e[j] = fast_exp2(S[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) p0[j] = f2h(e[j]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn[1], qn[1], Sn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 8; j < 12; ++j) e[j] = fast_exp2(S[j]);
    __builtin_amdgcn_sched_barrier(0);
    o = mfma32(v[0], p0, o);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 12; j < 16; ++j) e[j] = fast_exp2(S[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) p1[j] = f2h(e[8 + j]);
    __builtin_amdgcn_sched_barrier(0);
    o = mfma32(v[1], p1, o);
    __builtin_amdgcn_sched_barrier(0);
    {
      const f16x8 ps = p0 + p1;                     // four packed fp16 adds
      lacc = mfma4(ones4, lo4(ps) + hi4(ps), lacc);   // two more, then one product
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Software-pipelined form of the fast sweep for blocks without masked
  // keys (no mask, P a multiple of 32; H = 4, four units per wave and key
  // block).  Unit order within a block: (row 0, qb 0), (1, 0), (0, 1),
  // (1, 1).  Stream s of a block runs the softmax of unit s on the VALU and
  // issues, between its groups of exp2, the logits of unit s+1 and the P.V
  // product of unit s, so that the matrix cores work while the softmax runs
  // and no exp2 waits for the logits it reads.  The barrier that publishes
  // key block kb+1 sits at the start of stream 2 of block kb: the LDS reads
  // of the next K and bias tiles run under the softmax of units 2 and 3, and
  // the logits of the next block's first unit are issued in stream 3.
  //
  // Staging (per wave; NCW K/V and NCB bias copies per block):
  //   stream 0 of kb: K/V copies 2..3 of block kb+2
  //   stream 2 of kb: wait until at most NCW copies are in flight (bias
  //                   kb+1 and K/V kb+1 landed), barrier, bias copies of
  //                   block kb+2 (its stage held block kb, read before it)
  //   stream 3 of kb: K/V copies 0..1 of block kb+3 (stage of block kb,
  //                   already in registers)
  // Copies for blocks past the end are clamped dummies, so that every
  // counted wait sees the same number of copies behind it; the last block
  // issues none.  Each copy is addressed as a wave-uniform base (advanced
  // per block on the scalar unit) plus a fixed per-lane offset.
  //
  // Wave priority falls from 3 to 0 over the four streams of a block.  The
  // two waves sharing a SIMD are otherwise issued oldest first: the older
  // one finishes its block early and idles at the barrier while the younger
  // one runs the rest alone; with the ladder the wave that is behind in the
  // block wins the issue arbitration, and both reach the barrier together.
  //
  // The sweep runs over key blocks [lo, hi): every kept key of the
  // workgroup's rows lies there, so the blocks outside hold none and are
  // skipped (the fast sweep's sums do not depend on which blocks without a
  // kept key are left out).
  //   KMODE 0: no mask, P a multiple of 32 (lo = 0, hi = nkb): no select
  //   KMODE 1: no mask, only the last block holds keys past P
  //   KMODE 2: a mask; lo, hi from the rows' ranges; every block runs the
  //            masked streams, where a block whose keys are all kept skips
  //            the select on a uniform branch.  (Separate unmasked and
  //            masked loops in one kernel need more than 256 registers, and
  //            the spill reloads would drain the copies in flight.)
  auto sweep_pipe = [&](auto kmodec, int lo, int hi) {
   constexpr int KMODE = decltype(kmodec)::value;
   if constexpr (QW == 2 && RW == 2 && NCW == 4) {
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    f32x4 lacc[RW][QW];   // row sums of the sweep (every element holds the lane's sum)
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        O[rr][qq] = f32x16{};
        m_sh[rr][qq] = 0.0f;
        l_run[rr][qq] = 0.0f;
        lacc[rr][qq] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    // copy sources: one wave-uniform base per ring, per-lane byte offsets
    const f16* kv_base = kv_src[0];
    const f16* b_base = b_src[0];
    uint32_t kv_voff[NCW], b_voff[NCB];
#pragma unroll
    for (int j = 0; j < NCW; ++j) kv_voff[j] = (uint32_t)((kv_src[j] - kv_base) * 2) + lane * 16;
#pragma unroll
    for (int j = 0; j < NCB; ++j) b_voff[j] = (uint32_t)((b_src[j] - b_base) * 2) + lane * 16;
    auto copy_kv = [&](int kb, int j0, int j1) {
      const int kbc = min(kb, nkb - 1);
      const f16* src = kv_base + (int64_t)kbc * 1024;
      const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)(kv_lds + (kb % SH::NKV) * SH::KV_STAGE);
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        PA_DCHECK((src - ((wave & 3) < 2 ? k_ws : v_ws)) * 2 + kv_voff[j] + 16 <= (int64_t)nrows * H * nkb * 2048, 0);
        PA_DCHECK(kv_off[j] + 1024 <= SH::KV_STAGE, 2);
        g2lds16_sbase(src, kv_voff[j], base + kv_off[j]);
      }
    };
    auto copy_b = [&](int kb) {
      const int kbc = min(kb, nkb - 1);
      const f16* src = b_base + (int64_t)kbc * 1024;
      const uint32_t base = (uint32_t)(uintptr_t)(lds_void_t*)(b_lds + (kb & 1) * SH::B_STAGE);
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        PA_DCHECK((src - bias) * 2 + b_voff[j] + 16 <= (int64_t)H * nbq * nkb * 2048, 1);
        PA_DCHECK(b_off[j] + 1024 <= SH::B_STAGE, 2);
        g2lds16_sbase(src, b_voff[j], base + b_off[j]);
      }
    };
    auto kv_tile = [&](int kb, int rr) -> const char* {
      return kv_lds + (kb % SH::NKV) * SH::KV_STAGE + (rr * H + h) * SH::KV_TILE + lane * 16;
    };
    auto b_tile = [&](int kb, int qq) -> const char* {
      return b_lds + (kb & 1) * SH::B_STAGE + ((qgrp * QW + qq) * H + h) * SH::B_TILE + lane * 16;
    };
    struct Regs {
      f16x8 K[RW][2], V[RW][2], B1[2];   // K and V tiles of both rows, bias tile of query block 1
    };
    Regs ra;
    f32x16 S_pipe, C_pipe;   // logits of the unit the next stream runs; bias accumulator of its query block

    // prologue: stages of blocks lo and lo+1 and Q land together (one
    // latency instead of two), barrier, block lo in registers
    copy_b(lo);
    copy_kv(lo, 0, NCW);
    copy_kv(lo + 1, 0, NCW);
    wait_q();
    barrier();
    {
      f16x8 B0[2];
#pragma unroll
      for (int rr = 0; rr < RW; ++rr)
#pragma unroll
        for (int c = 0; c < 2; ++c) ra.K[rr][c] = lds_f16x8(kv_tile(lo, rr) + c * 1024);
#pragma unroll
      for (int c = 0; c < 2; ++c) B0[c] = lds_f16x8(b_tile(lo, 0) + c * 1024);
      copy_b(lo + 1);
      copy_kv(lo + 2, 0, 2);
#pragma unroll
      for (int rr = 0; rr < RW; ++rr)
#pragma unroll
        for (int c = 0; c < 2; ++c) ra.V[rr][c] = lds_f16x8(kv_tile(lo, rr) + 2048 + c * 1024);
#pragma unroll
      for (int c = 0; c < 2; ++c) ra.B1[c] = lds_f16x8(b_tile(lo, 1) + c * 1024);
      C_pipe = cvt_bias(B0);
      S_pipe = mfma32(ra.K[0][1], Q[0][0][1], mfma32(ra.K[0][0], Q[0][0][0], C_pipe));
    }
    // block kb from the registers in r; the next block's tiles are read into
    // r in place, each once its current value has had its last use (K of
    // row 0 after the logits of unit 2, K of row 1 after those of unit 3, V
    // of row 0 after the P.V of unit 2, V of row 1 and the bias tile of
    // query block 1 after that of unit 3)
    // bits0, bits1: keep bits of block kb for rows 0 and 1 (MASKED blocks)
    auto block = [&](int kb, auto morec, auto maskc, Regs& r, uint32_t bits0, uint32_t bits1) {
      constexpr bool MORE = decltype(morec)::value;
      f32x16 Sn;
      // stream 0: unit (0, 0); next (1, 0)
      __builtin_amdgcn_s_setprio(3);
      if constexpr (MORE) copy_kv(kb + 2, 2, 4);
      else load_epi();
      stream(T{}, maskc, S_pipe, Sn, r.K[1], Q[1][0], C_pipe, r.V[0], O[0][0], lacc[0][0], bits0);
      S_pipe = Sn;
      C_pipe = cvt_bias(r.B1);
      // stream 1: unit (1, 0); next (0, 1)
      __builtin_amdgcn_s_setprio(2);
      stream(T{}, maskc, S_pipe, Sn, r.K[0], Q[0][1], C_pipe, r.V[1], O[1][0], lacc[1][0], bits1);
      S_pipe = Sn;
      // stream 2: unit (0, 1); next (1, 1); block kb+1 published
      __builtin_amdgcn_s_setprio(1);
      f16x8 Bn0[2];
      if constexpr (MORE) {
        wait_vmcnt<NCW>();
        barrier();
#pragma unroll
        for (int c = 0; c < 2; ++c) r.K[0][c] = lds_f16x8(kv_tile(kb + 1, 0) + c * 1024);
#pragma unroll
        for (int c = 0; c < 2; ++c) Bn0[c] = lds_f16x8(b_tile(kb + 1, 0) + c * 1024);
        copy_b(kb + 2);
      }
      stream(T{}, maskc, S_pipe, Sn, r.K[1], Q[1][1], C_pipe, r.V[0], O[0][1], lacc[0][1], bits0);
      S_pipe = Sn;
      if constexpr (MORE) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          r.K[1][c] = lds_f16x8(kv_tile(kb + 1, 1) + c * 1024);
          r.V[0][c] = lds_f16x8(kv_tile(kb + 1, 0) + 2048 + c * 1024);
        }
        C_pipe = cvt_bias(Bn0);   // the bias of query block 1 had its last use in stream 2
      }
      // stream 3: unit (1, 1); next = unit (0, 0) of block kb+1
      __builtin_amdgcn_s_setprio(0);
      stream(morec, maskc, S_pipe, Sn, r.K[0], Q[0][0], C_pipe, r.V[1], O[1][1], lacc[1][1], bits1);
      if constexpr (MORE) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          r.V[1][c] = lds_f16x8(kv_tile(kb + 1, 1) + 2048 + c * 1024);
          r.B1[c] = lds_f16x8(b_tile(kb + 1, 1) + c * 1024);
        }
        copy_kv(kb + 3, 0, 2);
        S_pipe = Sn;
      }
    };
    int kb = lo;
    if constexpr (KMODE == 0) {
      for (; kb + 1 < hi; ++kb) block(kb, T{}, F{}, ra, ~0u, ~0u);
      block(kb, F{}, F{}, ra, ~0u, ~0u);
    } else if constexpr (KMODE == 1) {
      for (; kb + 1 < hi; ++kb) block(kb, T{}, F{}, ra, ~0u, ~0u);
      const uint32_t bl = keep_bits(0, kb);   // the last block: keys past P dropped
      block(kb, F{}, T{}, ra, bl, bl);
    } else {
      for (; kb + 1 < hi; ++kb) block(kb, T{}, T{}, ra, keep_bits(0, kb), keep_bits(1, kb));
      block(kb, F{}, T{}, ra, keep_bits(0, kb), keep_bits(1, kb));
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) l_run[rr][qq] = lacc[rr][qq][0];
   }
  };

  // Software-pipelined form of the fast sweep at H = 8 (one row and three
  // query blocks per wave).  No tile is shared between waves here: a wave's
  // K/V tile is its (row, head), its bias tiles are its head's tiles of the
  // workgroup's query blocks.  So each wave copies exactly its own chunks
  // into the ring stages and waits for its own copies only; no barrier
  // orders the rings.  Every tile of block kb is in registers before the
  // block runs, so its stage is refilled with block kb+2 after the first
  // stream (once the reads of the stage have landed).
  //   stream 0 of kb: unit of query block 0, logits of query block 1; then
  //                   the copies of block kb+2
  //   stream 1 of kb: query block 1, logits of query block 2; then block
  //                   kb+1's K and bias tiles into registers (its copies
  //                   waited for)
  //   stream 2 of kb: query block 2, logits of query block 0 of block kb+1;
  //                   then block kb+1's V tiles
  // KMODE as in sweep_pipe (masks enter through the bias operand, see
  // set_mask); the sweep runs over the row's key blocks [lo, hi).
  auto sweep_pipe8 = [&](auto kmodec, int lo, int hi) {
   constexpr int KMODE = decltype(kmodec)::value;
   if constexpr (H == 8 && RW == 1 && QW == 3) {
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    f32x4 lacc[QW];   // row sums (every element holds the lane's sum)
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      O[0][qq] = f32x16{};
      m_sh[0][qq] = 0.0f;
      l_run[0][qq] = 0.0f;
      lacc[qq] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // copy sources: wave-uniform bases (block 0) and per-lane byte offsets
    const int64_t rh = (int64_t)rows_c[0] * H + h;
    const f16* k_base = k_ws + qkv_chunk(rh, nkb, 0, 0);
    const f16* v_base = v_ws + qkv_chunk(rh, nkb, 0, 0);
    const int64_t b_first = b16_chunk(h, nbq, nkb, min(qb0_wg, nbq - 1), 0, 0);
    const f16* b_base = bias + b_first;
    const uint32_t lane16 = lane * 16;
    uint32_t b_voff[QW];
#pragma unroll
    for (int qq = 0; qq < QW; ++qq)
      b_voff[qq] = (uint32_t)((b16_chunk(h, nbq, nkb, min(qb0_wg + qq, nbq - 1), 0, 0) - b_first) * 2) + lane16;
    // this wave's tiles in the stages (the layout of the shared rings)
    auto kv_at = [&](int kb) -> char* { return kv_lds + (kb % SH::NKV) * SH::KV_STAGE + h * SH::KV_TILE; };
    auto b_at = [&](int kb, int qq) -> char* { return b_lds + (kb & 1) * SH::B_STAGE + (qq * H + h) * SH::B_TILE; };
    // the wave's ten chunks of block kb: K0 K1 V0 V1 and both chunks of each bias tile
    constexpr int NCPB = 4 + 2 * QW;
    auto copy_block = [&](int kb) {
      const int64_t e = (int64_t)kb * 1024;
      PA_DCHECK((k_base - k_ws) + e + 1024 <= (int64_t)nrows * H * nkb * 1024, 0);
      PA_DCHECK((b_base - bias) * 2 + e * 2 + b_voff[QW - 1] + 1024 + 16 <= (int64_t)H * nbq * nkb * 2048, 1);
      const uint32_t kv = (uint32_t)(uintptr_t)(lds_void_t*)kv_at(kb);
      g2lds16_sbase(k_base + e, lane16, kv);
      g2lds16_sbase(k_base + e, lane16 + 1024, kv + 1024);
      g2lds16_sbase(v_base + e, lane16, kv + 2048);
      g2lds16_sbase(v_base + e, lane16 + 1024, kv + 3072);
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        const uint32_t bl = (uint32_t)(uintptr_t)(lds_void_t*)b_at(kb, qq);
        g2lds16_sbase(b_base + e, b_voff[qq], bl);
        g2lds16_sbase(b_base + e, b_voff[qq] + 1024, bl + 1024);
      }
    };
    auto read2 = [&](f16x8* dst, const char* tile) {
#pragma unroll
      for (int c = 0; c < 2; ++c) dst[c] = lds_f16x8(tile + lane * 16 + c * 1024);
    };
    // Masked keys (KMODE 1, 2): the three units of a block share one row, so
    // the block's keep bits become one mask operand MB (0 or -inf per
    // accumulator register), added to the bias by the products that widen
    // it: the logits of masked keys are -inf from the start, with no select
    // per unit.
    f32x16 MB;
    auto set_mask = [&](uint32_t bits) {
      if constexpr (KMODE != 0) {
        MB = f32x16{};
        if (bits != 0xffffffffu) keep_unit(MB, bits);   // uniform
      }
    };
    auto cvt = [&](const f16x8* b) -> f32x16 {
      if constexpr (KMODE == 0) return cvt_bias(b);
      else return widen_bias_acc(b[0], b[1], ident4, MB);
    };

    // prologue: blocks lo and lo+1 and Q land together, block lo into registers
    copy_block(lo);
    if (lo + 1 < hi) copy_block(lo + 1);
    wait_q();
    f16x8 K[2], V[2], B1[2], B2[2];
    f32x16 S_pipe;
    {
      f16x8 B0[2];
      read2(K, kv_at(lo));
      read2(B0, b_at(lo, 0));
      read2(V, kv_at(lo) + 2048);
      read2(B1, b_at(lo, 1));
      read2(B2, b_at(lo, 2));
      set_mask(keep_bits(0, lo));
      S_pipe = mfma32(K[1], Q[0][0][1], mfma32(K[0], Q[0][0][0], cvt(B0)));
    }
    // bits_next: keep bits of block kb+1 (KMODE 1, 2)
    auto block = [&](int kb, auto morec, uint32_t bits_next) {
      constexpr bool MORE = decltype(morec)::value;
      f32x16 Sn, C;
      // stream 0: query block 0; next query block 1
      __builtin_amdgcn_s_setprio(3);
      if constexpr (!MORE) load_epi();
      C = cvt(B1);
      stream(T{}, F{}, S_pipe, Sn, K, Q[0][1], C, V, O[0][0], lacc[0], ~0u);
      S_pipe = Sn;
      if constexpr (MORE) {
        if (kb + 2 < hi) {
          wait_lgkm0();   // every read of this block's stage has landed
          copy_block(kb + 2);
        }
      }
      // stream 1: query block 1; next query block 2
      __builtin_amdgcn_s_setprio(2);
      C = cvt(B2);
      stream(T{}, F{}, S_pipe, Sn, K, Q[0][2], C, V, O[0][1], lacc[1], ~0u);
      S_pipe = Sn;
      if constexpr (MORE) {
        // block kb+1 landed (only block kb+2's copies may still be in flight)
        if (kb + 2 < hi) wait_vmcnt<NCPB>();
        else wait_vmcnt<0>();
        f16x8 B0n[2];
        read2(K, kv_at(kb + 1));
        read2(B0n, b_at(kb + 1, 0));
        read2(B1, b_at(kb + 1, 1));
        read2(B2, b_at(kb + 1, 2));
        set_mask(bits_next);
        C = cvt(B0n);
      }
      // stream 2: query block 2; next query block 0 of block kb+1
      __builtin_amdgcn_s_setprio(1);
      stream(morec, F{}, S_pipe, Sn, K, Q[0][0], C, V, O[0][2], lacc[2], ~0u);
      if constexpr (MORE) {
        read2(V, kv_at(kb + 1) + 2048);
        S_pipe = Sn;
      }
    };
    // (KMODE 1: only the last block drops keys, those past P)
    int kb = lo;
    for (; kb + 1 < hi; ++kb) block(kb, T{}, KMODE == 0 ? ~0u : keep_bits(0, kb + 1));
    block(kb, F{}, ~0u);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) l_run[0][qq] = lacc[qq][0];
   }
  };

  bool epi_loaded = false;
  if constexpr (H == 4) {
    if constexpr (!HAS_MASK) {
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) row_has_key[rr] = true;   // P >= 1: every row has a kept key
      if (Pk == nkb * 32) sweep_pipe(std::integral_constant<int, 0>{}, 0, nkb);
      else sweep_pipe(std::integral_constant<int, 1>{}, 0, nkb);
      epi_loaded = true;
    } else {
      // key-block range of each row: [lo, hi) holds its kept keys (lo = nkb,
      // hi = 0 without any)
      int rlo[RW], rhi[RW];
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const int* rg = mask_range + (int64_t)rows_c[rr] * 2;
        rlo[rr] = rg[0];
        rhi[rr] = rg[1];
        row_has_key[rr] = rlo[rr] < rhi[rr];
      }
      const int lo = min(rlo[0], rlo[1]), hi = max(rhi[0], rhi[1]);
      if (lo < hi) {
        sweep_pipe(std::integral_constant<int, 2>{}, lo, hi);
        epi_loaded = true;
      } else {   // no kept key in either row: o = 0
        wait_q();
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
#pragma unroll
          for (int qq = 0; qq < QW; ++qq) {
            O[rr][qq] = f32x16{};
            m_sh[rr][qq] = 0.0f;
            l_run[rr][qq] = 0.0f;
          }
      }
    }
  } else if constexpr (!HAS_MASK) {
    row_has_key[0] = true;   // P >= 1: the row has a kept key
    if (Pk == nkb * 32) sweep_pipe8(std::integral_constant<int, 0>{}, 0, nkb);
    else sweep_pipe8(std::integral_constant<int, 1>{}, 0, nkb);
    epi_loaded = true;
  } else {
    const int* rg = mask_range + (int64_t)rows_c[0] * 2;
    const int lo = rg[0], hi = rg[1];
    row_has_key[0] = lo < hi;
    if (lo < hi) {
      sweep_pipe8(std::integral_constant<int, 2>{}, lo, hi);
      epi_loaded = true;
    } else {   // no kept key in the row: o = 0
      wait_q();
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        O[0][qq] = f32x16{};
        m_sh[0][qq] = 0.0f;
        l_run[0][qq] = 0.0f;
      }
    }
  }
  if (!epi_loaded) load_epi();
  __builtin_amdgcn_s_setprio(0);
  wait_vm0();   // this wave's copies (dummies past the end included) have landed
  // The output projection's operands (W_o rows, b_o) go out now: their
  // latency passes while the workgroup gathers for the check below.
  if constexpr (MODE == 0) load_wo();
  bool bad = false;
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const float lt = l_run[rr][qq] + __shfl_xor(l_run[rr][qq], 32, 64);
      bad = bad || !(lt < __builtin_inff()) || (row_has_key[rr] && lt < 1.0f);
    }
  // Workgroup-wide "any wave bad", through the last words of the bias ring.
  // After the first barrier every copy of every wave has landed (each waited
  // for its own above) and no wave reads the rings any more; a rerun writes
  // that stage only after the first barrier of its own loop, which every
  // wave reaches after reading the flags.  Bare barriers: __syncthreads
  // would also wait for the W_o loads in flight.
  {
    int* flag = reinterpret_cast<int*>(b_lds + SH::LDS_B - 8 * sizeof(int));
    const bool wbad = __ballot(bad) != 0;
    barrier();
    if (lane == 0) flag[wave] = wbad ? 1 : 0;
    wait_lgkm0();
    barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) any |= flag[w];
    if (any) {
      sweep(std::integral_constant<bool, false>{});
      wait_vm0();
      __syncthreads();   // the rings are idle before the o tiles overwrite them
      // (reloaded, so that neither is live across the rerun)
      load_epi();
      if constexpr (MODE == 0) load_wo();
    }
  }
  if constexpr (MODE != 0) {
    // ---- one key shard: o and lse per (row, head, query), written or merged ----
    constexpr float kLn2 = 0.6931471805599453f;
    // Where one row's o tile fits the K/V ring, it is staged there (scaled
    // by its merge weight, with the old o's weight beside it) and leaves as
    // whole query rows of H*32 floats, so every store and merge load is a
    // contiguous 1 KB per instruction; else each lane writes its own pieces.
    constexpr int NQ = SH::QWG * 32;          // queries of the workgroup
    constexpr int OPF = HD + 4;               // staged row pitch (floats): 16-byte rows, spread banks
    constexpr bool STAGE_O = (NQ * OPF + NQ * H) * 4 <= SH::LDS_KV;
    float* o_st = reinterpret_cast<float*>(kv_lds);
    float* w_st = o_st + NQ * OPF;            // [NQ][H]: weight of the o already there (merge)
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      if (STAGE_O && rr > 0) __syncthreads();   // the previous row's stores have read the stage
#pragma unroll
      for (int qq = 0; qq < QW; ++qq) {
        const int r = r0 + rr, q = (qb0 + qq) * 32 + lq;
        const float ltot = l_run[rr][qq] + __shfl_xor(l_run[rr][qq], 32, 64);
        if (r >= nrows || q >= P) continue;
        const bool any = ltot > 0.0f;
        // l sums 2^(s - m) over the kept keys, s the logit in log2 units
        const float lse_new = any ? (m_sh[rr][qq] + __builtin_log2f(ltot)) * kLn2 : -__builtin_inff();
        const float inv = any ? 1.0f / ltot : 0.0f;
        float wn = 1.0f, wo = 0.0f, lse = lse_new;
        float* lse_at = lse_part + ((int64_t)r * H + h) * P + q;
        if constexpr (MODE == 2) {
          const float lse_old = *lse_at;
          const float mx = __builtin_fmaxf(lse_old, lse_new);
          if (mx == -__builtin_inff()) {
            wn = 0.0f;   // no kept key in either part: o stays 0, lse -inf
          } else {
            wo = __expf(lse_old - mx);
            wn = __expf(lse_new - mx);
            const float den = wo + wn;
            lse = mx + __logf(den);
            wo /= den;
            wn /= den;
          }
        }
        // O register jj*4+e holds channel jj*8 + g*4 + e of head h
        if constexpr (STAGE_O) {
          const int ql = (qgrp * QW + qq) * 32 + lq;
          float* srow = o_st + ql * OPF + h * 32 + 4 * g;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = O[rr][qq][4 * jj + e] * inv * wn;
            *reinterpret_cast<f32x4*>(srow + 8 * jj) = v;
          }
          if (MODE == 2 && g == 0) w_st[ql * H + h] = wo;
        } else {
          float* orow = o_part + ((int64_t)r * P + q) * (H * 32) + h * 32 + 4 * g;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f32x4* dst = reinterpret_cast<f32x4*>(orow + 8 * jj);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = O[rr][qq][4 * jj + e] * inv * wn;
            if constexpr (MODE == 2) {
              const f32x4 old = *dst;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += old[e] * wo;
            }
            *dst = v;
          }
        }
        if (g == 0) *lse_at = lse;
      }
      if constexpr (STAGE_O) {
        __syncthreads();
        constexpr int C4 = HD / 4;            // 16-byte pieces of a query row
        const int r = r0 + rr;
        for (int i = threadIdx.x; i < NQ * C4; i += 512) {
          const int ql = i / C4, c4 = (i % C4) * 4;
          const int q = qb0_wg * 32 + ql;
          if (r >= nrows || q >= P) continue;
          PA_DCHECK(ql * OPF + c4 + 4 <= NQ * OPF, 7);
          f32x4 v = *reinterpret_cast<const f32x4*>(o_st + ql * OPF + c4);
          f32x4* dst = reinterpret_cast<f32x4*>(o_part + ((int64_t)r * P + q) * HD + c4);
          if constexpr (MODE == 2) {
            const f32x4 old = *dst;
            const float wo = w_st[ql * H + c4 / 32];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += old[e] * wo;
          }
          *dst = v;
        }
      }
    }
    return;
  }

  // ---- epilogue: normalise, gate, output projection (both rows at once) ----
  constexpr int OP = HD + 8;                 // o tile pitch (fp16 elements)
  constexpr int NBLK = SH::QWG * CBN;        // 32x32 output blocks per row
  static_assert(8 % CBN == 0, "a wave keeps one output channel block");
  static_assert(RW * SH::QWG * 32 * OP * 2 <= SH::LDS_KV, "o tiles of both rows fit the K/V ring");
  f16* o_lds = reinterpret_cast<f16*>(kv_lds);
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
      const float ltot = l_run[rr][qq] + __shfl_xor(l_run[rr][qq], 32, 64);
      const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
      // gate chunk t holds the gates of O registers 8t..8t+7 (channels
      // slot_x(t, g, 0..7)) of this lane
      f16* dst = o_lds + ((rr * SH::QWG + qgrp * QW + qq) * 32 + lq) * OP + h * 32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {   // O register jj*4+e holds channel jj*8 + g*4 + e
        f16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jj * 4 + e;
          const float gv = (float)(j < 8 ? Gt[rr][qq][0][j] : Gt[rr][qq][1][j - 8]);
          ov[e] = f2h_sat(O[rr][qq][j] * inv * gv);
        }
        st8(dst + jj * 8 + g * 4, ov);
      }
    }
  }
  __syncthreads();
  // bf16 store of one 32x32 output block (+ b_o) at the caller's strides
  auto store_block = [&](int rr, int qbl, const f32x16& acc) {
    const int r = r0 + rr;
    const int q = (qb0_wg + qbl) * 32 + lq;
    if (r < nrows && q < P) {
      bf16* o = out + (int64_t)r * os_r + (int64_t)q * os_p + cb_w * 32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = f2bf(acc[jj * 4 + e] + bf2f(Bo[jj][e]));
        }
        st8(o + jj * 8 + g * 4, ov);
      }
    }
  };
  // every wave owns the output blocks blk = wave + 8j of each row (all of
  // channel block cb_w): their MFMA chains are interleaved, so that no MFMA
  // waits for the one before it
  constexpr int NBW = (NBLK + 7) / 8;
  f32x16 acc[RW][NBW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[rr][j] = f32x16{};
#pragma unroll
  for (int t = 0; t < KO; ++t)
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int blk = wave + 8 * j;
        if (NBLK % 8 == 0 || blk < NBLK) {   // uniform
          const f16* src = o_lds + ((rr * SH::QWG + blk / CBN) * 32 + lq) * OP + g * 8;
          acc[rr][j] = mfma32(Wo[t], lds_f16x8((const char*)(src + t * 16)), acc[rr][j]);
        }
      }
  if constexpr (C_OUT <= HD) {
    // The workgroup's output tile (+ b_o, bf16) is staged in LDS over the o
    // tiles, then stored query row by query row, 16 bytes per lane: the
    // C_OUT channels of a query are contiguous at the caller's strides (and
    // the whole tile is one run when positions are), so every store
    // instruction writes whole cache lines, not 64-byte pieces of 32 rows.
    constexpr int SP = C_OUT + 8;          // staged row pitch (bf16), rows 16-byte aligned
    constexpr int NQ = SH::QWG * 32;       // queries of the workgroup
    constexpr int CH = C_OUT / 8;          // 16-byte chunks of a query row
    static_assert(RW * NQ * SP * 2 <= SH::LDS_KV, "staged output tile fits the K/V ring");
    bf16* st_lds = reinterpret_cast<bf16*>(kv_lds);
    __syncthreads();   // every wave has read the o tiles
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int blk = wave + 8 * j;
        if (NBLK % 8 == 0 || blk < NBLK) {
          PA_DCHECK(((rr * SH::QWG + blk / CBN) * 32 + lq) * SP + cb_w * 32 + 32 <= RW * NQ * SP, 7);
          bf16* o = st_lds + ((rr * SH::QWG + blk / CBN) * 32 + lq) * SP + cb_w * 32;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            bf16x4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ov[e] = f2bf(acc[rr][j][jj * 4 + e] + bf2f(Bo[jj][e]));
            }
            st8(o + jj * 8 + g * 4, ov);
          }
        }
      }
    __syncthreads();
    for (int i = threadIdx.x; i < RW * NQ * CH; i += 512) {
      const int ch = i % CH, row = i / CH;
      const int rr = row / NQ, qi = row % NQ;
      const int r = r0 + rr, q = qb0_wg * 32 + qi;
      if (r < nrows && q < P)
        st16(out + (int64_t)r * os_r + (int64_t)q * os_p + ch * 8,
             *reinterpret_cast<const bf16x8*>(st_lds + row * SP + ch * 8));
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int blk = wave + 8 * j;
        if (NBLK % 8 == 0 || blk < NBLK) store_block(rr, blk / CBN, acc[rr][j]);
      }
  }
}


// Keep bits and key-block range of each row, one wave per row (mask_bits_row)
__global__ void mask_bits_kernel(const uint8_t* __restrict__ mask, int64_t ms_r, int64_t ms_k,
                                 uint32_t* __restrict__ bits, int* __restrict__ range, int nrows, int P, int nkb) {
  const int64_t row = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kWave;
  if (row >= nrows) return;   // uniform over the wave
  mask_bits_row(mask != nullptr ? mask + row * ms_r : nullptr, ms_k, bits + row * nkb, range + row * 2, P, nkb);
}

hipError_t debug_take_attn(unsigned int* out) { return pa_debug_take(out); }

hipError_t launch_mask_bits(const uint8_t* mask, int64_t ms_r, int64_t ms_k, uint32_t* bits, int nrows, int P,
                            int nkb, hipStream_t s) {
  const int blocks = (int)(((int64_t)nrows + 3) / 4);   // 4 waves (rows) per block
  hipLaunchKernelGGL(mask_bits_kernel, dim3(blocks), dim3(256), 0, s, mask, ms_r, ms_k, bits,
                     mask_range_of(bits, nrows, nkb), nrows, P, nkb);
  return hipGetLastError();
}

// Gate, output projection and store of merged partial outputs (the end of
// ring attention): for each (row r, query block) tile,
//   og = o_part * gate   as fp16 into LDS (gate: sigmoid applied, layout of q)
//   out = og W_o + b_o   (C_OUT/32 output blocks of K = H*32 over 4 waves)
template <int H, int C_OUT>
__global__ __launch_bounds__(256) void attn_finish_kernel(const f16* __restrict__ g_ws,
                                                          const float* __restrict__ o_part,
                                                          const f16* __restrict__ woT, const bf16* __restrict__ b_o,
                                                          bf16* __restrict__ out, int64_t os_r, int64_t os_p,
                                                          int nrows, int P, int nbq) {
  constexpr int HD = H * 32, OP = HD + 8, KO = HD / 16, CBN = C_OUT / 32;
  __shared__ __attribute__((aligned(16))) f16 og[32 * OP];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int64_t ntiles = (int64_t)nrows * nbq;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int r = (int)(tile / nbq), qb = (int)(tile % nbq);
    // groups of 4 channels: 16 bytes of o, 8 bytes of the gate
    for (int gi = tid; gi < 32 * HD / 4; gi += 256) {
      const int q = gi / (HD / 4), c4 = (gi % (HD / 4)) * 4;
      const int pos = qb * 32 + q;
      f32x4 ov = {};
      if (pos < P) ov = *reinterpret_cast<const f32x4*>(o_part + ((int64_t)r * P + pos) * HD + c4);
      const f16x4 gv =
          *reinterpret_cast<const f16x4*>(g_ws + q_off((int64_t)r * H + c4 / 32, nbq, pos, c4 % 32));
      f16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = f2h_sat(ov[e] * (float)gv[e]);
      *reinterpret_cast<f16x4*>(og + q * OP + c4) = v;
    }
    __syncthreads();
    const int pos = qb * 32 + lq;
    for (int blk = wave; blk < CBN; blk += 4) {
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KO; ++t)
        acc = mfma32(ld16(woT + (int64_t)(blk * 32 + lq) * HD + t * 16 + g * 8),
                     lds_f16x8((const char*)(og + lq * OP + t * 16 + g * 8)), acc);
      if (pos < P) {
        bf16* o = out + (int64_t)r * os_r + (int64_t)pos * os_p + blk * 32;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = jj * 8 + g * 4 + e;
            ov[e] = f2bf(acc[jj * 4 + e] + (b_o != nullptr ? bf2f(b_o[blk * 32 + c]) : 0.0f));
          }
          st8(o + jj * 8 + g * 4, ov);
        }
      }
    }
    __syncthreads();   // og is rewritten by the next tile
  }
}

template <int H, int C_OUT>
static hipError_t finish_dispatch(const AttnArgs& a, hipStream_t s) {
  const int nbq = a.Pp / 32;
  if (nbq < 1 || a.Pp != nbq * 32 || a.P < 1 || a.P > a.Pp || a.nrows < 1 || a.o_part == nullptr)
    return hipErrorInvalidValue;
  const int64_t ntiles = (int64_t)a.nrows * nbq;
  const int blocks = (int)std::min<int64_t>(ntiles, 65536);
  hipLaunchKernelGGL((attn_finish_kernel<H, C_OUT>), dim3(blocks), dim3(256), 0, s, (const f16*)a.g_ws,
                     (const float*)a.o_part, (const f16*)a.woT, (const bf16*)a.b_o, (bf16*)a.out, a.os_r, a.os_p,
                     a.nrows, a.P, nbq);
  return hipGetLastError();
}

hipError_t launch_finish_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.H == 4) {
    if (a.c_out == 64) return finish_dispatch<4, 64>(a, s);
    if (a.c_out == 128) return finish_dispatch<4, 128>(a, s);
    if (a.c_out == 256) return finish_dispatch<4, 256>(a, s);
  } else if (a.H == 8) {
    if (a.c_out == 64) return finish_dispatch<8, 64>(a, s);
    if (a.c_out == 128) return finish_dispatch<8, 128>(a, s);
    if (a.c_out == 256) return finish_dispatch<8, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

// Query groups per super-column of the workgroup order.  The XCD of a
// workgroup takes a contiguous range of n_qg * n_rg / 8 logical tiles; a
// super-column holds n_rg * w of them.  Measured at H = 4: super-columns that
// are whole multiples or whole fractions of an XCD range are faster than
// ones that straddle range boundaries (I = 1536, 12 query groups: w = 3, 6,
// 12 beat 4, 5, 8 by 1-2%, 6 best), and the first such width from 4 up was
// the fastest measured (4096 residues, 32 groups: 4 = 8, then 16, 32;
// 16384 in blocks of 1024 rows, 128 groups: 4, then 8, 16).  So: the first
// w in 4..8 that divides the query groups and lines up with the ranges,
// else 4.  At H = 8 (MSA rows) one super-column of up to 16 groups.
static int super_column_width(int H, int n_qg, int n_rg) {
  if (H != 4) return 16;
  const int64_t per = (int64_t)n_qg * n_rg / 8;
  for (int w = 4; w <= 8; ++w) {
    if (n_qg % w != 0) continue;
    const int64_t t = (int64_t)n_rg * w;
    if (per > 0 && (t % per == 0 || per % t == 0)) return w;
  }
  return 4;
}

template <int H, int C_OUT, bool HAS_MASK, int MODE>
static hipError_t attn_dispatch(const AttnArgs& a, hipStream_t s) {
  using SH = AttnShape<H>;
  const int nbq = a.Pp / 32;
  // the sweeps assume at least one key block and rows to work on
  if (nbq < 1 || a.Pp != nbq * 32 || a.P < 1 || a.P > a.Pp || a.nrows < 1) return hipErrorInvalidValue;
  const int nbk = MODE == 0 ? nbq : a.Ppk / 32;
  const int Pk = MODE == 0 ? a.P : a.Pk;
  if (MODE != 0 && (nbk < 1 || a.Ppk != nbk * 32 || Pk < 1 || Pk > a.Ppk || a.o_part == nullptr ||
                    a.lse_part == nullptr))
    return hipErrorInvalidValue;
  const int n_qg = (nbq + SH::QWG - 1) / SH::QWG;
  const int n_rg = (a.nrows + SH::RWG - 1) / SH::RWG;
  const int64_t n = (int64_t)n_qg * n_rg;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;   // one-dimensional grid
  hipLaunchKernelGGL((attn_kernel<H, C_OUT, HAS_MASK, MODE>), dim3((unsigned)n), dim3(512), 0, s,
                     (const f16*)a.q_ws, (const f16*)a.k_ws, (const f16*)a.v_ws, (const f16*)a.g_ws,
                     (const f16*)a.bias, a.mask_bits, a.mask_range, (const f16*)a.woT, (const bf16*)a.b_o, (bf16*)a.out, a.os_r,
                     a.os_p, a.nrows, a.P, a.Pp, n_qg, n_rg, super_column_width(H, n_qg, n_rg), nbq, Pk, nbk,
                     a.o_part, a.lse_part);
  return hipGetLastError();
}

template <int H, int C_OUT, int MODE>
static hipError_t attn_dispatch_m(const AttnArgs& a, hipStream_t s) {
  if (a.mask_bits != nullptr && a.mask_range == nullptr) return hipErrorInvalidValue;   // ranges come with the bits
  return a.mask_bits != nullptr ? attn_dispatch<H, C_OUT, true, MODE>(a, s)
                                : attn_dispatch<H, C_OUT, false, MODE>(a, s);
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.mode == 1 || a.mode == 2) {   // no output projection: one instance per head count
    if (a.H == 4) return a.mode == 1 ? attn_dispatch_m<4, 128, 1>(a, s) : attn_dispatch_m<4, 128, 2>(a, s);
    if (a.H == 8) return a.mode == 1 ? attn_dispatch_m<8, 128, 1>(a, s) : attn_dispatch_m<8, 128, 2>(a, s);
    return hipErrorInvalidValue;
  }
  if (a.mode != 0) return hipErrorInvalidValue;
  if (a.H == 4) {
    if (a.c_out == 64) return attn_dispatch_m<4, 64, 0>(a, s);
    if (a.c_out == 128) return attn_dispatch_m<4, 128, 0>(a, s);
    if (a.c_out == 256) return attn_dispatch_m<4, 256, 0>(a, s);
  } else if (a.H == 8) {
    if (a.c_out == 64) return attn_dispatch_m<8, 64, 0>(a, s);
    if (a.c_out == 128) return attn_dispatch_m<8, 128, 0>(a, s);
    if (a.c_out == 256) return attn_dispatch_m<8, 256, 0>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
