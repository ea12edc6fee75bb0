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
//   workgroup = 8 waves: QB query blocks of 32 x R_WG rows x all H heads
//     H = 4: QB = 2, two row groups of 2 rows (wave = head x row group)
//     H = 8: QB = 1, one row group of 2 rows  (wave = head)
//   unit = 32 queries x 32 keys of one (row, head): five 32x32x16 MFMAs
//     S^T = K Q^T + bias^T + [1 1 mask] [-m_hi -m_lo 1]^T   (three MFMAs)
//     O^T += V^T P^T                                          (two MFMAs)
//   The third MFMA subtracts the running maximum m (held as two fp16 terms)
//   and adds -inf for masked keys, so the softmax needs no VALU max,
//   subtract or select per logit: p = exp2(S), sum, convert.  The maximum is
//   refreshed (and O, l rescaled) only on a row's first key block or when a
//   lane's block sum exceeds 2^8, which bounds every p by 256.
// Memory path per key block (no VGPR staging): every wave copies its own K
// and V tiles (2 rows) and one bias tile (shared through LDS by the waves of
// the same head) with global_load_lds_dwordx4 directly into LDS.  The
// workspace is stored in MFMA operand order, so each copy is one contiguous
// 1 KB read and every LDS read one conflict-free ds_read_b128 per lane.  The
// bias tiles are double buffered; the next block's copies are in flight
// while the current block computes.
// Register maps (32x32 accumulator: column = lane % 32, register j of half g
// = row (j/4)*8 + g*4 + j%4): keys are fed to the S^T MFMA in the order
// pi(m) = m with bits 2 and 3 swapped, which makes S^T register j hold key
// (j/8)*16 + g*8 + j%8, exactly the K-slot order of the P operand.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane, global -> LDS at lds_base + lane*16 (lds_base wave-uniform)
__device__ __forceinline__ void g2lds16(const void* gsrc, char* lds_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)gsrc, (lds_void_t*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x4 lds_f32x4(const char* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f16x8 lds_f16x8(const char* p) { return *reinterpret_cast<const f16x8*>(p); }

template <int H, int C_OUT>
__global__ __launch_bounds__(512, 1) void attn_kernel(
    const f16* __restrict__ q_ws, const f16* __restrict__ k_ws, const f16* __restrict__ v_ws,
    const f16* __restrict__ g_ws, const float* __restrict__ bias, const uint32_t* __restrict__ mask_bits,
    const f16* __restrict__ woT, const bf16* __restrict__ b_o, bf16* __restrict__ out, int64_t os_r,
    int64_t os_p, int nrows, int P, int Pp, int n_qp, int n_rg) {
  static_assert(H == 4 || H == 8, "4 or 8 heads");
  constexpr int HD = H * 32;
  constexpr int QB = H == 4 ? 2 : 1;        // query blocks per wave
  constexpr int RG = 8 / H;                 // row groups per workgroup
  constexpr int RW = 2;                     // rows per wave
  constexpr int RWG = RG * RW;              // rows per workgroup
  constexpr int KV_WAVE = 8192;             // K (2 rows x 2 KB) + V (2 rows x 2 KB)
  constexpr int KV_BYTES = 8 * KV_WAVE;     // 64 KB
  constexpr int TILE = 4096;                // one bias tile (32 q x 32 k fp32)
  constexpr int STAGE = 8 * TILE;           // QB*H = 8 tiles
  constexpr int LDS_BYTES = KV_BYTES + 2 * STAGE;   // 128 KB
  constexpr int OP = HD + 8;                // epilogue o tile pitch (fp16 elements)
  static_assert(RG * QB * 32 * OP * 2 <= LDS_BYTES, "epilogue tile fits");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int h = wave % H;
  const int rg = wave / H;

  // XCD-aware tile order: consecutive workgroup ids are spread round-robin
  // over the 8 XCDs, so give each XCD a contiguous range of logical tiles,
  // and walk tiles in super-columns of 8 query pairs so the workgroups that
  // run together on one XCD share row groups (K/V) and query pairs (bias).
  int L = blockIdx.x;
  {
    const int n = gridDim.x, per = n / 8;
    if (L < per * 8) L = (L % 8) * per + L / 8;
  }
  constexpr int QPB = 8;
  const int sc = L / (n_rg * QPB);
  const int sc_w = min(QPB, n_qp - sc * QPB);
  const int rem = L - sc * n_rg * QPB;
  const int rgi = rem / sc_w;
  const int qp = sc * QPB + rem % sc_w;
  const int q0 = qp * (QB * 32);
  const int r0 = rgi * RWG + rg * RW;

  char* kv_lds = smem + wave * KV_WAVE;
  char* bias_lds = smem + KV_BYTES;
  const int kp_lane = kperm(lq);            // the key this lane feeds to the S^T MFMA
  const int nkb = Pp / 32;
  const f16 HZERO = f2h(0.0f), HONE = f2h(1.0f);
  const f16 HNEG_INF = f2h(-__builtin_inff());

  int rows_c[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) rows_c[rr] = min(r0 + rr, nrows - 1);

  // ---- per-(row, query block) state ----
  f16x8 Q[RW][QB][2];
  f16x8 QA[RW][QB];
  f32x16 O[RW][QB];
  float m_rep[RW][QB], l_run[RW][QB];
  bool mset[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    mset[rr] = false;
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      const int qblk = min(q0 / 32 + qq, nkb - 1);
      const int64_t rh = (int64_t)rows_c[rr] * H + h;
      Q[rr][qq][0] = ld16(q_ws + qkv_chunk(rh, nkb, qblk, 0) + lane * 8);
      Q[rr][qq][1] = ld16(q_ws + qkv_chunk(rh, nkb, qblk, 1) + lane * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) QA[rr][qq][e] = HZERO;
      if (g == 0) QA[rr][qq][2] = HONE;
      O[rr][qq] = f32x16{};
      m_rep[rr][qq] = 0.0f;
      l_run[rr][qq] = 0.0f;
    }
  }

  // ---- staging of key block kb ----
  const int btile_qq = wave / H, btile_h = wave % H;     // the bias tile this wave copies
  const int btile_qb = min(q0 / 32 + btile_qq, nkb - 1);
  auto stage = [&](int kb, int buf) {
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const int64_t rh = (int64_t)rows_c[rr] * H + h;
      g2lds16(k_ws + qkv_chunk(rh, nkb, kb, 0) + lane * 8, kv_lds + rr * 2048);
      g2lds16(k_ws + qkv_chunk(rh, nkb, kb, 1) + lane * 8, kv_lds + rr * 2048 + 1024);
      g2lds16(v_ws + qkv_chunk(rh, nkb, kb, 0) + lane * 8, kv_lds + 4096 + rr * 2048);
      g2lds16(v_ws + qkv_chunk(rh, nkb, kb, 1) + lane * 8, kv_lds + 4096 + rr * 2048 + 1024);
    }
    char* bt = bias_lds + buf * STAGE + wave * TILE;
#pragma unroll
    for (int c = 0; c < 4; ++c) g2lds16(bias + b_chunk(btile_h, nkb, btile_qb, kb, c) + lane * 4, bt + c * 1024);
  };
  // keep bits: word (row, kb) of mask_bits holds bit b = key kb*32+b kept
  auto load_bits = [&](int rr, int kb) -> uint32_t {
    return mask_bits[(int64_t)rows_c[rr] * nkb + kb];
  };
  auto km_operand = [&](uint32_t bits) -> f16x8 {
    f16x8 km;
#pragma unroll
    for (int e = 0; e < 8; ++e) km[e] = HZERO;
    if (g == 0) {
      km[0] = HONE;
      km[1] = HONE;
      km[2] = ((bits >> kp_lane) & 1u) ? HZERO : HNEG_INF;
    }
    return km;
  };

  stage(0, 0);
  uint32_t bits_next[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) bits_next[rr] = load_bits(rr, 0);

  constexpr int NU = RW * QB;   // units per key block
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    wait_vm0();
    __syncthreads();

    // operands of this block from LDS: K/V first, then the bias tiles
    f16x8 K[RW][2], V[RW][2], KM[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      K[rr][0] = lds_f16x8(kv_lds + rr * 2048 + lane * 16);
      K[rr][1] = lds_f16x8(kv_lds + rr * 2048 + 1024 + lane * 16);
      V[rr][0] = lds_f16x8(kv_lds + 4096 + rr * 2048 + lane * 16);
      V[rr][1] = lds_f16x8(kv_lds + 4096 + rr * 2048 + 1024 + lane * 16);
      KM[rr] = km_operand(bits_next[rr]);
    }
    f32x16 Bt[QB];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      const char* bt = bias_lds + buf * STAGE + (qq * H + h) * TILE + lane * 16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 v = lds_f32x4(bt + c * 1024);
#pragma unroll
        for (int e = 0; e < 4; ++e) Bt[qq][c * 4 + e] = v[e];
      }
    }
    // the K/V reads (issued first; LDS returns in order) are complete once at
    // most the 4*QB bias reads are outstanding: the K/V area can be refilled
    if constexpr (QB == 2) asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory");
    if (kb + 1 < nkb) {
      stage(kb + 1, buf ^ 1);
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) bits_next[rr] = load_bits(rr, kb + 1);
    }

    auto qk = [&](int rr, int qq) -> f32x16 {
      f32x16 S = mfma32(K[rr][0], Q[rr][qq][0], Bt[qq]);
      S = mfma32(K[rr][1], Q[rr][qq][1], S);
      return mfma32(KM[rr], QA[rr][qq], S);
    };
    bool keyed[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) keyed[rr] = false;   // block holds a kept key of row rr

    // software pipeline: the logits of unit u+1 are on the matrix cores
    // while the softmax of unit u runs on the VALU
    f32x16 Scur = qk(0, 0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int rr = u / QB, qq = u % QB;
      f32x16 Snext;
      if (u + 1 < NU) Snext = qk((u + 1) / QB, (u + 1) % QB);
      const f32x16 S = Scur;

      float p[16];
      float psum;
      bool slow = !mset[rr];
      if (!slow) {
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = fast_exp2(S[j]);
        float a0 = (p[0] + p[1]) + (p[2] + p[3]), a1 = (p[4] + p[5]) + (p[6] + p[7]);
        float a2 = (p[8] + p[9]) + (p[10] + p[11]), a3 = (p[12] + p[13]) + (p[14] + p[15]);
        psum = (a0 + a1) + (a2 + a3);
        slow = __ballot(!(psum <= 256.0f)) != 0;
      }
      if (slow) {
        float bmax = S[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) bmax = fmaxf(bmax, S[j]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        const bool any_key = __ballot(bmax > -__builtin_inff()) != 0;
        keyed[rr] = keyed[rr] || any_key;
        float d_use = 0.0f;
        if (any_key) {
          const float delta = mset[rr] ? fmaxf(bmax, 0.0f) : bmax;
          const float m_new = m_rep[rr][qq] + delta;
          const f16 hi = f2h(m_new);
          const f16 lo = f2h(m_new - (float)hi);
          const float m_new_rep = (float)hi + (float)lo;
          d_use = m_new_rep - m_rep[rr][qq];
          const float alpha = mset[rr] ? fast_exp2(-d_use) : 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) O[rr][qq][j] *= alpha;
          l_run[rr][qq] *= alpha;
          m_rep[rr][qq] = m_new_rep;
          if (g == 0) {
            QA[rr][qq][0] = -hi;
            QA[rr][qq][1] = -lo;
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = fast_exp2(S[j] - d_use);
        float a0 = (p[0] + p[1]) + (p[2] + p[3]), a1 = (p[4] + p[5]) + (p[6] + p[7]);
        float a2 = (p[8] + p[9]) + (p[10] + p[11]), a3 = (p[12] + p[13]) + (p[14] + p[15]);
        psum = (a0 + a1) + (a2 + a3);
      }
      l_run[rr][qq] += psum;
      f16x8 P0, P1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        P0[j] = f2h(p[j]);
        P1[j] = f2h(p[8 + j]);
      }
      O[rr][qq] = mfma32(V[rr][0], P0, O[rr][qq]);
      O[rr][qq] = mfma32(V[rr][1], P1, O[rr][qq]);
      if (u + 1 < NU) Scur = Snext;
    }
    // the first block with a kept key sets the reference maximum of the row
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) mset[rr] = mset[rr] || keyed[rr];
  }

  // ---- epilogue: normalise, gate, output projection ----
  wait_vm0();
  __syncthreads();   // LDS is reused for the gated o tiles
  constexpr int CBN = C_OUT / 32;
  constexpr int NBLK = RG * QB * CBN;       // 32x32 output blocks per round
  static_assert(8 % CBN == 0, "a wave keeps one output channel block");
  constexpr int KO = HD / 16;
  const int cb_w = wave % CBN;
  f16x8 Wo[KO];
#pragma unroll
  for (int t = 0; t < KO; ++t) Wo[t] = ld16(woT + (int64_t)(cb_w * 32 + lq) * HD + t * 16 + g * 8);
  f16* o_lds = reinterpret_cast<f16*>(smem);

#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      const float ltot = l_run[rr][qq] + __shfl_xor(l_run[rr][qq], 32, 64);
      const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
      const int qpos = min(q0 + qq * 32 + lq, P - 1);
      const f16* gp = g_ws + ((int64_t)rows_c[rr] * P + qpos) * HD + h * 32;
      f16* dst = o_lds + (rg * QB * 32 + qq * 32 + lq) * OP + h * 32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f16x4 gv = *reinterpret_cast<const f16x4*>(gp + jj * 8 + g * 4);
        f16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = f2h_sat(O[rr][qq][jj * 4 + e] * inv * (float)gv[e]);
        st8(dst + jj * 8 + g * 4, ov);
      }
    }
    __syncthreads();
    for (int blk = wave; blk < NBLK; blk += 8) {
      const int rest = blk / CBN;           // (row group, query block)
      const int qq = rest % QB, rgt = rest / QB;
      const f16* src = o_lds + (rgt * QB * 32 + qq * 32 + lq) * OP + g * 8;
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KO; ++t) acc = mfma32(Wo[t], lds_f16x8((const char*)(src + t * 16)), acc);
      const int r = rgi * RWG + rgt * RW + rr;
      const int q = q0 + qq * 32 + lq;
      if (r < nrows && q < P) {
        bf16* o = out + (int64_t)r * os_r + (int64_t)q * os_p + cb_w * 32;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = jj * 8 + g * 4 + e;
            const float bo = b_o != nullptr ? bf2f(b_o[cb_w * 32 + c]) : 0.0f;
            ov[e] = f2bf(acc[jj * 4 + e] + bo);
          }
          st8(o + jj * 8 + g * 4, ov);
        }
      }
    }
    __syncthreads();
  }
}

// keep bits per (row, 32-key block): bit b of word (r, kb) = key kb*32+b is
// kept (key < P and mask[r*ms_r + key*ms_k] != 0, or no mask).  One wave
// per word group: lane = key within the block, ballot packs the bits.
__global__ void mask_bits_kernel(const uint8_t* __restrict__ mask, int64_t ms_r, int64_t ms_k,
                                 uint32_t* __restrict__ bits, int nrows, int P, int nkb) {
  const int64_t nwords = (int64_t)nrows * nkb;
  const int lane = threadIdx.x % kWave;
  const int64_t wave0 = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t w = wave0 * 2; w < nwords; w += nwaves * 2) {   // two words per wave (lane halves)
    const int64_t word = w + (lane >> 5);
    bool keep = false;
    if (word < nwords) {
      const int r = (int)(word / nkb), kb = (int)(word % nkb);
      const int key = kb * 32 + (lane & 31);
      keep = key < P && (mask == nullptr || mask[(int64_t)r * ms_r + (int64_t)key * ms_k] != 0);
    }
    const uint64_t b = __ballot(keep);
    if (lane == 0) bits[w] = (uint32_t)b;
    if (lane == 32 && word < nwords) bits[word] = (uint32_t)(b >> 32);
  }
}

hipError_t launch_mask_bits(const uint8_t* mask, int64_t ms_r, int64_t ms_k, uint32_t* bits, int nrows, int P,
                            int nkb, hipStream_t s) {
  const int64_t nwords = (int64_t)nrows * nkb;
  const int64_t waves = (nwords + 1) / 2;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((waves + 3) / 4, 4096));
  hipLaunchKernelGGL(mask_bits_kernel, dim3(blocks), dim3(256), 0, s, mask, ms_r, ms_k, bits, nrows, P, nkb);
  return hipGetLastError();
}

template <int H, int C_OUT>
static hipError_t attn_dispatch(const AttnArgs& a, hipStream_t s) {
  constexpr int QB = H == 4 ? 2 : 1;
  constexpr int RWG = (8 / H) * 2;
  const int n_qp = (a.Pp + QB * 32 - 1) / (QB * 32);
  const int n_rg = (a.nrows + RWG - 1) / RWG;
  const int64_t n = (int64_t)n_qp * n_rg;
  hipLaunchKernelGGL((attn_kernel<H, C_OUT>), dim3((unsigned)n), dim3(512), 0, s, (const f16*)a.q_ws,
                     (const f16*)a.k_ws, (const f16*)a.v_ws, (const f16*)a.g_ws, a.bias, a.mask_bits,
                     (const f16*)a.woT, (const bf16*)a.b_o, (bf16*)a.out, a.os_r, a.os_p, a.nrows, a.P, a.Pp, n_qp,
                     n_rg);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.H == 4) {
    if (a.c_out == 64) return attn_dispatch<4, 64>(a, s);
    if (a.c_out == 128) return attn_dispatch<4, 128>(a, s);
    if (a.c_out == 256) return attn_dispatch<4, 256>(a, s);
  } else if (a.H == 8) {
    if (a.c_out == 64) return attn_dispatch<8, 64>(a, s);
    if (a.c_out == 128) return attn_dispatch<8, 128>(a, s);
    if (a.c_out == 256) return attn_dispatch<8, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
