// bf16-interface kernels for gated pair-biased attention on gfx950.
//
// Inputs, weights and outputs are bf16.  Every MFMA operand inside the path
// (normalised activations, packed weights, q, k, v, softmax weights, gated
// o) is stored as fp16, which gfx950 multiplies at the same rate as bf16 but
// with 11 instead of 8 significant bits; accumulation, LayerNorm statistics,
// the bias and the softmax run in fp32.  Values headed for fp16 are
// saturated at +-65504.
//
// The attention of every supported operation is cast as "row attention":
// nrows independent rows, each with P positions that are both the queries
// and the keys, H heads of width 32, and a bias[h][query][key] shared by all
// rows.  The orientation (starting node, ending node, MSA rows) only changes
// how a (row, position) pair is addressed in the input, mask and output,
// which every kernel takes as strides.  The ending node is thus read with
// strided loads of Z and written with strided stores; Z is never transposed.
//
// Workspace (Pp = P rounded up to 32; padded positions hold zeros); q, k, v
// and the bias use the operand-ordered layouts of pa_device.h:
//   q, k, v  nrows*H*Pp*32 fp16 (q scaled by log2(e)/sqrt(d))
//   g        nrows*H*Pp*32 fp16 in the layout of q, sigmoid already applied
//   bias     H*Pp*Pp fp16, log2 units (natural bias * log2(e)), zero padding
#include "pa_device.h"

namespace pa {

// --------------------------------------------------------------------------
// weight packing, once per call.
//   wimg [4*HD/32][C_IN/16][64][8] fp16: the projection operand image of
//        gamma o W (LayerNorm's scale folded into the q|k|v|g columns), in
//        the order the projection keeps it in LDS: block b of 32 columns,
//        K-step t, lane l holds column b*32 + l%32 and channels
//        t*16 + (l/32)*8 .. +7.
//   cst  [4*HD] float: beta . W per column (LayerNorm's shift), plus the gate
//        bias for the g columns.
//   woT  [C_OUT][HD] fp16: W_o transposed (the output projection operand).
// bf16 -> fp16 is exact for magnitudes in [2^-14, 65504]; smaller values
// keep an absolute error below 2^-25; larger ones saturate.
// --------------------------------------------------------------------------
__global__ void pack_weights_kernel(const bf16* __restrict__ wq, const bf16* __restrict__ wk,
                                    const bf16* __restrict__ wv, const bf16* __restrict__ wg,
                                    const bf16* __restrict__ wo, const bf16* __restrict__ gamma,
                                    f16* __restrict__ wimg, f16* __restrict__ woT, int c_in, int hd, int c_out) {
  const int ks = c_in / 16;
  const int64_t n_w = (int64_t)4 * hd / 32 * ks * 64;   // 8-element lane slots of the image
  const int64_t n_o = (int64_t)c_out * hd;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_w + n_o;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n_w) {
      const int l = (int)(i & 63), t = (int)((i >> 6) % ks), b = (int)((i >> 6) / ks);
      const int col = b * 32 + (l & 31), k0 = t * 16 + (l >> 5) * 8;
      const int tensor = col / hd, c = col % hd;
      const bf16* src = tensor == 0 ? wq : tensor == 1 ? wk : tensor == 2 ? wv : wg;
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f2h_sat(bf2f(src[(int64_t)(k0 + e) * hd + c]) * bf2f(gamma[k0 + e]));
      *reinterpret_cast<f16x8*>(wimg + i * 8) = o;
    } else {
      const int64_t j = i - n_w;
      const int c = (int)(j / hd), k = (int)(j % hd);
      woT[j] = f2h_sat(bf2f(wo[(int64_t)k * c_out + c]));
    }
  }
}

// cst[col] = sum_k beta[k] W[k][col] (+ b_g for the gate columns): one wave
// per column, fp32 partial sums over lanes, then a wave reduction.
__global__ void pack_consts_kernel(const bf16* __restrict__ wq, const bf16* __restrict__ wk,
                                   const bf16* __restrict__ wv, const bf16* __restrict__ wg,
                                   const bf16* __restrict__ beta, const bf16* __restrict__ b_g,
                                   float* __restrict__ cst, int c_in, int hd) {
  const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (col >= 4 * hd) return;
  const int tensor = col / hd, c = col % hd;
  const bf16* src = tensor == 0 ? wq : tensor == 1 ? wk : tensor == 2 ? wv : wg;
  float acc = 0.0f;
  for (int k = lane; k < c_in; k += kWave) acc += bf2f(beta[k]) * bf2f(src[(int64_t)k * hd + c]);
  acc = group_sum<kWave>(acc);
  if (lane == 0) cst[col] = acc + (tensor == 3 && b_g != nullptr ? bf2f(b_g[c]) : 0.0f);
}

// --------------------------------------------------------------------------
// Fused LayerNorm + projections.
//
// Every wave works on its own tiles of 32 positions of one row; there is no
// barrier in the tile loop.  A lane holds one position (lane % 32) and half
// of its channels, exactly the register image of the activation operand of
// a 32x32x16 MFMA: in K-step t the lane of half g holds channels
// t*16 + g*8 .. +7.  LayerNorm therefore runs in registers (one cross-half
// exchange per statistic), and the same registers serve as the A operand
// (v = X W, rows = positions) or the B operand (q, k, g: out^T = W^T X^T,
// columns = positions).  The raw rows of the next PF tiles are loaded
// before the current tile is computed.
//
// The weight operands of this workgroup's NCOL projection columns sit in
// LDS in operand order ([column block][K-step][lane][8]), copied once from
// the packed image (LayerNorm's gamma already folded in) with the column
// constants; when the pair bias is produced, so is the w_b operand (rows =
// heads, zero beyond H), folded here.
//   MODE 0: q, k, v, g          MODE 1: q, k, v, g and the pair bias
//   MODE 2: pair bias only (NCOL = 0)
// Column group blockIdx.y covers columns [y*NCOL, (y+1)*NCOL) of q|k|v|g;
// the pair bias is produced by group 0.
// --------------------------------------------------------------------------
template <int C_IN, int HD, int NCOL, int MODE>
struct ProjShape {
  static constexpr int KS = C_IN / 16;                 // MFMA K-steps
  static constexpr int NBLK = NCOL / 32;               // 32-column blocks
  static constexpr bool HAS_BIAS = MODE != 0;
  static constexpr int W_BYTES = NCOL * C_IN * 2;
  static constexpr int WB_BYTES = HAS_BIAS ? KS * 1024 : 0;
  static constexpr int LDS = W_BYTES + WB_BYTES + NCOL * 4 + 8 * 4;
  // tiles prefetched ahead (the bias-only form has registers to spare for a
  // deeper prefetch, which its pure read stream needs to cover HBM latency)
  static constexpr int PF = MODE == 2 ? (C_IN <= 128 ? 4 : 1) : (C_IN <= 128 ? 2 : 1);
  static_assert(LDS <= 160 * 1024, "projection operands exceed LDS");
};

constexpr int kProjThreads = 512;

template <int C_IN, int HD, int NCOL, int MODE>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(
    const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p, int tile_rmajor, const bf16* __restrict__ gamma,
    const bf16* __restrict__ beta, float eps, const f16* __restrict__ wimg, const float* __restrict__ cst,
    const bf16* __restrict__ wb, float q_scale, f16* __restrict__ q_ws, f16* __restrict__ k_ws,
    f16* __restrict__ v_ws, f16* __restrict__ g_ws, float* __restrict__ bias, int bias_swizzled, float bias_scale,
    int nrows, int P, int Pp, int H) {
  using SH = ProjShape<C_IN, HD, NCOL, MODE>;
  constexpr int KS = SH::KS;
  constexpr int NW = kProjThreads / kWave;
  __shared__ __attribute__((aligned(1024))) char smem[SH::LDS];
  f16* w_lds = reinterpret_cast<f16*>(smem);
  f16* wb_lds = reinterpret_cast<f16*>(smem + SH::W_BYTES);
  float* cb = reinterpret_cast<float*>(smem + SH::W_BYTES + SH::WB_BYTES);   // [NCOL] column constants
  float* cbb = cb + NCOL;                                                      // [8] pair-bias constants

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int col0 = blockIdx.y * NCOL;
  const bool do_bias = SH::HAS_BIAS && blockIdx.y == 0;

  // ---- operands into LDS (once per workgroup) ----
  // LayerNorm's affine map is folded into the projection:
  //   ((x-mu)*rstd*gamma + beta) . W = ((x-mu)*rstd) . (gamma o W) + beta . W
  // so the operands hold gamma o W and the per-column constants beta . W
  // (plus the gate bias for g columns) are added to the accumulators.  Both
  // come packed: a linear copy of this group's slice.
  {
    const f16x8* src = reinterpret_cast<const f16x8*>(wimg) + (int64_t)(col0 / 32) * KS * 64;
    f16x8* dst = reinterpret_cast<f16x8*>(w_lds);
    for (int i = tid; i < SH::NBLK * KS * 64; i += kProjThreads) dst[i] = src[i];
  }
  for (int n = tid; n < NCOL; n += kProjThreads) cb[n] = cst[col0 + n];
  if (SH::HAS_BIAS) {
    for (int i = tid; i < KS * 64; i += kProjThreads) {
      const int l = i & 63, t = i >> 6, hh = l & 31;
      const int k0 = t * 16 + (l >> 5) * 8;
      f16x8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = hh < H ? f2h_sat(bf2f(wb[(int64_t)(k0 + e) * H + hh]) * bf2f(gamma[k0 + e])) : f2h(0.0f);
      *reinterpret_cast<f16x8*>(wb_lds + i * 8) = w;
    }
    if (tid < 8) {
      float acc = 0.0f;
      if (tid < H)
        for (int k = 0; k < C_IN; ++k) acc += bf2f(beta[k]) * bf2f(wb[(int64_t)k * H + tid]);
      cbb[tid] = acc;
    }
  }
  __syncthreads();

  const int nb = Pp / 32;
  const int64_t ntiles = (int64_t)nb * nrows;
  const int64_t stride = (int64_t)gridDim.x * NW;
  // tile -> (row, first position): row-major when positions are contiguous
  // in memory, else position-block-major, so that the waves running at the
  // same time read neighbouring bytes of x.
  auto tile_rp = [&](int64_t tile, int& r, int& p0) {
    if (tile_rmajor) {
      r = (int)(tile / nb);
      p0 = (int)(tile % nb) * 32;
    } else {
      r = (int)(tile % nrows);
      p0 = (int)(tile / nrows) * 32;
    }
  };
  auto load_tile = [&](int64_t tile, bf16x8* raw) {
    if (tile < ntiles) {
      int r, p0;
      tile_rp(tile, r, p0);
      const int p = p0 + lq;
      if (p < P) {
        const bf16* src = x + (int64_t)r * xs_r + (int64_t)p * xs_p + g * 8;
#pragma unroll
        for (int t = 0; t < KS; ++t) raw[t] = ld16(src + t * 16);
        return;
      }
    }
#pragma unroll
    for (int t = 0; t < KS; ++t) raw[t] = bf16x8{};
  };

  constexpr int PF = SH::PF;
  bf16x8 pre[PF][KS];
  int64_t tile = (int64_t)blockIdx.x * NW + wave;
#pragma unroll
  for (int f = 0; f < PF; ++f) load_tile(tile + f * stride, pre[f]);

  for (; tile < ntiles; tile += stride) {
    bf16x8 raw[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) raw[t] = pre[0][t];
#pragma unroll
    for (int f = 0; f + 1 < PF; ++f)
#pragma unroll
      for (int t = 0; t < KS; ++t) pre[f][t] = pre[f + 1][t];
    load_tile(tile + PF * stride, pre[PF - 1]);

    int r, p0;
    tile_rp(tile, r, p0);
    const int p = p0 + lq;
    const bool valid = p < P;

    // ---- LayerNorm in registers (two passes, fp32); affine map folded into W ----
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += bf2f(raw[t][e]);
    s += __shfl_xor(s, 32, 64);
    const float mean = s * (1.0f / C_IN);
    float s2 = 0.0f;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = bf2f(raw[t][e]) - mean;
        s2 += d * d;
      }
    s2 += __shfl_xor(s2, 32, 64);
    const float rstd = 1.0f / __builtin_sqrtf(s2 * (1.0f / C_IN) + eps);
    f16x8 X[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) X[t][e] = f2h_sat((bf2f(raw[t][e]) - mean) * rstd);

    // ---- q | k | v | g column blocks ----
    // Register 8t+e of lane half g holds accumulator row slot_x(t, g, e), so
    // registers 8t..8t+7 are exactly this lane's 16-byte slot of chunk t of
    // the operand image: every chunk is written as one contiguous 1 KB store.
#pragma unroll 2
    for (int b = 0; b < SH::NBLK; ++b) {
      const int col = col0 + b * 32;
      const int tensor = col / HD;            // 0 q, 1 k, 2 v, 3 g
      // a NULL plane is not wanted (partial attention projects the query and
      // the key pairs separately)
      if ((tensor == 0 ? q_ws : tensor == 1 ? k_ws : tensor == 2 ? v_ws : g_ws) == nullptr) continue;
      const int hcol = col - tensor * HD;     // first column within the tensor
      const int64_t rh = (int64_t)r * H + hcol / 32;
      const int64_t chunk0 = (rh * nb + (p0 >> 5)) * 2;   // chunk of (rh, position block), t = 0
      const f16* wop = w_lds + (b * KS) * 512 + lane * 8;
      const float* cbk = cb + b * 32;
      f32x16 acc = {};
      if (tensor == 2) {                      // v = X W: rows = positions, lane = channel lq
#pragma unroll
        for (int t = 0; t < KS; ++t) acc = mfma32(X[t], *reinterpret_cast<const f16x8*>(wop + t * 512), acc);
        const float c = cbk[lq];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            o[e] = p0 + slot_x(t, g, e) < P ? f2h_sat(acc[8 * t + e] + c) : f2h(0.0f);
          st16(v_ws + (chunk0 + t) * 512 + lane * 8, o);
        }
      } else {                                // out^T = W^T X^T: rows = channels, lane = position
#pragma unroll
        for (int t = 0; t < KS; ++t) acc = mfma32(*reinterpret_cast<const f16x8*>(wop + t * 512), X[t], acc);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // channels slot_x(t, g, 0..7): two runs of four
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(cbk + 16 * t + 4 * g);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(cbk + 16 * t + 8 + 4 * g);
          f16x8 o;
          if (tensor <= 1) {
            const float sc = valid ? (tensor == 0 ? q_scale : 1.0f) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = f2h_sat((acc[8 * t + e] + c0[e]) * sc);
              o[4 + e] = f2h_sat((acc[8 * t + 4 + e] + c1[e]) * sc);
            }
            st16((tensor == 0 ? q_ws : k_ws) + (chunk0 + t) * 512 + lane * 8, o);
          } else {                            // gate: sigmoid, same layout as q
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = f2h(1.0f / (1.0f + __expf(-(acc[8 * t + e] + c0[e]))));
              o[4 + e] = f2h(1.0f / (1.0f + __expf(-(acc[8 * t + 4 + e] + c1[e]))));
            }
            st16(g_ws + (chunk0 + t) * 512 + lane * 8, o);
          }
        }
      }
    }

    // ---- pair bias: rows = heads (zero beyond H), columns = positions ----
    if (do_bias) {
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KS; ++t)
        acc = mfma32(*reinterpret_cast<const f16x8*>(wb_lds + t * 512 + lane * 8), X[t], acc);
      if (bias_swizzled) {   // attention layout: fp16, log2 units, padded to Pp x Pp with zeros
        f16* b16 = reinterpret_cast<f16*>(bias);
#pragma unroll
        for (int j = 0; j < 4; ++j) {          // heads (< 8) are rows g*4 + j of registers 0..3
          const int hh = acc_row(j, g);
          if (hh < H) {
            b16[b16_off(hh, nb, nb, r, p)] = valid ? f2h_sat((acc[j] + cbb[hh]) * bias_scale) : f2h(0.0f);
            if (r == P - 1)   // the padded query rows get zeros at the same keys
              for (int rp = P; rp < Pp; ++rp) b16[b16_off(hh, nb, nb, rp, p)] = f2h(0.0f);
          }
        }
      } else if (valid) {    // caller layout [H][P][P] float
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int hh = acc_row(j, g);
          if (hh < H) bias[((int64_t)hh * P + r) * P + p] = (acc[j] + cbb[hh]) * bias_scale;
        }
      }
    }
  }
}

// Copy of a caller-provided bias [H][Pq][Pk] (float, natural-log units) into
// the attention layout (fp16 operand order, log2 units, Ppq x Ppk with zero
// padding).  Each thread writes one lane's 16-byte slot of a chunk, so the
// stores of a wave are one contiguous 1 KB; its 8 keys are two runs of 4 in
// the source row.
__global__ void bias_to_attn_layout_kernel(const float* __restrict__ src, f16* __restrict__ dst, int H, int Pq,
                                           int Pk, int Ppq, int Ppk) {
  const int nbq = Ppq / 32, nbk = Ppk / 32;
  const int64_t slots = (int64_t)H * nbq * nbk * 2 * 64;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < slots; i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const int64_t c = i >> 6;                         // chunk (h, qb, kb, t)
    const int t = (int)(c & 1);
    const int kb = (int)((c >> 1) % nbk);
    const int64_t hq = (c >> 1) / nbk;
    const int qb = (int)(hq % nbq), h = (int)(hq / nbq);
    const int q = qb * 32 + (lane & 31), hg = lane >> 5;
    const float* row = src + ((int64_t)h * Pq + q) * Pk;
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = kb * 32 + slot_x(t, hg, e);
      o[e] = (q < Pq && k < Pk) ? f2h_sat(row[k] * kLog2e) : f2h(0.0f);
    }
    *reinterpret_cast<f16x8*>(dst + i * 8) = o;
  }
}

}  // namespace pa

// ----------------------------------------------------------------------------
// launchers (called from the host API in pairattn_api.hip)
// ----------------------------------------------------------------------------
#include <atomic>

#include "pa_launch.h"

namespace pa {

hipError_t launch_bias_to_attn_layout(const float* src, void* dst, int H, int Pq, int Pk, int Ppq, int Ppk,
                                      hipStream_t s) {
  const int64_t slots = (int64_t)H * Ppq * Ppk / 8;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((slots + 255) / 256, 16384));
  hipLaunchKernelGGL(bias_to_attn_layout_kernel, dim3(blocks), dim3(256), 0, s, src, (f16*)dst, H, Pq, Pk, Ppq,
                     Ppk);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const PackArgs& a, hipStream_t s) {
  if (a.c_in % 16 != 0 || a.hd % 32 != 0) return hipErrorInvalidValue;
  const int64_t total = (int64_t)4 * a.hd * a.c_in / 8 + (int64_t)a.c_out * a.hd;
  const int threads = 256;
  const int blocks = (int)std::min<int64_t>((total + threads - 1) / threads, 4096);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(threads), 0, s, (const bf16*)a.wq, (const bf16*)a.wk,
                     (const bf16*)a.wv, (const bf16*)a.wg, (const bf16*)a.wo, (const bf16*)a.gamma, (f16*)a.wT,
                     (f16*)a.woT, a.c_in, a.hd, a.c_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cols = 4 * a.hd, per_block = threads / kWave;
  hipLaunchKernelGGL(pack_consts_kernel, dim3((cols + per_block - 1) / per_block), dim3(threads), 0, s,
                     (const bf16*)a.wq, (const bf16*)a.wk, (const bf16*)a.wv, (const bf16*)a.wg, (const bf16*)a.beta,
                     (const bf16*)a.b_g, a.cst, a.c_in, a.hd);
  return hipGetLastError();
}

template <int C_IN, int HD, int MODE>
static hipError_t proj_dispatch(const ProjArgs& a, int num_cu, hipStream_t s) {
  // columns per group: all of q|k|v|g when their operands fit in 128 KB of LDS
  constexpr int NCOL = MODE == 2 ? 0 : std::min(4 * HD, 65536 / C_IN);
  constexpr int groups = MODE == 2 ? 1 : 4 * HD / NCOL;
  const int64_t ntiles = (int64_t)(a.Pp / 32) * a.nrows;
  // resident workgroups per CU (registers and LDS), asked once per instance;
  // concurrent first calls ask the same question and store the same answer
  static std::atomic<int> wg_cache{0};
  int wg_per_cu = wg_cache.load(std::memory_order_relaxed);
  if (wg_per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, proj_kernel<C_IN, HD, NCOL, MODE>, kProjThreads, 0) !=
            hipSuccess ||
        n < 1)
      n = 1;
    wg_per_cu = n;
    wg_cache.store(n, std::memory_order_relaxed);
  }
  const int64_t want = (ntiles + kProjThreads / kWave - 1) / (kProjThreads / kWave);
  // one resident wave of workgroups: the column groups of a position range
  // run at the same time (their reads of x meet in the caches) and each CU
  // fills its LDS operands once
  const int grid_x = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)num_cu * wg_per_cu / groups));
  const int rmajor = a.xs_p <= a.xs_r ? 1 : 0;
  hipLaunchKernelGGL((proj_kernel<C_IN, HD, NCOL, MODE>), dim3(grid_x, groups), dim3(kProjThreads), 0, s,
                     (const bf16*)a.x, a.xs_r, a.xs_p, rmajor, (const bf16*)a.gamma, (const bf16*)a.beta, a.eps,
                     (const f16*)a.wT, a.cst, (const bf16*)a.wb, a.q_scale, (f16*)a.q_ws,
                     (f16*)a.k_ws, (f16*)a.v_ws, (f16*)a.g_ws, a.bias, a.bias_swizzled, a.bias_scale, a.nrows, a.P,
                     a.Pp, a.H);
  return hipGetLastError();
}

template <int C_IN, int MODE>
static hipError_t proj_dispatch_hd(const ProjArgs& a, int num_cu, hipStream_t s) {
  if (MODE == 2) return proj_dispatch<C_IN, 128, 2>(a, num_cu, s);
  if (a.hd == 128) return proj_dispatch<C_IN, 128, MODE>(a, num_cu, s);
  if (a.hd == 256) return proj_dispatch<C_IN, 256, MODE>(a, num_cu, s);
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t proj_dispatch_c(const ProjArgs& a, int num_cu, hipStream_t s) {
  switch (a.c_in) {
    case 64: return proj_dispatch_hd<64, MODE>(a, num_cu, s);
    case 128: return proj_dispatch_hd<128, MODE>(a, num_cu, s);
    case 256: return proj_dispatch_hd<256, MODE>(a, num_cu, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_proj_bf16(const ProjArgs& a, int mode, int num_cu, hipStream_t s) {
  switch (mode) {
    case 0: return proj_dispatch_c<0>(a, num_cu, s);
    case 1: return proj_dispatch_c<1>(a, num_cu, s);
    case 2: return proj_dispatch_c<2>(a, num_cu, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
