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
// Workspace (Pp = P rounded up to 32); q, k, v and the bias use the
// operand-ordered layouts of pa_device.h:
//   q, k, v  nrows*H*Pp*32 fp16 (q scaled by log2(e)/sqrt(d)); padded
//            positions: v zero, q and k finite (keys past P are dropped by
//            every sweep, queries past P never stored)
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
__device__ void pack_weights(const bf16* __restrict__ wq, const bf16* __restrict__ wk, const bf16* __restrict__ wv,
                             const bf16* __restrict__ wg, const bf16* __restrict__ wo, const bf16* __restrict__ gamma,
                             f16* __restrict__ wimg, f16* __restrict__ woT, int c_in, int hd, int c_out) {
  // q columns carry the logit scale log2(e)/sqrt(d) and the gate columns
  // -log2(e): the projection then stores q = acc + c and forms the gate as
  // 1 / (1 + 2^(acc + c)) with no multiply per element
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
      const float sc = column_scale(tensor);
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f2h_sat(bf2f(src[(int64_t)(k0 + e) * hd + c]) * bf2f(gamma[k0 + e]) * sc);
      *reinterpret_cast<f16x8*>(wimg + i * 8) = o;
    } else {
      const int64_t j = i - n_w;
      const int c = (int)(j / hd), k = (int)(j % hd);
      woT[j] = f2h_sat(bf2f(wo[(int64_t)k * c_out + c]));
    }
  }
}

// cst[col] = (sum_k beta[k] W[k][col] (+ b_g for the gate columns)) times the
// column's scale: one wave per column, fp32 partial sums over lanes, then a
// wave reduction.
__device__ void pack_consts(const bf16* __restrict__ wq, const bf16* __restrict__ wk, const bf16* __restrict__ wv,
                            const bf16* __restrict__ wg, const bf16* __restrict__ beta, const bf16* __restrict__ b_g,
                            float* __restrict__ cst, int c_in, int hd) {
  const int col = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (col >= 4 * hd) return;
  const int tensor = col / hd, c = col % hd;
  const bf16* src = tensor == 0 ? wq : tensor == 1 ? wk : tensor == 2 ? wv : wg;
  float acc = 0.0f;
  for (int k = lane; k < c_in; k += kWave) acc += bf2f(beta[k]) * bf2f(src[(int64_t)k * hd + c]);
  acc = group_sum<kWave>(acc);
  if (lane == 0) cst[col] = (acc + (tensor == 3 && b_g != nullptr ? bf2f(b_g[c]) : 0.0f)) * column_scale(tensor);
}

// One launch for both: blockIdx.y = 0 packs the weights, 1 the constants.
// The pair-bias operand of the projection: w_b [c_in][H] with the
// LayerNorm gamma of the biased tensor folded in, in the order the
// projection keeps it in LDS (rows = heads, zero beyond H), and the
// constants beta . w_b per head (pair_bias_const, as where the projection
// builds the operand itself).
__device__ void pack_bias_operand(const bf16* __restrict__ wb, const bf16* __restrict__ gamma,
                                  const bf16* __restrict__ beta, f16* __restrict__ img, float* __restrict__ cbb,
                                  int c_in, int H) {
  const int ks = c_in / 16;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < ks * 64; i += gridDim.x * blockDim.x) {
    const int l = i & 63, t = i >> 6, hh = l & 31;
    const int k0 = t * 16 + (l >> 5) * 8;
    f16x8 w;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      w[e] = hh < H ? f2h_sat(bf2f(wb[(int64_t)(k0 + e) * H + hh]) * bf2f(gamma[k0 + e])) : f2h(0.0f);
    *reinterpret_cast<f16x8*>(img + i * 8) = w;
  }
  // constants: one wave per head, heads 0..7 over the first two blocks
  const int hh = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (hh < 8) {
    const float c = hh < H ? pair_bias_const(beta, wb, c_in, H, hh) : 0.0f;
    if (threadIdx.x % kWave == 0) cbb[hh] = c;
  }
}

// One launch for a call's preparation, by blockIdx.y: 0 the q|k|v|g operand
// image and W_o^T, 1 the column constants, 2 the pair-bias operand (when
// wb_img is set), 3 the keep bits and key-block ranges of the mask rows
// (when bits is set; one wave per row).
__global__ void pack_kernel(const bf16* __restrict__ wq, const bf16* __restrict__ wk, const bf16* __restrict__ wv,
                            const bf16* __restrict__ wg, const bf16* __restrict__ wo, const bf16* __restrict__ gamma,
                            const bf16* __restrict__ beta, const bf16* __restrict__ b_g, f16* __restrict__ wimg,
                            f16* __restrict__ woT, float* __restrict__ cst, int c_in, int hd, int c_out,
                            const bf16* __restrict__ wb, const bf16* __restrict__ b_gamma,
                            const bf16* __restrict__ b_beta, f16* __restrict__ wb_img, float* __restrict__ wb_cst,
                            int b_c_in, int H, const uint8_t* __restrict__ mask, int64_t ms_r, int64_t ms_k,
                            uint32_t* __restrict__ bits, int* __restrict__ range, int nrows, int P, int nkb) {
  if (blockIdx.y == 0) {
    pack_weights(wq, wk, wv, wg, wo, gamma, wimg, woT, c_in, hd, c_out);
  } else if (blockIdx.y == 1) {
    pack_consts(wq, wk, wv, wg, beta, b_g, cst, c_in, hd);
  } else if (blockIdx.y == 2) {
    if (wb_img != nullptr) pack_bias_operand(wb, b_gamma, b_beta, wb_img, wb_cst, b_c_in, H);
  } else if (bits != nullptr) {
    const int64_t row = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kWave;
    if (row < nrows)   // uniform over the wave
      mask_bits_row(mask != nullptr ? mask + row * ms_r : nullptr, ms_k, bits + row * nkb, range + row * 2, P, nkb);
  }
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
// Tiles prefetched ahead by default: the bias-only form has registers to
// spare for a deeper prefetch, which its pure read stream needs to cover
// HBM latency when each wave loops over many tiles.
template <int C_IN, int MODE>
constexpr int proj_prefetch() {
  return MODE == 2 ? (C_IN <= 128 ? 4 : 1) : (C_IN <= 128 ? 2 : 1);
}

template <int C_IN, int HD, int NCOL, int MODE, int PF_ = proj_prefetch<C_IN, MODE>()>
struct ProjShape {
  static constexpr int KS = C_IN / 16;                 // MFMA K-steps
  static constexpr int NBLK = NCOL / 32;               // 32-column blocks
  static constexpr bool HAS_BIAS = MODE != 0;
  static constexpr int W_BYTES = NCOL * C_IN * 2;
  static constexpr int WB_BYTES = HAS_BIAS ? KS * 1024 : 0;
  static constexpr int LDS = W_BYTES + WB_BYTES + NCOL * 4 + 8 * 4;
  static constexpr int PF = PF_;
  static_assert(PF >= 1, "prefetch depth");
  static_assert(LDS <= 160 * 1024, "projection operands exceed LDS");
};

constexpr int kProjThreads = 512;

// tile -> (row, first position): row-major when positions are contiguous in
// memory, else position-block-major, so that the waves running at the same
// time read neighbouring bytes of x.
__device__ __forceinline__ void proj_tile_rp(int64_t tile, int nb, int nrows, int rmajor, int& r, int& p0) {
  if (rmajor) {
    r = (int)(tile / nb);
    p0 = (int)(tile % nb) * 32;
  } else {
    r = (int)(tile % nrows);
    p0 = (int)(tile / nrows) * 32;
  }
}

// The raw rows of a tile into raw[t] (channels t*16 + half*8 .. +7 of the
// lane's position; zeros past the last tile and past P).  lane_off is the
// lane's element offset within a tile; the tile's own offset is
// wave-uniform and computed on the scalar unit.
template <int KS>
__device__ __forceinline__ void proj_load_tile(const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p,
                                               int64_t lane_off, int64_t tile, int64_t ntiles, int nb, int nrows,
                                               int rmajor, int P, int lq, bf16x8 (&raw)[KS]) {
  if (tile < ntiles) {
    int r, p0;
    proj_tile_rp(tile, nb, nrows, rmajor, r, p0);
    if (p0 + lq < P) {
      const bf16* src = x + ((int64_t)r * xs_r + (int64_t)p0 * xs_p) + lane_off;
#pragma unroll
      for (int t = 0; t < KS; ++t) raw[t] = ld16(src + t * 16);
      return;
    }
  }
#pragma unroll
  for (int t = 0; t < KS; ++t) raw[t] = bf16x8{};
}

// LayerNorm of the lane's position in registers (two passes, fp32, one
// cross-half exchange per statistic) into the fp16 activation operand; the
// affine map is folded into the packed weights.  |x - mean| * rstd <=
// sqrt(C_IN - 1) < 16 for any row: no saturation needed.
template <int KS>
__device__ __forceinline__ void proj_layernorm(const bf16x8 (&raw)[KS], float eps, f16x8 (&X)[KS]) {
  constexpr float inv_c = 1.0f / (KS * 16);
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += bf2f(raw[t][e]);
  s += __shfl_xor(s, 32, 64);
  const float mean = s * inv_c;
  float s2 = 0.0f;
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = bf2f(raw[t][e]) - mean;
      s2 += d * d;
    }
  s2 += __shfl_xor(s2, 32, 64);
  const float rstd = 1.0f / __builtin_sqrtf(s2 * inv_c + eps);
#pragma unroll
  for (int t = 0; t < KS; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) X[t][e] = f2h((bf2f(raw[t][e]) - mean) * rstd);
}

// One 32-column block (first column col) of q|k|v|g for the tile of
// positions p0 .. p0+31 of row r: the products of the normalised tile X with
// the block's operand (wop: this lane's slot of K-step 0, K-steps 512 halfs
// apart), + the block's column constants cbk, in the layout of its tensor.
// The result is this lane's two 16-byte slots (chunks t = 0, 1 of the
// tile's operand image, 512 halfs apart) and where they go (NULL: a plane
// that is not wanted; partial attention projects the query and the key
// pairs separately).
struct QkvgOut {
  f16* dst;
  f16x8 o[2];
};
template <int KS, int HD>
__device__ __forceinline__ QkvgOut qkvg_block(const f16x8 (&X)[KS], const f16* wop, const float* cbk, int col, int r,
                                              int p0, int P, int H, int nb, int nrows, int lane, f16* q_ws,
                                              f16* k_ws, f16* v_ws, f16* g_ws) {
  const int lq = lane & 31, g = lane >> 5;
  const int tensor = col / HD;            // 0 q, 1 k, 2 v, 3 g
  f16* plane = tensor == 0 ? q_ws : tensor == 1 ? k_ws : tensor == 2 ? v_ws : g_ws;
  QkvgOut res;
  res.dst = nullptr;
  if (plane == nullptr) return res;
  const int hcol = col - tensor * HD;     // first column within the tensor
  const int64_t rh = (int64_t)r * H + hcol / 32;
  const int64_t chunk0 = (rh * nb + (p0 >> 5)) * 2;   // chunk of (rh, position block), t = 0
  PA_DCHECK((chunk0 + 2) * 512 <= (int64_t)nrows * H * nb * 1024, 4);
  res.dst = plane + chunk0 * 512 + lane * 8;
  // Register 8t+e of lane half g holds accumulator row slot_x(t, g, e), so
  // registers 8t..8t+7 are exactly this lane's 16-byte slot of chunk t of
  // the operand image: every chunk is written as one contiguous 1 KB store.
  f32x16 acc = {};
  if (tensor == 2) {                      // v = X W: rows = positions, lane = channel lq
#pragma unroll
    for (int t = 0; t < KS; ++t) acc = mfma32(X[t], *reinterpret_cast<const f16x8*>(wop + t * 512), acc);
    const float c = cbk[lq];
    const bool full_tile = p0 + 32 <= P;   // uniform: no padded position in this tile
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (full_tile) {
#pragma unroll
        for (int e = 0; e < 8; ++e) res.o[t][e] = f2h_sat(acc[8 * t + e] + c);
      } else {   // padded positions (keys past P) hold zeros: their weight is 0, so P.V must see 0
#pragma unroll
        for (int e = 0; e < 8; ++e)
          res.o[t][e] = p0 + slot_x(t, g, e) < P ? f2h_sat(acc[8 * t + e] + c) : f2h(0.0f);
      }
    }
  } else {                                // out^T = W^T X^T: rows = channels, lane = position
#pragma unroll
    for (int t = 0; t < KS; ++t) acc = mfma32(*reinterpret_cast<const f16x8*>(wop + t * 512), X[t], acc);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // channels slot_x(t, g, 0..7): two runs of four
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cbk + 16 * t + 4 * g);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(cbk + 16 * t + 8 + 4 * g);
      if (tensor <= 1) {
        // q (scale folded into its columns) and k; padded positions keep
        // finite values: every sweep drops keys past P, and queries past
        // P are never stored
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          res.o[t][e] = f2h_sat(acc[8 * t + e] + c0[e]);
          res.o[t][4 + e] = f2h_sat(acc[8 * t + 4 + e] + c1[e]);
        }
      } else {                            // gate: sigmoid, same layout as q
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          res.o[t][e] = f2h(sigmoid_from_log2(acc[8 * t + e] + c0[e]));
          res.o[t][4 + e] = f2h(sigmoid_from_log2(acc[8 * t + 4 + e] + c1[e]));
        }
      }
    }
  }
  return res;
}
__device__ __forceinline__ void qkvg_store(const QkvgOut& b) {
  if (b.dst == nullptr) return;
  st16(b.dst, b.o[0]);
  st16(b.dst + 512, b.o[1]);
}

template <int C_IN, int HD, int NCOL, int MODE, int PF_ = proj_prefetch<C_IN, MODE>()>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(
    const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p, int tile_rmajor, const bf16* __restrict__ gamma,
    const bf16* __restrict__ beta, float eps, const f16* __restrict__ wimg, const float* __restrict__ cst,
    const bf16* __restrict__ wb, f16* __restrict__ q_ws, f16* __restrict__ k_ws,
    f16* __restrict__ v_ws, f16* __restrict__ g_ws, float* __restrict__ bias, int bias_swizzled, float bias_scale,
    int nrows, int P, int Pp, int H, const f16* __restrict__ wb_img, const float* __restrict__ wb_cst) {
  using SH = ProjShape<C_IN, HD, NCOL, MODE, PF_>;
  constexpr int KS = SH::KS;
  constexpr int NW = kProjThreads / kWave;
  __shared__ __attribute__((aligned(1024))) char smem[SH::LDS];
  f16* w_lds = reinterpret_cast<f16*>(smem);
  f16* wb_lds = reinterpret_cast<f16*>(smem + SH::W_BYTES);
  float* cb = reinterpret_cast<float*>(smem + SH::W_BYTES + SH::WB_BYTES);   // [NCOL] column constants
  float* cbb = cb + NCOL;                                                      // [8] pair-bias constants

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
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
  if (SH::HAS_BIAS && wb_img != nullptr) {   // built by the preparation launch
    for (int i = tid; i < KS * 64; i += kProjThreads)
      *reinterpret_cast<f16x8*>(wb_lds + i * 8) = *reinterpret_cast<const f16x8*>(wb_img + i * 8);
    if (tid < 8) cbb[tid] = wb_cst[tid];
  } else if (SH::HAS_BIAS) {
    for (int i = tid; i < KS * 64; i += kProjThreads) {
      const int l = i & 63, t = i >> 6, hh = l & 31;
      const int k0 = t * 16 + (l >> 5) * 8;
      f16x8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = hh < H ? f2h_sat(bf2f(wb[(int64_t)(k0 + e) * H + hh]) * bf2f(gamma[k0 + e])) : f2h(0.0f);
      *reinterpret_cast<f16x8*>(wb_lds + i * 8) = w;
    }
    {   // one wave per head (8 waves)
      const float c = wave < H ? pair_bias_const(beta, wb, C_IN, H, wave) : 0.0f;
      if (lane == 0) cbb[wave] = c;
    }
  }
  __syncthreads();

  const int nb = Pp / 32;
  const int64_t ntiles = (int64_t)nb * nrows;
  const int64_t stride = (int64_t)gridDim.x * NW;
  const int64_t lane_off = (int64_t)lq * xs_p + g * 8;
  auto load_tile = [&](int64_t tile, bf16x8 (&raw)[KS]) {
    proj_load_tile<KS>(x, xs_r, xs_p, lane_off, tile, ntiles, nb, nrows, tile_rmajor, P, lq, raw);
  };

  constexpr int PF = SH::PF;
  bf16x8 pre[PF][KS];
  int64_t tile = (int64_t)blockIdx.x * NW + wave;
#pragma unroll
  for (int f = 0; f < PF; ++f) load_tile(tile + f * stride, pre[f]);

  // The PF buffers take the tiles in turn (unrolled, so that each is a fixed
  // set of registers): a tile's rows are read by LayerNorm, then its buffer
  // is refilled with the tile PF strides ahead.
  while (tile < ntiles) {
#pragma unroll
   for (int u = 0; u < PF; ++u) {
    if (tile >= ntiles) break;

    int r, p0;
    proj_tile_rp(tile, nb, nrows, tile_rmajor, r, p0);
    const int p = p0 + lq;
    const bool valid = p < P;

    f16x8 X[KS];
    proj_layernorm<KS>(pre[u], eps, X);
    load_tile(tile + PF * stride, pre[u]);

    // ---- q | k | v | g column blocks ----
#pragma unroll 4
    for (int b = 0; b < SH::NBLK; ++b)
      qkvg_store(qkvg_block<KS, HD>(X, w_lds + (b * KS) * 512 + lane * 8, cb + b * 32, col0 + b * 32, r, p0, P, H,
                                    nb, nrows, lane, q_ws, k_ws, v_ws, g_ws));

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
            PA_DCHECK(b16_off(hh, nb, nb, r, p) < (int64_t)H * nb * nb * 1024, 5);
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
    tile += stride;
   }
  }
}

// LayerNorm + q|k|v|g where the operands of all 4*HD columns exceed the LDS
// (C_IN = 256: 512 KB).  proj_kernel would split the columns over workgroups
// and normalise every tile once per group; here a workgroup normalises a
// batch of 8 position tiles once (one per wave, held in registers) and
// streams the packed operand through LDS in slices of 4 column blocks,
// double-buffered: the copy of slice s+1 (8 KB per wave, global -> LDS
// without registers) is issued at the start of slice s and waited for at its
// end, where one barrier hands both buffers over.  Each wave holds back the
// stores of a slice's last block until after that barrier, so that the wait
// finds only stores issued a block or more earlier.
template <int C_IN, int HD>
struct ProjStreamShape {
  static constexpr int KS = C_IN / 16;
  static constexpr int SBLK = 4;                   // 32-column blocks per slice
  static constexpr int NS = 4 * HD / 32 / SBLK;    // slices
  static constexpr int SLICE = SBLK * KS * 512;    // halfs per slice
  static constexpr int LDS = 2 * SLICE * 2 + 4 * HD * 4;
  static_assert(NS % 2 == 0, "slice s lives in buffer s % 2 across batches");
  static_assert(SLICE * 2 % (kProjThreads * 16) == 0, "a slice is whole rounds of 16 bytes per thread");
  static_assert(LDS <= 160 * 1024, "slice buffers exceed LDS");
};

template <int C_IN, int HD>
__global__ __launch_bounds__(kProjThreads) void proj_stream_kernel(
    const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p, int tile_rmajor, float eps,
    const f16* __restrict__ wimg, const float* __restrict__ cst, f16* __restrict__ q_ws, f16* __restrict__ k_ws,
    f16* __restrict__ v_ws, f16* __restrict__ g_ws, int nrows, int P, int Pp, int H) {
  using SH = ProjStreamShape<C_IN, HD>;
  constexpr int KS = SH::KS, SBLK = SH::SBLK, NS = SH::NS, SLICE = SH::SLICE;
  constexpr int NW = kProjThreads / kWave;
  constexpr int ROUNDS = SLICE * 2 / (kProjThreads * 16);   // 16-byte copies per thread and slice
  __shared__ __attribute__((aligned(1024))) f16 w_lds[2 * SLICE];
  __shared__ float cb[4 * HD];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int nb = Pp / 32;
  const int64_t ntiles = (int64_t)nb * nrows;
  const int64_t nbatch = (ntiles + NW - 1) / NW;
  int64_t batch = blockIdx.x;
  if (batch >= nbatch) return;   // the whole workgroup

  // slice s of the packed image (column blocks s*SBLK ..) into buffer s % 2:
  // a round of a wave is one contiguous 1 KB in the image and in LDS
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)w_lds;
  auto copy_slice = [&](int s) {
    const char* src = reinterpret_cast<const char*>(wimg + (int64_t)s * SLICE) + wave * 1024;
    const uint32_t dst = lds0 + (uint32_t)((s & 1) * SLICE * 2 + wave * 1024);
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k) {
      PA_DCHECK((int64_t)s * SLICE * 2 + k * kProjThreads * 16 + wave * 1024 + 1024 <= (int64_t)NS * SLICE * 2, 8);
      g2lds16_sbase(src + k * kProjThreads * 16, lane * 16, dst + k * kProjThreads * 16);
    }
  };
  auto handover = [&]() {   // this wave's copies, stores and loads done, then the workgroup's
    wait_vm0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int64_t lane_off = (int64_t)lq * xs_p + g * 8;
  auto load_tile = [&](int64_t tile, bf16x8 (&raw)[KS]) {
    proj_load_tile<KS>(x, xs_r, xs_p, lane_off, tile, ntiles, nb, nrows, tile_rmajor, P, lq, raw);
  };

  for (int n = tid; n < 4 * HD; n += kProjThreads) cb[n] = cst[n];
  copy_slice(0);
  bf16x8 raw[KS];
  load_tile(batch * NW + wave, raw);
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the constants are in LDS
  handover();

  for (; batch < nbatch; batch += gridDim.x) {
    const int64_t tile = batch * NW + wave;
    const bool more = batch + gridDim.x < nbatch;   // workgroup-uniform
    const bool mine = tile < ntiles;                // wave-uniform
    int r = 0, p0 = 0;
    if (mine) proj_tile_rp(tile, nb, nrows, tile_rmajor, r, p0);
    f16x8 X[KS];
    proj_layernorm<KS>(raw, eps, X);
    if (more) load_tile(tile + (int64_t)gridDim.x * NW, raw);
    QkvgOut held;
    held.dst = nullptr;
    for (int s = 0; s < NS; ++s) {
      if (s + 1 < NS) copy_slice(s + 1);
      else if (more) copy_slice(0);
      qkvg_store(held);   // the last block of the slice before (issued after its handover)
      held.dst = nullptr;
      if (mine) {
        const f16* wbuf = w_lds + (s & 1) * SLICE + lane * 8;
#pragma unroll
        for (int j = 0; j < SBLK; ++j) {
          const int b = s * SBLK + j;
          const QkvgOut o = qkvg_block<KS, HD>(X, wbuf + j * KS * 512, cb + b * 32, b * 32, r, p0, P, H, nb, nrows,
                                               lane, q_ws, k_ws, v_ws, g_ws);
          if (j + 1 < SBLK) qkvg_store(o);
          else held = o;
        }
      }
      handover();   // slice s+1 in its buffer; every wave is done with buffer s % 2
    }
    qkvg_store(held);
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

hipError_t debug_take_bf16(unsigned int* out) { return pa_debug_take(out); }

hipError_t launch_pack_bf16(const PackArgs& a, hipStream_t s) {
  if (a.c_in % 16 != 0 || a.hd % 32 != 0) return hipErrorInvalidValue;
  if (a.wb_img != nullptr && (a.b_c_in % 16 != 0 || a.b_c_in > 256 || a.H < 1 || a.H > 8)) return hipErrorInvalidValue;
  const int64_t total = (int64_t)4 * a.hd * a.c_in / 8 + (int64_t)a.c_out * a.hd;
  const int threads = 256;
  const int blocks_w = (int)std::min<int64_t>((total + threads - 1) / threads, 4096);   // grid-stride
  const int cols = 4 * a.hd, per_block = threads / kWave;
  const int blocks_c = (cols + per_block - 1) / per_block;                              // one wave per column
  // (at least two blocks: their eight waves form the eight head constants)
  const int blocks_b = a.wb_img != nullptr ? std::max(2, (a.b_c_in / 16 * 64 + threads - 1) / threads) : 0;
  const int blocks_m = a.bits != nullptr ? (a.nrows + per_block - 1) / per_block : 0;   // one wave per row
  const int blocks = std::max(std::max(blocks_w, blocks_c), std::max(blocks_b, blocks_m));
  hipLaunchKernelGGL(pack_kernel, dim3(blocks, a.bits != nullptr ? 4 : a.wb_img != nullptr ? 3 : 2), dim3(threads), 0,
                     s, (const bf16*)a.wq, (const bf16*)a.wk, (const bf16*)a.wv, (const bf16*)a.wg,
                     (const bf16*)a.wo, (const bf16*)a.gamma, (const bf16*)a.beta, (const bf16*)a.b_g, (f16*)a.wT,
                     (f16*)a.woT, a.cst, a.c_in, a.hd, a.c_out, (const bf16*)a.wb, (const bf16*)a.b_gamma,
                     (const bf16*)a.b_beta, (f16*)a.wb_img, a.wb_cst, a.b_c_in, a.H, a.mask, a.ms_r, a.ms_k, a.bits,
                     a.bits != nullptr ? mask_range_of(a.bits, a.nrows, a.nkb) : nullptr, a.nrows, a.P, a.nkb);
  return hipGetLastError();
}

// resident workgroups of a kernel per CU (registers and LDS), asked once per
// instance; concurrent first calls ask the same question and store the same
// answer
template <typename K>
static int resident_per_cu(K kernel, std::atomic<int>& cache) {
  int n = cache.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kProjThreads, 0) != hipSuccess || n < 1) n = 1;
    cache.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int C_IN, int HD, int NCOL, int MODE, int PF>
static hipError_t proj_launch(const ProjArgs& a, int wg_per_cu, int64_t ntiles, int num_cu, int groups,
                              hipStream_t s) {
  const int64_t want = (ntiles + kProjThreads / kWave - 1) / (kProjThreads / kWave);
  // one resident wave of workgroups: the column groups of a position range
  // run at the same time (their reads of x meet in the caches) and each CU
  // fills its LDS operands once
  const int grid_x = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)num_cu * wg_per_cu / groups));
  const int rmajor = a.xs_p <= a.xs_r ? 1 : 0;
  hipLaunchKernelGGL((proj_kernel<C_IN, HD, NCOL, MODE, PF>), dim3(grid_x, groups), dim3(kProjThreads), 0, s,
                     (const bf16*)a.x, a.xs_r, a.xs_p, rmajor, (const bf16*)a.gamma, (const bf16*)a.beta, a.eps,
                     (const f16*)a.wT, a.cst, (const bf16*)a.wb, (f16*)a.q_ws,
                     (f16*)a.k_ws, (f16*)a.v_ws, (f16*)a.g_ws, a.bias, a.bias_swizzled, a.bias_scale, a.nrows, a.P,
                     a.Pp, a.H, (const f16*)a.wb_img, a.wb_cst);
  return hipGetLastError();
}

template <int C_IN, int HD, int MODE>
static hipError_t proj_dispatch(const ProjArgs& a, int num_cu, hipStream_t s) {
  // columns per group: all of q|k|v|g when their operands fit in 128 KB of LDS
  constexpr int NCOL = MODE == 2 ? 0 : std::min(4 * HD, 65536 / C_IN);
  constexpr int groups = MODE == 2 ? 1 : 4 * HD / NCOL;
  const int64_t ntiles = (int64_t)(a.Pp / 32) * a.nrows;
  if constexpr (MODE == 0 && groups > 1) {
    // q|k|v|g only, operands larger than the LDS: one normalisation per tile
    // with the operand streamed (persistent, batches of 8 tiles)
    static std::atomic<int> wg_cache{0};
    const int wg_per_cu = resident_per_cu(proj_stream_kernel<C_IN, HD>, wg_cache);
    const int64_t nbatch = (ntiles + kProjThreads / kWave - 1) / (kProjThreads / kWave);
    const int grid_x = (int)std::max<int64_t>(1, std::min<int64_t>(nbatch, (int64_t)num_cu * wg_per_cu));
    const int rmajor = a.xs_p <= a.xs_r ? 1 : 0;
    hipLaunchKernelGGL((proj_stream_kernel<C_IN, HD>), dim3(grid_x), dim3(kProjThreads), 0, s, (const bf16*)a.x,
                       a.xs_r, a.xs_p, rmajor, a.eps, (const f16*)a.wT, a.cst, (f16*)a.q_ws, (f16*)a.k_ws,
                       (f16*)a.v_ws, (f16*)a.g_ws, a.nrows, a.P, a.Pp, a.H);
    return hipGetLastError();
  }
  if constexpr (MODE == 2 && proj_prefetch<C_IN, MODE>() > 1) {
    // The bias alone of a small tensor: when a wave of the grid has at most
    // four tiles, a one-tile prefetch is faster (measured at Z[384,384,128],
    // 2.25 tiles per wave: 20.8 -> 17.1 us); with hundreds of tiles per wave
    // (4096 residues) the deep prefetch is 2% faster.
    static std::atomic<int> shallow_cache{0};
    const int wg_shallow = resident_per_cu(proj_kernel<C_IN, HD, NCOL, MODE, 1>, shallow_cache);
    if (ntiles <= (int64_t)4 * num_cu * wg_shallow * (kProjThreads / kWave))
      return proj_launch<C_IN, HD, NCOL, MODE, 1>(a, wg_shallow, ntiles, num_cu, groups, s);
  }
  static std::atomic<int> wg_cache{0};
  const int wg_per_cu = resident_per_cu(proj_kernel<C_IN, HD, NCOL, MODE>, wg_cache);
  return proj_launch<C_IN, HD, NCOL, MODE, proj_prefetch<C_IN, MODE>()>(a, wg_per_cu, ntiles, num_cu, groups, s);
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
