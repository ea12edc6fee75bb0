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
//   g        [nrows][P][H*32] fp16, sigmoid already applied
//   bias     H*Pp*Pp fp16, log2 units (natural bias * log2(e)), zero padding
#include "pa_device.h"

namespace pa {

// --------------------------------------------------------------------------
// weight packing: transposed fp16 copies so that every MFMA operand lane
// reads 16 contiguous bytes.  bf16 -> fp16 is exact for magnitudes in
// [2^-14, 65504]; smaller weights keep an absolute error below 2^-25.
//   wT  [4*HD][C_IN]  rows: q cols, k cols, v cols, g cols
//   woT [C_OUT][HD]
// --------------------------------------------------------------------------
__global__ void pack_weights_kernel(const bf16* __restrict__ wq, const bf16* __restrict__ wk,
                                    const bf16* __restrict__ wv, const bf16* __restrict__ wg,
                                    const bf16* __restrict__ wo, f16* __restrict__ wT,
                                    f16* __restrict__ woT, int c_in, int hd, int c_out) {
  const int64_t n_w = (int64_t)4 * hd * c_in;
  const int64_t n_o = (int64_t)c_out * hd;
  const int64_t total = n_w + n_o;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n_w) {
      const int row = (int)(i / c_in), k = (int)(i % c_in);
      const int t = row / hd, col = row % hd;
      const bf16* src = t == 0 ? wq : t == 1 ? wk : t == 2 ? wv : wg;
      wT[i] = f2h_sat(bf2f(src[(int64_t)k * hd + col]));
    } else {
      const int64_t j = i - n_w;
      const int c = (int)(j / hd), k = (int)(j % hd);
      woT[j] = f2h_sat(bf2f(wo[(int64_t)k * c_out + c]));
    }
  }
}

// --------------------------------------------------------------------------
// LayerNorm of a tile of 32 positions of one row into LDS (fp16, row pitch
// C_IN + 8 elements).  Positions >= P are written as zeros.
// --------------------------------------------------------------------------
template <int C_IN, int NT>
__device__ __forceinline__ void ln_tile_to_lds(const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p,
                                               int r, int p0, int P, const bf16* __restrict__ gamma,
                                               const bf16* __restrict__ beta, float eps, f16* xs) {
  constexpr int TPP = C_IN / 8;           // threads per position (8 channels each)
  constexpr int PPP = NT / TPP;           // positions per pass
  static_assert(TPP <= 64 && (64 % TPP) == 0, "channel groups must tile a wave");
  const int tid = threadIdx.x;
  const int sub = tid % TPP;
#pragma unroll
  for (int base = 0; base < 32; base += PPP) {
    const int pl = base + tid / TPP;
    if (PPP <= 32 || pl < 32) {
      const int p = p0 + pl;
      float v[8];
      if (p < P) {
        const bf16x8 raw = ld16(x + (int64_t)r * xs_r + (int64_t)p * xs_p + sub * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf2f(raw[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[e];
      const float mean = group_sum<TPP>(s) * (1.0f / C_IN);
      float s2 = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = v[e] - mean;
        s2 += t * t;
      }
      const float var = group_sum<TPP>(s2) * (1.0f / C_IN);
      const float rstd = 1.0f / __builtin_sqrtf(var + eps);
      const bf16x8 gm = ld16(gamma + sub * 8);
      const bf16x8 bt = ld16(beta + sub * 8);
      f16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        y[e] = (p < P) ? f2h_sat((v[e] - mean) * rstd * bf2f(gm[e]) + bf2f(bt[e])) : f2h(0.0f);
      *reinterpret_cast<f16x8*>(xs + pl * (C_IN + 8) + sub * 8) = y;
    }
  }
}

// --------------------------------------------------------------------------
// Fused LayerNorm + projections.  One workgroup of 8 waves loops over tiles
// of 32 positions of one row; each wave keeps its 64 (or 96) weight columns
// in registers for the whole kernel.
//   MODE 0: q, k, v, g          MODE 1: q, k, v, g and the pair bias
//   MODE 2: pair bias only (wave 0 computes, the other waves only normalise)
// Column group blockIdx.y selects 512 of the 4*HD projection columns.
// --------------------------------------------------------------------------
template <int C_IN, int HD, int MODE>
__global__ __launch_bounds__(512) void proj_kernel(
    const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p, const bf16* __restrict__ gamma,
    const bf16* __restrict__ beta, float eps, const f16* __restrict__ wT, const bf16* __restrict__ wb,
    const bf16* __restrict__ b_g, float q_scale, f16* __restrict__ q_ws, f16* __restrict__ k_ws,
    f16* __restrict__ v_ws, f16* __restrict__ g_ws, float* __restrict__ bias, int bias_swizzled, float bias_scale,
    int nrows, int P, int Pp, int H) {
  constexpr int NT = 512;
  constexpr int KS = C_IN / 16;          // MFMA K-steps
  constexpr bool HAS_QKVG = MODE != 2;
  constexpr bool HAS_BIAS = MODE != 0;
  __shared__ __attribute__((aligned(16))) f16 xs[32 * (C_IN + 8)];

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int colbase = blockIdx.y * 512 + wave * 64;    // first of this wave's 64 columns
  const int tensor = colbase / HD;                     // 0 q, 1 k, 2 v, 3 g
  const bool bias_wave = HAS_BIAS && blockIdx.y == 0 && wave == 0;

  f16x8 W[2][KS];
  f16x8 WB[KS];
  if (HAS_QKVG) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int t = 0; t < KS; ++t) W[mb][t] = ld16(wT + (int64_t)(colbase + mb * 32 + lq) * C_IN + t * 16 + g * 8);
  }
  if (bias_wave) {   // w_b is [C_IN][H]; rows >= H of the operand are zero
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) WB[t][e] = lq < H ? f2h_sat(bf2f(wb[(int64_t)(t * 16 + g * 8 + e) * H + lq])) : f2h(0.0f);
  }

  const int tiles_per_row = Pp / 32;
  const int64_t ntiles = (int64_t)tiles_per_row * nrows;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int r = (int)(tile / tiles_per_row);
    const int p0 = (int)(tile % tiles_per_row) * 32;
    __syncthreads();   // previous tile's LDS reads are done
    ln_tile_to_lds<C_IN, NT>(x, xs_r, xs_p, r, p0, P, gamma, beta, eps, xs);
    __syncthreads();

    if (HAS_QKVG) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 acc = {};
        if (tensor == 2) {   // v: out = X W, rows = positions, columns = channels
#pragma unroll
          for (int t = 0; t < KS; ++t) acc = mfma32(ld16(xs + lq * (C_IN + 8) + t * 16 + g * 8), W[mb][t], acc);
        } else {             // q, k, g: out^T = W^T X^T, rows = channels, columns = positions
#pragma unroll
          for (int t = 0; t < KS; ++t) acc = mfma32(W[mb][t], ld16(xs + lq * (C_IN + 8) + t * 16 + g * 8), acc);
        }
        const int col = colbase + mb * 32 - tensor * HD;   // first column within the tensor
        const int h = col / 32;
        const int64_t rh = (int64_t)r * H + h;
        const int nb = Pp / 32;
        if (tensor == 0 || tensor == 1) {   // lane = position p0+lq; registers = 4 runs of 4 channels
          const float sc = tensor == 0 ? q_scale : 1.0f;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = f2h_sat(acc[jj * 4 + e] * sc);
            const int d0 = jj * 8 + g * 4;
            st8((tensor == 0 ? q_ws + q_off(rh, nb, p0 + lq, d0) : k_ws + k_off(rh, nb, p0 + lq, d0)), o);
          }
        } else if (tensor == 2) {           // lane = channel lq; registers = 4 runs of 4 positions
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = f2h_sat(acc[jj * 4 + e]);
            st8(v_ws + v_off(rh, nb, p0 + jj * 8 + g * 4, lq), o);
          }
        } else {
          const int p = p0 + lq;
          if (p < P) {
            f16* dst = g_ws + ((int64_t)r * P + p) * HD + col;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              f16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int d = jj * 8 + g * 4 + e;
                const float bg = b_g != nullptr ? bf2f(b_g[col + d]) : 0.0f;
                const float t = acc[jj * 4 + e] + bg;
                o[e] = f2h(1.0f / (1.0f + __expf(-t)));
              }
              st8(dst + jj * 8 + g * 4, o);
            }
          }
        }
      }
    }
    if (bias_wave) {
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KS; ++t) acc = mfma32(WB[t], ld16(xs + lq * (C_IN + 8) + t * 16 + g * 8), acc);
      const int p = p0 + lq;
      if (bias_swizzled) {   // attention layout: fp16, log2 units, padded to Pp x Pp with zeros
        const int nb = Pp / 32;
        f16* b16 = reinterpret_cast<f16*>(bias);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int hh = acc_row(j, g);
          if (hh < H) {
            b16[b16_off(hh, nb, r, p)] = p < P ? f2h_sat(acc[j] * bias_scale) : f2h(0.0f);
            if (r == P - 1)   // the padded query rows get zeros at the same keys
              for (int rp = P; rp < Pp; ++rp) b16[b16_off(hh, nb, rp, p)] = f2h(0.0f);
          }
        }
      } else if (p < P) {    // caller layout [H][P][P] float
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int hh = acc_row(j, g);
          if (hh < H) bias[((int64_t)hh * P + r) * P + p] = acc[j] * bias_scale;
        }
      }
    }
  }
}

// Copy of a caller-provided bias [H][P][P] (float, natural-log units) into
// the attention layout (fp16 operand order, log2 units, zero padding).
__global__ void bias_to_attn_layout_kernel(const float* __restrict__ src, f16* __restrict__ dst, int H, int P,
                                           int Pp) {
  const int64_t total = (int64_t)H * Pp * Pp;
  const int nb = Pp / 32;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(i / ((int64_t)Pp * Pp));
    const int64_t rem = i % ((int64_t)Pp * Pp);
    const int q = (int)(rem / Pp), k = (int)(rem % Pp);
    dst[b16_off(h, nb, q, k)] = (q < P && k < P) ? f2h_sat(src[((int64_t)h * P + q) * P + k] * kLog2e) : f2h(0.0f);
  }
}

}  // namespace pa

// ----------------------------------------------------------------------------
// launchers (called from the host API in pairattn_api.hip)
// ----------------------------------------------------------------------------
#include "pa_launch.h"

namespace pa {

hipError_t launch_bias_to_attn_layout(const float* src, void* dst, int H, int P, int Pp, hipStream_t s) {
  const int64_t total = (int64_t)H * Pp * Pp;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(bias_to_attn_layout_kernel, dim3(blocks), dim3(256), 0, s, src, (f16*)dst, H, P, Pp);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const PackArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)4 * a.hd * a.c_in + (int64_t)a.c_out * a.hd;
  const int threads = 256;
  const int blocks = (int)std::min<int64_t>((total + threads - 1) / threads, 4096);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(threads), 0, s, (const bf16*)a.wq, (const bf16*)a.wk,
                     (const bf16*)a.wv, (const bf16*)a.wg, (const bf16*)a.wo, (f16*)a.wT, (f16*)a.woT, a.c_in,
                     a.hd, a.c_out);
  return hipGetLastError();
}

template <int C_IN, int HD, int MODE>
static hipError_t proj_dispatch(const ProjArgs& a, int grid_x, int grid_y, hipStream_t s) {
  hipLaunchKernelGGL((proj_kernel<C_IN, HD, MODE>), dim3(grid_x, grid_y), dim3(512), 0, s, (const bf16*)a.x, a.xs_r,
                     a.xs_p, (const bf16*)a.gamma, (const bf16*)a.beta, a.eps, (const f16*)a.wT,
                     (const bf16*)a.wb, (const bf16*)a.b_g, a.q_scale, (f16*)a.q_ws, (f16*)a.k_ws,
                     (f16*)a.v_ws, (f16*)a.g_ws, a.bias, a.bias_swizzled, a.bias_scale, a.nrows, a.P, a.Pp, a.H);
  return hipGetLastError();
}

template <int C_IN, int MODE>
static hipError_t proj_dispatch_hd(const ProjArgs& a, int grid_x, int grid_y, hipStream_t s) {
  if (MODE == 2) return proj_dispatch<C_IN, 128, 2>(a, grid_x, 1, s);
  if (a.hd == 128) return proj_dispatch<C_IN, 128, MODE>(a, grid_x, grid_y, s);
  if (a.hd == 256) return proj_dispatch<C_IN, 256, MODE>(a, grid_x, grid_y, s);
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t proj_dispatch_c(const ProjArgs& a, int grid_x, int grid_y, hipStream_t s) {
  switch (a.c_in) {
    case 64: return proj_dispatch_hd<64, MODE>(a, grid_x, grid_y, s);
    case 128: return proj_dispatch_hd<128, MODE>(a, grid_x, grid_y, s);
    case 256: return proj_dispatch_hd<256, MODE>(a, grid_x, grid_y, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_proj_bf16(const ProjArgs& a, int mode, int num_cu, hipStream_t s) {
  const int64_t ntiles = (int64_t)(a.Pp / 32) * a.nrows;
  const int grid_y = mode == 2 ? 1 : (4 * a.hd) / 512;
  const int grid_x = (int)std::max<int64_t>(1, std::min<int64_t>(ntiles, (int64_t)num_cu * 2));
  switch (mode) {
    case 0: return proj_dispatch_c<0>(a, grid_x, grid_y, s);
    case 1: return proj_dispatch_c<1>(a, grid_x, grid_y, s);
    case 2: return proj_dispatch_c<2>(a, grid_x, grid_y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
