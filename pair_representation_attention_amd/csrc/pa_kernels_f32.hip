// fp32 kernels for gated pair-biased attention on gfx950.
//
// fp32 in, fp32 out, fp32-accurate, on the matrix cores.  Every product of
// the path (projections, logits, P.V, output projection) takes its operands
// as fp16 pairs: an fp32 value x is held as hi + lo, where hi is x rounded to
// fp16 and lo = x - hi (exact in fp32) rounded to fp16.  A product a.b is
// formed from the three fp16 products hi.hi + hi.lo + lo.hi, each a
// 32x32x16 f16 MFMA accumulating in fp32.  For |a|, |b| in [2^-14, 65504]
// what is dropped (lo.lo and the rounding of lo) is below 2^-21 of |a||b|,
// against 2^-24 for fp32 itself, at three fp16 MFMAs per product instead of
// the sixteen-fold cost of fp32 MFMAs.
// Operands must stay below 65504 in magnitude; below 2^-14 they keep an
// absolute error under 2^-24.  The softmax, LayerNorm, sigmoid, bias and all
// accumulation run in fp32.
//
// Row-attention formulation as in the bf16 path: nrows rows of P positions
// (queries = keys), H heads of width 32, bias[h][query][key] shared by all
// rows.  Workspace (Pp = P rounded up to 32, nb = Pp / 32, rh = row*H + h;
// padded positions hold zeros):
//   q, k, v  hi and lo planes, nrows*H*Pp*32 fp16 each, in the operand-ordered
//            layouts of pa_device.h (q scaled by log2(e)/sqrt(d))
//   g        nrows*H*Pp*32 float, sigmoid applied, one 4 KB tile per (rh,
//            query block) holding the O^T accumulator image: lane = query %
//            32 + 32*half, register j = channel acc_row(j, half)
//   bias     H*Pp*Pp float in log2 units, one 4 KB tile per (h, query block,
//            key block) holding the S^T accumulator image (lane = query % 32
//            + 32*half, register j = key acc_row(j, half)); keys >= P hold
//            -inf, so padded keys get weight 0 without a mask
//   packed weights: gamma-folded q|k|v|g (+ pair bias) operands, hi and lo
//            planes, [block of 32 columns][K-step][64 lanes][8]; W_o as the
//            B operand of out = og.W_o, [c block][head][chunk][64 lanes][8]
#include "pa_device.h"
#include "pa_launch.h"

#include <type_traits>

namespace pa {

// ---------------------------------------------------------------------------
// fp16 pairs
// ---------------------------------------------------------------------------
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// x - h exactly, h the low (or high) fp16 half of a packed register: one
// mixed-precision FMA (h * -1 + x) instead of a convert and a subtract
__device__ __forceinline__ float minus_lo_half(f16x2 h, float x) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}
__device__ __forceinline__ float minus_hi_half(f16x2 h, float x) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x));
  return r;
}
// hi = fp16(x) (round to nearest even), lo = fp16(x - hi): two VALU
// operations per value (a packed convert per pair for each plane, one FMA)
__device__ __forceinline__ void split8(const float* x, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f16x2 h = {(f16)x[e], (f16)x[e + 1]};
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = (f16)minus_lo_half(h, x[e]);
    lo[e + 1] = (f16)minus_hi_half(h, x[e + 1]);
  }
}
// D = A.B + C with A = ah + al, B = bh + bl (the small terms first)
__device__ __forceinline__ f32x16 mfma3(const f16x8& ah, const f16x8& al, const f16x8& bh, const f16x8& bl,
                                        f32x16 c) {
  c = mfma32(al, bh, c);
  c = mfma32(ah, bl, c);
  return mfma32(ah, bh, c);
}

// ---------------------------------------------------------------------------
// Weight packing.  LayerNorm's affine map is folded into the projection:
//   ((x-mu)*rstd*gamma + beta) . W = ((x-mu)*rstd) . (gamma o W) + beta . W
// Block b of the packed list is columns b*32..+31 of q|k|v|g (each H*32
// wide).  Lane l of K-step t holds column l%32 and channels t*16 + (l/32)*8
// .. +7 (the activation operand uses the same slots).
// cst[n] = beta . W[:, n] (+ b_g for gate columns): one wave per column,
// fp32 partial sums over the lanes, then a wave reduction (blockIdx.y = 1;
// blockIdx.y = 0 packs the operands).
// W_o is packed as the B operand of out = og . W_o: lane l of (c block cb,
// head hh, chunk t) holds output column cb*32 + l%32 and, in element e, the
// head channel slot_x(t, l/32, e), the order in which an O^T accumulator
// holds its rows.
// ---------------------------------------------------------------------------
__global__ void pack_f32_kernel(const float* __restrict__ wq, const float* __restrict__ wk,
                                const float* __restrict__ wv, const float* __restrict__ wg,
                                const float* __restrict__ gamma, const float* __restrict__ beta,
                                const float* __restrict__ b_g, int c_in, int hd, int H, int nqkvg,
                                f16* __restrict__ w_hi, f16* __restrict__ w_lo,
                                float* __restrict__ cst, const float* __restrict__ wo, f16* __restrict__ wo_hi,
                                f16* __restrict__ wo_lo, int c_out) {
  if (blockIdx.y == 1) {
    const int n = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (n >= nqkvg * 32) return;   // the whole wave
    const int tsr = n / hd, cc = n % hd;
    const float* src = tsr == 0 ? wq : tsr == 1 ? wk : tsr == 2 ? wv : wg;
    float acc = 0.0f;
    for (int k = lane; k < c_in; k += kWave) acc = __builtin_fmaf(beta[k], src[(int64_t)k * hd + cc], acc);
    acc = group_sum<kWave>(acc);
    if (lane == 0) cst[n] = acc + (tsr == 3 && b_g != nullptr ? b_g[cc] : 0.0f);
    return;
  }
  const int ks = c_in / 16;
  const int64_t n_w = (int64_t)nqkvg * ks * 64;    // 8-element slots of the projection operands
  const int64_t n_o = wo != nullptr ? (int64_t)(c_out / 32) * H * 2 * 64 : 0;
  const int64_t total = n_w + n_o;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n_w) {
      const int l = (int)(i & 63), t = (int)((i >> 6) % ks), b = (int)((i >> 6) / ks);
      const int k0 = t * 16 + (l >> 5) * 8;
      const int col = b * 32 + (l & 31);
      const int tsr = col / hd, cc = col % hd;
      const float* src = tsr == 0 ? wq : tsr == 1 ? wk : tsr == 2 ? wv : wg;
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = src[(int64_t)(k0 + e) * hd + cc] * gamma[k0 + e];
      f16x8 hi, lo;
      split8(w, hi, lo);
      *reinterpret_cast<f16x8*>(w_hi + i * 8) = hi;
      *reinterpret_cast<f16x8*>(w_lo + i * 8) = lo;
    } else {
      const int64_t j = i - n_w;
      const int l = (int)(j & 63), t = (int)((j >> 6) & 1), hh = (int)((j >> 7) % H), cb = (int)((j >> 7) / H);
      const int col = cb * 32 + (l & 31);
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = wo[(int64_t)(hh * 32 + slot_x(t, l >> 5, e)) * c_out + col];
      f16x8 hi, lo;
      split8(w, hi, lo);
      *reinterpret_cast<f16x8*>(wo_hi + j * 8) = hi;
      *reinterpret_cast<f16x8*>(wo_lo + j * 8) = lo;
    }
  }
}

// offset (floats) of bias element (h, query, key) in the tiled S^T image
__device__ __forceinline__ int64_t bias_c_off(int h, int nb, int q, int k) {
  const int x = k & 31;
  const int lane = (q & 31) + 32 * slot_hg(x);
  const int j = (x >> 3) * 4 + (x & 3);
  return ((((int64_t)h * nb + (q >> 5)) * nb + (k >> 5)) * 64 + lane) * 16 + j;
}

// ---------------------------------------------------------------------------
// Fused LayerNorm + projections.  Each wave works on its own tiles of 32
// positions of one row; a lane holds one position (lane % 32) and, in K-step
// t, channels t*16 + half*8 .. +7, which is the register image of both MFMA
// operand kinds.  LayerNorm runs in registers; the normalised activations
// are split into fp16 pairs.  The launch computes the q|k|v|g blocks
// [b_first, b_first + nqkvg) of the packed list (q only, k and v only, ...).
// The workgroup's NB column blocks sit in LDS
// (hi and lo planes): packed q|k|v|g blocks are copied, the pair-bias block
// (rows = heads, zero beyond H; the last block when with_bias) is built here
// from w_b and gamma, with its constants beta . w_b.  Block kinds: q and k (out^T = W^T X^T, rows =
// channels, lane = position) are written as operand chunks; v (X W, rows =
// positions, lane = channel) likewise in its own order; the gate as its
// fp32 O^T image; the pair bias (rows = heads) into the tiled S^T image
// (log2 units) or, with bias_natural, as [H][P][P] float.
// ---------------------------------------------------------------------------
template <int C_IN>
struct ProjF32Shape {
  static constexpr int KS = C_IN / 16;
  // 8 waves and 128 KB of operands (fewer column groups, so fewer passes
  // over x) where the registers allow two waves per SIMD; 4 waves and 64 KB
  // for 256 input channels
  static constexpr int THREADS = C_IN <= 128 ? 512 : 256;
  static constexpr int NB = (C_IN <= 128 ? 64 : 32) / KS;   // column blocks per workgroup
  static constexpr int LDS = NB * KS * 2 * 1024;
};

template <int C_IN>
__global__ __launch_bounds__(ProjF32Shape<C_IN>::THREADS) void proj_f32_kernel(
    const float* __restrict__ x, int64_t xs_r, int64_t xs_p, int tile_rmajor, float eps, const f16* __restrict__ w_hi,
    const f16* __restrict__ w_lo, const float* __restrict__ cst, int b_first, int nqkvg, int with_bias,
    const float* __restrict__ wb, const float* __restrict__ gamma, const float* __restrict__ beta, int hd,
    float q_scale,
    f16* __restrict__ q_hi, f16* __restrict__ q_lo, f16* __restrict__ k_hi, f16* __restrict__ k_lo,
    f16* __restrict__ v_hi, f16* __restrict__ v_lo, float* __restrict__ g_ws, float* __restrict__ bias,
    int bias_natural, float bias_scale, int nrows, int P, int Pp, int H) {
  using SH = ProjF32Shape<C_IN>;
  constexpr int KS = SH::KS;
  constexpr int NW = SH::THREADS / kWave;
  __shared__ __attribute__((aligned(1024))) char smem[SH::LDS];
  __shared__ float cstb[8];
  f16* wl_hi = reinterpret_cast<f16*>(smem);
  f16* wl_lo = wl_hi + SH::NB * KS * 512;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int lq = lane & 31, g = lane >> 5;
  const int nblk = nqkvg + with_bias;
  const int b0 = blockIdx.y * SH::NB;
  const int nbl = min(SH::NB, nblk - b0);   // blocks of this workgroup

  for (int i = tid; i < nbl * KS * 64; i += SH::THREADS) {
    const int b = b0 + i / (KS * 64);
    if (b < nqkvg) {
      const int64_t src = (int64_t)(b_first + b0) * KS * 64 + i;
      *reinterpret_cast<f16x8*>(wl_hi + i * 8) = *reinterpret_cast<const f16x8*>(w_hi + src * 8);
      *reinterpret_cast<f16x8*>(wl_lo + i * 8) = *reinterpret_cast<const f16x8*>(w_lo + src * 8);
    } else {
      const int l = i & 63, t = (i >> 6) % KS, hh = l & 31;
      const int k0 = t * 16 + (l >> 5) * 8;
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = hh < H ? wb[(int64_t)(k0 + e) * H + hh] * gamma[k0 + e] : 0.0f;
      f16x8 hi, lo;
      split8(w, hi, lo);
      *reinterpret_cast<f16x8*>(wl_hi + i * 8) = hi;
      *reinterpret_cast<f16x8*>(wl_lo + i * 8) = lo;
    }
  }
  if (with_bias) {   // beta . w_b per head: a wave per head, partial sums over the lanes
    for (int hh = wave; hh < 8; hh += NW) {
      float acc = 0.0f;
      if (hh < H)
        for (int k = lane; k < C_IN; k += kWave) acc = __builtin_fmaf(beta[k], wb[(int64_t)k * H + hh], acc);
      acc = group_sum<kWave>(acc);
      if (lane == 0) cstb[hh] = acc;
    }
  }
  __syncthreads();

  const int nb = Pp / 32;
  const int64_t ntiles = (int64_t)nb * nrows;
  const int64_t stride = (int64_t)gridDim.x * NW;
  auto tile_rp = [&](int64_t tile, int& r, int& p0) {
    if (tile_rmajor) {
      r = (int)(tile / nb);
      p0 = (int)(tile % nb) * 32;
    } else {
      r = (int)(tile % nrows);
      p0 = (int)(tile / nrows) * 32;
    }
  };
  // this lane's raw channels of a tile (zeros past P or past the last tile)
  // element offset of this lane's position and channel half within a tile
  // (the tile's own offset is wave-uniform and computed on the scalar unit)
  const int64_t lane_off = (int64_t)lq * xs_p + g * 8;
  auto load_raw = [&](int64_t tile, float (*raw)[8]) {
    if (tile < ntiles) {
      int r, p0;
      tile_rp(tile, r, p0);
      const int p = p0 + lq;
      if (p < P) {
        const float* src = x + ((int64_t)r * xs_r + (int64_t)p0 * xs_p) + lane_off;
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(src + t * 16);
          const f32x4 b = *reinterpret_cast<const f32x4*>(src + t * 16 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            raw[t][e] = a[e];
            raw[t][4 + e] = b[e];
          }
        }
        return;
      }
    }
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[t][e] = 0.0f;
  };
  // the next tile's rows are loaded before this one is computed where the
  // registers allow it (64 input channels)
  constexpr bool PF = C_IN <= 64;
  float nxt[KS][8];
  int64_t tile = (int64_t)blockIdx.x * NW + wave;
  if (PF) load_raw(tile, nxt);
  for (; tile < ntiles; tile += stride) {
    int r, p0;
    tile_rp(tile, r, p0);
    const int p = p0 + lq;
    const bool valid = p < P;

    // ---- LayerNorm (two passes, fp32) and fp16 pairs ----
    float raw[KS][8];
    if (PF) {
#pragma unroll
      for (int t = 0; t < KS; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[t][e] = nxt[t][e];
      load_raw(tile + stride, nxt);
    } else {
      load_raw(tile, raw);
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += raw[t][e];
    s += __shfl_xor(s, 32, 64);
    const float mean = s * (1.0f / C_IN);
    float s2 = 0.0f;
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = raw[t][e] - mean;
        s2 = __builtin_fmaf(d, d, s2);
      }
    s2 += __shfl_xor(s2, 32, 64);
    const float rstd = 1.0f / __builtin_sqrtf(s2 * (1.0f / C_IN) + eps);
    f16x8 Xh[KS], Xl[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      float xn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xn[e] = valid ? (raw[t][e] - mean) * rstd : 0.0f;
      split8(xn, Xh[t], Xl[t]);
    }

    for (int bl = 0; bl < nbl; ++bl) {
      const int b = b0 + bl;
      const f16* oph = wl_hi + bl * KS * 512 + lane * 8;
      const f16* opl = wl_lo + bl * KS * 512 + lane * 8;
      f32x16 acc = {};
      if (b < nqkvg) {
        const int col = (b_first + b) * 32;
        const int tsr = col / hd;                 // 0 q, 1 k, 2 v, 3 g
        const int64_t rh = (int64_t)r * H + (col - tsr * hd) / 32;
        const int64_t chunk0 = (rh * nb + (p0 >> 5)) * 2;
        const float* cb = cst + col;
        if (tsr == 2) {                           // v = X W: rows = positions, lane = channel
#pragma unroll
          for (int t = 0; t < KS; ++t)
            acc = mfma3(Xh[t], Xl[t], *reinterpret_cast<const f16x8*>(oph + t * 512),
                        *reinterpret_cast<const f16x8*>(opl + t * 512), acc);
          const float c = cb[lq];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = p0 + slot_x(t, g, e) < P ? acc[8 * t + e] + c : 0.0f;
            f16x8 hi, lo;
            split8(o, hi, lo);
            st16(v_hi + (chunk0 + t) * 512 + lane * 8, hi);
            st16(v_lo + (chunk0 + t) * 512 + lane * 8, lo);
          }
        } else {                                  // out^T = W^T X^T: rows = channels, lane = position
#pragma unroll
          for (int t = 0; t < KS; ++t)
            acc = mfma3(*reinterpret_cast<const f16x8*>(oph + t * 512),
                        *reinterpret_cast<const f16x8*>(opl + t * 512), Xh[t], Xl[t], acc);
          if (tsr <= 1) {
            const float sc = valid ? (tsr == 0 ? q_scale : 1.0f) : 0.0f;
            f16* dh = tsr == 0 ? q_hi : k_hi;
            f16* dl = tsr == 0 ? q_lo : k_lo;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              float o[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] = (acc[8 * t + e] + cb[slot_x(t, g, e)]) * sc;
              f16x8 hi, lo;
              split8(o, hi, lo);
              st16(dh + (chunk0 + t) * 512 + lane * 8, hi);
              st16(dl + (chunk0 + t) * 512 + lane * 8, lo);
            }
          } else {                                // gate: sigmoid, O^T image in fp32
            f32x16 o;
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = sigmoid_fast(acc[j] + cb[acc_row(j, g)]);
            float* dst = g_ws + ((rh * nb + (p0 >> 5)) * 64 + lane) * 16;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<f32x4*>(dst + 4 * q4) = f32x4{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]};
          }
        }
      } else {                                    // pair bias: rows = heads, lane = position (key)
#pragma unroll
        for (int t = 0; t < KS; ++t)
          acc = mfma3(*reinterpret_cast<const f16x8*>(oph + t * 512),
                      *reinterpret_cast<const f16x8*>(opl + t * 512), Xh[t], Xl[t], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) {            // heads (< 8) are rows g*4 + j of registers 0..3
          const int hh = acc_row(j, g);
          if (hh >= H) continue;
          const float val = (acc[j] + cstb[hh]) * bias_scale;
          if (bias_natural) {
            if (valid) bias[((int64_t)hh * P + r) * P + p] = val;
          } else {
            bias[bias_c_off(hh, nb, r, p)] = valid ? val : -__builtin_inff();
            if (r == P - 1)   // padded query rows: finite at real keys, -inf at padded ones
              for (int rp = P; rp < Pp; ++rp) bias[bias_c_off(hh, nb, rp, p)] = valid ? 0.0f : -__builtin_inff();
          }
        }
      }
    }
  }
}

// Caller-provided bias [H][Pq][Pk] float (natural-log units) -> tiled S^T
// image ([h][query block][key block] tiles) in log2 units, -inf at padded
// keys, 0 at padded queries.
__global__ void bias_to_f32_layout_kernel(const float* __restrict__ src, float* __restrict__ dst, int H, int Pq,
                                          int Pk, int Ppq, int Ppk) {
  const int64_t total = (int64_t)H * Ppq * Ppk;
  const int nbk = Ppk / 32;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int h = (int)(i / ((int64_t)Ppq * Ppk));
    const int64_t rem = i % ((int64_t)Ppq * Ppk);
    const int q = (int)(rem / Ppk), k = (int)(rem % Ppk);
    float v = -__builtin_inff();
    if (k < Pk) v = q < Pq ? src[((int64_t)h * Pq + q) * Pk + k] * kLog2e : 0.0f;
    const int x = k & 31;
    const int ln = (q & 31) + 32 * slot_hg(x);
    const int j = (x >> 3) * 4 + (x & 3);
    dst[((((int64_t)h * (Ppq / 32) + (q >> 5)) * nbk + (k >> 5)) * 64 + ln) * 16 + j] = v;
  }
}

// ---------------------------------------------------------------------------
// Attention.  A workgroup is H waves (wave = head) over one row and two query
// blocks (64 queries); a unit is 32 queries x 32 keys of one head.  Per unit:
//   S^T = K.Q^T + C      six MFMAs (two K-steps of three), C = bias tile
//   online softmax per query (lane): running maximum m raised only when a
//   block's maximum passes it by more than 8 (log2 units), so p = exp2(s - m)
//   <= 256; l accumulates p in fp32
//   O^T += V^T.P^T       six MFMAs, P split into fp16 pairs
// The units are software-pipelined: each unit's softmax VALU runs with the
// next unit's logit MFMAs and its own P.V MFMAs issued in between.
// Epilogue: o = O/l times the gate, as fp16 pairs into LDS; then the waves
// share the output tiles (query block x 32 columns), each a K = H*32
// contraction of og with W_o, + b_o, fp32 stores.
// ---------------------------------------------------------------------------
template <int H>
__device__ __forceinline__ void gate_project_store(f16* og_lds, const f32x16 (&O)[2], const float (&inv)[2],
                                                   const f32x16& G0, const f32x16& G1, int h, int wave, int lane,
                                                   const f16* __restrict__ wo_hi, const f16* __restrict__ wo_lo,
                                                   const float* __restrict__ b_o, float* __restrict__ out,
                                                   int64_t os_r, int64_t os_p, int c_out, int r, int P, int qb0,
                                                   int qb1);

template <int H, bool HAS_MASK, int MODE>
__global__ __launch_bounds__(H * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_f32_kernel(
    const f16* __restrict__ q_hi, const f16* __restrict__ q_lo, const f16* __restrict__ k_hi,
    const f16* __restrict__ k_lo, const f16* __restrict__ v_hi, const f16* __restrict__ v_lo,
    const float* __restrict__ g_ws, const float* __restrict__ bias, const uint32_t* __restrict__ mask_bits,
    const f16* __restrict__ wo_hi, const f16* __restrict__ wo_lo, const float* __restrict__ b_o,
    float* __restrict__ out, int64_t os_r, int64_t os_p, int c_out, int nrows, int P, int nbq, int nbk, int ngroups,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  // og tiles: [query block u][head][chunk t][plane][64 lanes][8] fp16
  __shared__ __attribute__((aligned(1024))) f16 og_lds[2 * H * 2 * 2 * 512];

  // the wave index (= head) as a scalar, so that every load is a uniform
  // base plus a 32-bit lane offset
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane >> 5;
  const int h = wave;
  // lane's 16-byte slot of a 1 KB operand chunk
  auto ld_chunk = [&](const f16* base) { return reinterpret_cast<const f16x8*>(base)[lane]; };

  // XCD-aware order: consecutive ids go round-robin over the 8 XCDs; give
  // each XCD a contiguous range of tiles so that the query groups of a row
  // (which share K and V) meet in one L2
  const int64_t ntile = (int64_t)ngroups * nrows;
  int64_t tile = blockIdx.x;
  if ((ntile & 7) == 0) tile = (tile & 7) * (ntile >> 3) + (tile >> 3);
  const int r = (int)(tile / ngroups);
  const int grp = (int)(tile % ngroups);
  const int qb0 = 2 * grp, qb1 = min(2 * grp + 1, nbq - 1);   // an odd last group repeats its block
  const int64_t rh = (int64_t)r * H + h;

  f16x8 Qh[2][2], Ql[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    Qh[0][t] = ld_chunk(q_hi + qkv_chunk(rh, nbq, qb0, t));
    Ql[0][t] = ld_chunk(q_lo + qkv_chunk(rh, nbq, qb0, t));
    Qh[1][t] = ld_chunk(q_hi + qkv_chunk(rh, nbq, qb1, t));
    Ql[1][t] = ld_chunk(q_lo + qkv_chunk(rh, nbq, qb1, t));
  }

  struct KV {
    f16x8 kh[2], kl[2], vh[2], vl[2];
  };
  auto load_k = [&](KV& d, int kb) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t o = qkv_chunk(rh, nbk, kb, t);
      d.kh[t] = ld_chunk(k_hi + o);
      d.kl[t] = ld_chunk(k_lo + o);
    }
  };
  auto load_v = [&](KV& d, int kb) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t o = qkv_chunk(rh, nbk, kb, t);
      d.vh[t] = ld_chunk(v_hi + o);
      d.vl[t] = ld_chunk(v_lo + o);
    }
  };
  // a lane's 16 floats of a 4 KB accumulator-image tile
  auto load_bias_like = [&](f32x16& d, const float* tile) {
    const f32x4* src = reinterpret_cast<const f32x4*>(tile) + lane * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = src[q4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * q4 + e] = v[e];
    }
  };
  auto load_bias = [&](f32x16& d, int qb, int kb) {
    load_bias_like(d, bias + (((int64_t)h * nbq + qb) * nbk + kb) * 1024);
  };

  f32x16 O[2] = {};
  float m[2] = {-__builtin_inff(), -__builtin_inff()};
  float l[2] = {0.0f, 0.0f};
  // logits of the units of query block 0 in SA, of query block 1 in SB; the
  // bias tiles prefetched for them in CA and CB
  f32x16 SA, SB, CA, CB;
  const uint32_t* brow = HAS_MASK ? mask_bits + (int64_t)r * nbk : nullptr;
  uint32_t bits_cur = 0, bits_nxt = 0;

  // Unit u (key block kb, query block J) as one instruction stream: the
  // softmax of u on the VALU, with the six logit MFMAs of unit u+1 (bias of
  // u+1 in its C buffer, K of u+1's key block in `kn`) and the six P.V MFMAs
  // of u issued between its groups, so that the matrix cores run while the
  // softmax does.  Loads: K (J = 0) or V (J = 1) of block kb+1 first, one
  // stream before their first use, into registers whose last reader has
  // been issued (at most three of the four K/V tiles of two blocks are
  // live); the bias tile of unit u+3 at the end, into the C buffer that u+1
  // has just consumed.  FAST: shift 0 for every weight (no running
  // maximum), the sweep that the check below accepts or reruns.
  auto stream = [&](auto jc, auto nextc, auto fastc, int kb, KV& cur, KV& oth) {
    constexpr int J = decltype(jc)::value;
    constexpr int JN = 1 - J;
    constexpr bool NEXT = decltype(nextc)::value;
    constexpr bool FAST = decltype(fastc)::value;
    f32x16& Sc = J ? SB : SA;
    f32x16& Sn = J ? SA : SB;
    f32x16& Cn = J ? CA : CB;
    const KV& kn = J ? oth : cur;
    // every path issues the same loads (past the last block they repeat it,
    // into registers nobody reads), so the compiler's counted waits are exact
    const int kb1 = min(kb + 1, nbk - 1);
    if constexpr (J == 0) {
      load_k(oth, kb1);
    } else {
      load_v(oth, kb1);
      if (HAS_MASK) bits_nxt = brow[kb1];
    }
    // ---- running maximum and rescale (uniform branch, rarely taken) ----
    if constexpr (HAS_MASK) {
      // register j holds key (j/4)*8 + 4*half + j%4
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int k0 = (j >> 2) * 8 + (j & 3);
        const uint64_t lanes = (((bits_cur >> k0) & 1u) ? 0x00000000ffffffffull : 0ull) |
                               (((bits_cur >> (k0 + 4)) & 1u) ? 0xffffffff00000000ull : 0ull);
        Sc[j] = __builtin_amdgcn_inverse_ballot_w64(lanes) ? Sc[j] : -__builtin_inff();
      }
    }
    if constexpr (!FAST) {
      float bm = Sc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) bm = __builtin_fmaxf(bm, Sc[j]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
        bm = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mn = bm > m[J] + 8.0f ? bm : m[J];
      if (__builtin_amdgcn_ballot_w64(mn != m[J]) != 0) {
        const float alpha = fast_exp2(m[J] - mn);   // 0 while m is -inf
#pragma unroll
        for (int j = 0; j < 16; ++j) O[J][j] *= alpha;
        l[J] *= alpha;
        m[J] = mn;
      }
    }
    const float ms = FAST || m[J] == -__builtin_inff() ? 0.0f : m[J];
    __builtin_amdgcn_sched_barrier(0);
    // ---- softmax weights and fp16 pairs, with the MFMAs in between ----
    float p[16];
    f16x8 ph0, pl0, ph1, pl1;
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(Sc[j] - ms);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kl[0], Qh[JN][0], Cn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 4; j < 8; ++j) p[j] = fast_exp2(Sc[j] - ms);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kh[0], Ql[JN][0], Sn);
    __builtin_amdgcn_sched_barrier(0);
    split8(p, ph0, pl0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kh[0], Qh[JN][0], Sn);
    __builtin_amdgcn_sched_barrier(0);
    {
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ls += p[j];
      l[J] += ls;
    }
#pragma unroll
    for (int j = 8; j < 10; ++j) p[j] = fast_exp2(Sc[j] - ms);
    __builtin_amdgcn_sched_barrier(0);
    O[J] = mfma32(cur.vl[0], ph0, O[J]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 10; j < 13; ++j) p[j] = fast_exp2(Sc[j] - ms);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kl[1], Qh[JN][1], Sn);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 13; j < 16; ++j) p[j] = fast_exp2(Sc[j] - ms);
    __builtin_amdgcn_sched_barrier(0);
    O[J] = mfma32(cur.vh[0], pl0, O[J]);
    __builtin_amdgcn_sched_barrier(0);
    split8(p + 8, ph1, pl1);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kh[1], Ql[JN][1], Sn);
    __builtin_amdgcn_sched_barrier(0);
    {
      float ls = 0.0f;
#pragma unroll
      for (int j = 8; j < 16; ++j) ls += p[j];
      l[J] += ls;
    }
    __builtin_amdgcn_sched_barrier(0);
    O[J] = mfma32(cur.vh[0], ph0, O[J]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) Sn = mfma32(kn.kh[1], Qh[JN][1], Sn);
    __builtin_amdgcn_sched_barrier(0);
    O[J] = mfma32(cur.vl[1], ph1, O[J]);
    O[J] = mfma32(cur.vh[1], pl1, O[J]);
    O[J] = mfma32(cur.vh[1], ph1, O[J]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) load_bias(Cn, JN ? qb1 : qb0, min(kb + (J + 3) / 2, nbk - 1));   // unit u+3
    if constexpr (J == 1 && HAS_MASK) bits_cur = bits_nxt;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using BT = std::true_type;
  using BF = std::false_type;
  KV X, Y;   // key blocks of even / odd index
  // the gate tiles (read once, from HBM) are loaded two streams before the
  // sweep ends, so their latency hides under the last key block
  f32x16 G0, G1;
  auto load_gate = [&]() {
    if constexpr (MODE == 0) {
      load_bias_like(G0, g_ws + (rh * nbq + qb0) * 1024);
      load_bias_like(G1, g_ws + (rh * nbq + qb1) * 1024);
    }
  };
  auto sweep = [&](auto fastc) {
    // prologue: K, V of block 0, the first bias tiles, the logits of unit 0
    load_k(X, 0);
    load_v(X, 0);
    load_bias(CA, qb0, 0);
    load_bias(CB, qb1, 0);
    if (HAS_MASK) bits_cur = brow[0];
    SA = mfma3(X.kh[0], X.kl[0], Qh[0][0], Ql[0][0], CA);
    SA = mfma3(X.kh[1], X.kl[1], Qh[0][1], Ql[0][1], SA);
    load_bias(CA, qb0, min(1, nbk - 1));
    int kb = 0;
    for (; kb + 2 < nbk; kb += 2) {
      stream(I0{}, BT{}, fastc, kb, X, Y);
      stream(I1{}, BT{}, fastc, kb, X, Y);
      stream(I0{}, BT{}, fastc, kb + 1, Y, X);
      stream(I1{}, BT{}, fastc, kb + 1, Y, X);
    }
    if (nbk - kb == 2) {
      stream(I0{}, BT{}, fastc, kb, X, Y);
      stream(I1{}, BT{}, fastc, kb, X, Y);
      load_gate();
      stream(I0{}, BT{}, fastc, kb + 1, Y, X);
      stream(I1{}, BF{}, fastc, kb + 1, Y, X);
    } else {
      load_gate();
      stream(I0{}, BT{}, fastc, kb, X, Y);
      stream(I1{}, BF{}, fastc, kb, X, Y);
    }
  };

  // Shift 0 first.  Its weights 2^s are exact as fp16 pairs (relative 2^-22)
  // down to 2^-14 and within 2^-25 absolute below, the same bound as with
  // the running maximum, as long as no weight passes 65504 (then l, their
  // fp32 sum, does) and l >= 1 for every query of a row with a kept key.
  // Where a query of this wave fails, the wave sweeps again with the running
  // maximum (waves share nothing before the epilogue).
  sweep(BT{});
  {
    bool bad = false, zero = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[u]), __float_as_uint(l[u]), false, false);
      const float lq = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int q = (u == 0 ? qb0 : qb1) * 32 + (lane & 31);
      if (q < P) {
        bad = bad || !(lq < 65504.0f) || (lq > 0.0f && lq < 1.0f);
        zero = zero || lq == 0.0f;
      }
    }
    bool rerun = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (!rerun && __builtin_amdgcn_ballot_w64(zero) != 0) {
      // l = 0 is exact only for a row with no kept key
      if constexpr (HAS_MASK) {
        uint32_t kept = 0;
        for (int b = 0; b < nbk; ++b) kept |= brow[b];
        rerun = kept != 0;
      } else {
        rerun = true;
      }
    }
    if (rerun) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        O[u] = f32x16{};
        m[u] = -__builtin_inff();
        l[u] = 0.0f;
      }
      sweep(BF{});
    }
  }

  // ---- epilogue ----
  float lt[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[u]), __float_as_uint(l[u]), false, false);
    lt[u] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // the query's l over both lane halves
  }
  if constexpr (MODE == 0) {
    const float inv[2] = {lt[0] > 0.0f ? 1.0f / lt[0] : 0.0f, lt[1] > 0.0f ? 1.0f / lt[1] : 0.0f};
    gate_project_store<H>(og_lds, O, inv, G0, G1, h, wave, lane, wo_hi, wo_lo, b_o, out, os_r, os_p, c_out, r, P,
                          qb0, qb1);
  } else {
    // one key shard: o = O/l per head ([row][query][h*32 + channel]) and
    // lse = ln(l) + m ln 2 per (row, head, query); MODE 2 merges them into
    // the values already there (log-sum-exp weights, fp32)
    constexpr float kLn2 = 0.6931471805599453f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && qb1 == qb0) continue;   // repeated block of an odd last group
      const int q = (u == 0 ? qb0 : qb1) * 32 + (lane & 31);
      if (q >= P) continue;
      const bool any = lt[u] > 0.0f;
      const float ms = m[u] == -__builtin_inff() ? 0.0f : m[u];
      const float lse_new = any ? (ms + __builtin_log2f(lt[u])) * kLn2 : -__builtin_inff();
      const float inv = any ? 1.0f / lt[u] : 0.0f;
      float wn = 1.0f, wo = 0.0f, lse = lse_new;
      float* lse_at = lse_part + ((int64_t)r * H + h) * P + q;
      if constexpr (MODE == 2) {
        const float lse_old = *lse_at;
        const float mx = __builtin_fmaxf(lse_old, lse_new);
        if (mx == -__builtin_inff()) {
          wn = 0.0f;   // no kept key in either part: o stays 0, lse -inf
        } else {
          wo = expf(lse_old - mx);
          wn = expf(lse_new - mx);
          const float den = wo + wn;
          lse = mx + logf(den);
          wo /= den;
          wn /= den;
        }
      }
      // registers 4i..4i+3 hold channels 8i + 4*half + 0..3
      float* orow = o_part + ((int64_t)r * P + q) * (H * 32) + h * 32 + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4* dst = reinterpret_cast<f32x4*>(orow + 8 * i);
        f32x4 v = {O[u][4 * i] * inv * wn, O[u][4 * i + 1] * inv * wn, O[u][4 * i + 2] * inv * wn,
                   O[u][4 * i + 3] * inv * wn};
        if constexpr (MODE == 2) {
          const f32x4 old = *dst;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += old[e] * wo;
        }
        *dst = v;
      }
      if (g == 0) *lse_at = lse;
    }
  }
}

// Gate, output projection and store of one workgroup's two query blocks:
// og = o * inv * G (o the O^T accumulator image of each head's wave, G the
// gate tile) as fp16 pairs into LDS, one barrier, then the output tiles
// (query block u, 32 columns cb) shared by the waves, each a K = H*32
// contraction of og with W_o.  The tiles (+ b_o) are staged over og in LDS
// and leave one query block at a time as whole query rows, 16 bytes per lane
// (a row's c_out channels are contiguous at the caller's strides).
template <int H>
__device__ __forceinline__ void gate_project_store(f16* og_lds, const f32x16 (&O)[2], const float (&inv)[2],
                                                   const f32x16& G0, const f32x16& G1, int h, int wave, int lane,
                                                   const f16* __restrict__ wo_hi, const f16* __restrict__ wo_lo,
                                                   const float* __restrict__ b_o, float* __restrict__ out,
                                                   int64_t os_r, int64_t os_p, int c_out, int r, int P, int qb0,
                                                   int qb1) {
  const int g = lane >> 5;
  const int ncb = c_out / 32;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const f32x16& G = u == 0 ? G0 : G1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = O[u][8 * t + e] * inv[u] * G[8 * t + e];
      f16x8 hi, lo;
      split8(o, hi, lo);
      f16* dst = og_lds + ((((u * H + h) * 2 + t) * 2) * 64 + lane) * 8;
      *reinterpret_cast<f16x8*>(dst) = hi;
      *reinterpret_cast<f16x8*>(dst + 512) = lo;
    }
  }
  // this wave's output tiles: ti = wave + k*H of the 2*ncb (c_out <= 256)
  constexpr int NT = 16 / H;
  f32x16 acc[NT];
  float bo[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int ti = wave + k * H;
    const int c = (ti % ncb) * 32 + (lane & 31);
    bo[k] = b_o != nullptr && ti < 2 * ncb ? b_o[c] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int ti = wave + k * H;
    acc[k] = f32x16{};
    if (ti >= 2 * ncb) continue;   // wave-uniform
    const int u = ti / ncb, cb = ti % ncb;
#pragma unroll
    for (int hh = 0; hh < H; ++hh)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f16* a = og_lds + ((((u * H + hh) * 2 + t) * 2) * 64 + lane) * 8;
        const int64_t wo = (((int64_t)cb * H + hh) * 2 + t) * 512;
        acc[k] = mfma3(*reinterpret_cast<const f16x8*>(a), *reinterpret_cast<const f16x8*>(a + 512),
                       reinterpret_cast<const f16x8*>(wo_hi + wo)[lane],
                       reinterpret_cast<const f16x8*>(wo_lo + wo)[lane], acc[k]);
      }
  }
  // staged rows of 32 queries over og (every wave has read og after the
  // barrier below); a padded pitch where it fits
  constexpr int OG_FLOATS = H * 2048;
  float* st = reinterpret_cast<float*>(og_lds);
  const int sp = 32 * (c_out + 4) <= OG_FLOATS ? c_out + 4 : c_out;
  const int nq4 = c_out / 4;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (u == 1 && qb1 == qb0) break;   // repeated block of an odd last group
    __syncthreads();   // og read (u = 0) or the rows of block 0 stored (u = 1)
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      const int ti = wave + k * H;
      if (ti >= 2 * ncb || ti / ncb != u) continue;
      // rows = queries, lane = output column
      const int c = (ti % ncb) * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < 16; ++j) st[acc_row(j, g) * sp + c] = acc[k][j] + bo[k];
    }
    __syncthreads();
    const int q0 = (u == 0 ? qb0 : qb1) * 32;
    for (int i = threadIdx.x; i < 32 * nq4; i += H * 64) {
      const int row = i / nq4, c4 = i - row * nq4;
      if (q0 + row < P)
        *reinterpret_cast<f32x4*>(out + (int64_t)r * os_r + (int64_t)(q0 + row) * os_p + 4 * c4) =
            *reinterpret_cast<const f32x4*>(st + row * sp + 4 * c4);
    }
  }
}

// Finish of a query block's partial attention over key shards: o from
// o_part (per head, already merged), the gate from the projection of the
// query pairs, then gate, output projection and store as in the one-pass
// kernel.  Same workgroup shape and tile order as attn_f32_kernel.
template <int H>
__global__ __launch_bounds__(H * 64) void attn_f32_finish_kernel(
    const float* __restrict__ o_part, const float* __restrict__ g_ws, const f16* __restrict__ wo_hi,
    const f16* __restrict__ wo_lo, const float* __restrict__ b_o, float* __restrict__ out, int64_t os_r,
    int64_t os_p, int c_out, int nrows, int P, int nbq, int ngroups) {
  __shared__ __attribute__((aligned(1024))) f16 og_lds[2 * H * 2 * 2 * 512];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g = lane >> 5;
  const int h = wave;
  const int64_t ntile = (int64_t)ngroups * nrows;
  int64_t tile = blockIdx.x;
  if ((ntile & 7) == 0) tile = (tile & 7) * (ntile >> 3) + (tile >> 3);
  const int r = (int)(tile / ngroups);
  const int grp = (int)(tile % ngroups);
  const int qb0 = 2 * grp, qb1 = min(2 * grp + 1, nbq - 1);
  const int64_t rh = (int64_t)r * H + h;
  f32x16 O[2], G[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qb = u == 0 ? qb0 : qb1;
    const int q = qb * 32 + (lane & 31);
    const float* orow = o_part + ((int64_t)r * P + min(q, P - 1)) * (H * 32) + h * 32 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(orow + 8 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[u][4 * i + e] = q < P ? v[e] : 0.0f;
    }
    const f32x4* gt = reinterpret_cast<const f32x4*>(g_ws + (rh * nbq + qb) * 1024) + lane * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = gt[q4];
#pragma unroll
      for (int e = 0; e < 4; ++e) G[u][4 * q4 + e] = v[e];
    }
  }
  const float one[2] = {1.0f, 1.0f};
  gate_project_store<H>(og_lds, O, one, G[0], G[1], h, wave, lane, wo_hi, wo_lo, b_o, out, os_r, os_p, c_out, r, P,
                        qb0, qb1);
}


// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_pack_f32(const PackF32Args& a, hipStream_t s) {
  const int64_t n_w = (int64_t)a.nqkvg * (a.c_in / 16) * 64;
  const int64_t n_o = a.wo != nullptr ? (int64_t)(a.c_out / 32) * a.H * 2 * 64 : 0;
  const int64_t total = n_w + n_o;
  const int64_t blocks_c = ((int64_t)a.nqkvg * 32 + 3) / 4;   // 4 waves (columns) per block
  const int blocks = (int)std::max<int64_t>({int64_t(1), blocks_c, std::min<int64_t>((total + 255) / 256, 4096)});
  hipLaunchKernelGGL(pack_f32_kernel, dim3(blocks, 2), dim3(256), 0, s, (const float*)a.wq, (const float*)a.wk,
                     (const float*)a.wv, (const float*)a.wg, (const float*)a.gamma, (const float*)a.beta,
                     (const float*)a.b_g, a.c_in, a.hd, a.H, a.nqkvg, (f16*)a.w_hi, (f16*)a.w_lo, a.cst, (const float*)a.wo, (f16*)a.wo_hi, (f16*)a.wo_lo, a.c_out);
  return hipGetLastError();
}

template <int C_IN>
static hipError_t proj_f32_dispatch(const ProjF32Args& a, int num_cu, hipStream_t s) {
  using SH = ProjF32Shape<C_IN>;
  const int groups = (a.nqkvg + a.with_bias + SH::NB - 1) / SH::NB;
  const int64_t ntiles = (int64_t)(a.Pp / 32) * a.nrows;
  const int64_t want = (ntiles + SH::THREADS / kWave - 1) / (SH::THREADS / kWave);
  const int grid_x = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)num_cu * 2));
  const int rmajor = a.xs_p <= a.xs_r ? 1 : 0;
  hipLaunchKernelGGL((proj_f32_kernel<C_IN>), dim3(grid_x, groups), dim3(SH::THREADS), 0, s, (const float*)a.x,
                     a.xs_r, a.xs_p, rmajor, a.eps, (const f16*)a.w_hi, (const f16*)a.w_lo, a.cst, a.b_first,
                     a.nqkvg, a.with_bias, (const float*)a.wb, (const float*)a.gamma, (const float*)a.beta, a.hd,
                     a.q_scale, (f16*)a.q_hi, (f16*)a.q_lo, (f16*)a.k_hi, (f16*)a.k_lo, (f16*)a.v_hi, (f16*)a.v_lo,
                     a.g_ws, a.bias, a.bias_natural, a.bias_scale, a.nrows, a.P, a.Pp, a.H);
  return hipGetLastError();
}

hipError_t launch_proj_f32(const ProjF32Args& a, int num_cu, hipStream_t s) {
  if (a.nqkvg + a.with_bias < 1 || a.b_first < 0 || a.b_first + a.nqkvg > 4 * a.hd / 32 || a.Pp % 32 != 0 ||
      a.P < 1 || a.P > a.Pp || a.nrows < 1)
    return hipErrorInvalidValue;
  switch (a.c_in) {
    case 64: return proj_f32_dispatch<64>(a, num_cu, s);
    case 128: return proj_f32_dispatch<128>(a, num_cu, s);
    case 256: return proj_f32_dispatch<256>(a, num_cu, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bias_to_f32_layout(const float* src, float* dst, int H, int Pq, int Pk, int Ppq, int Ppk,
                                     hipStream_t s) {
  const int64_t total = (int64_t)H * Ppq * Ppk;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 8192));
  hipLaunchKernelGGL(bias_to_f32_layout_kernel, dim3(blocks), dim3(256), 0, s, src, dst, H, Pq, Pk, Ppq, Ppk);
  return hipGetLastError();
}

template <int H, bool HAS_MASK, int MODE>
static hipError_t attn_f32_dispatch(const AttnF32Args& a, hipStream_t s) {
  const int nbq = a.Pp / 32, nbk = a.Ppk / 32;
  const int ngroups = (nbq + 1) / 2;
  const int64_t n = (int64_t)ngroups * a.nrows;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_f32_kernel<H, HAS_MASK, MODE>), dim3((unsigned)n), dim3(H * 64), 0, s,
                     (const f16*)a.q_hi, (const f16*)a.q_lo, (const f16*)a.k_hi, (const f16*)a.k_lo,
                     (const f16*)a.v_hi, (const f16*)a.v_lo, a.g_ws, a.bias, a.mask_bits, (const f16*)a.wo_hi,
                     (const f16*)a.wo_lo, (const float*)a.b_o, (float*)a.out, a.os_r, a.os_p, a.c_out, a.nrows, a.P,
                     nbq, nbk, ngroups, a.o_part, a.lse_part);
  return hipGetLastError();
}

template <int H, bool HAS_MASK>
static hipError_t attn_f32_dispatch_mode(const AttnF32Args& a, hipStream_t s) {
  switch (a.mode) {
    case 0: return attn_f32_dispatch<H, HAS_MASK, 0>(a, s);
    case 1: return attn_f32_dispatch<H, HAS_MASK, 1>(a, s);
    case 2: return attn_f32_dispatch<H, HAS_MASK, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_f32(const AttnF32Args& a, hipStream_t s) {
  if (a.Pp < 32 || a.Pp % 32 != 0 || a.P < 1 || a.P > a.Pp || a.Ppk < 32 || a.Ppk % 32 != 0 || a.nrows < 1 ||
      a.c_out % 32 != 0 || a.c_out > 256 || (a.mode != 0 && (a.o_part == nullptr || a.lse_part == nullptr)))
    return hipErrorInvalidValue;
  const bool m = a.mask_bits != nullptr;
  if (a.H == 4) return m ? attn_f32_dispatch_mode<4, true>(a, s) : attn_f32_dispatch_mode<4, false>(a, s);
  if (a.H == 8) return m ? attn_f32_dispatch_mode<8, true>(a, s) : attn_f32_dispatch_mode<8, false>(a, s);
  return hipErrorInvalidValue;
}

template <int H>
static hipError_t finish_f32_dispatch(const AttnF32Args& a, hipStream_t s) {
  const int nbq = a.Pp / 32;
  const int ngroups = (nbq + 1) / 2;
  const int64_t n = (int64_t)ngroups * a.nrows;
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_f32_finish_kernel<H>), dim3((unsigned)n), dim3(H * 64), 0, s, a.o_part, a.g_ws,
                     (const f16*)a.wo_hi, (const f16*)a.wo_lo, (const float*)a.b_o, (float*)a.out, a.os_r, a.os_p,
                     a.c_out, a.nrows, a.P, nbq, ngroups);
  return hipGetLastError();
}

hipError_t launch_finish_f32(const AttnF32Args& a, hipStream_t s) {
  if (a.Pp < 32 || a.Pp % 32 != 0 || a.P < 1 || a.P > a.Pp || a.nrows < 1 || a.c_out % 32 != 0 || a.c_out > 256 ||
      a.o_part == nullptr)
    return hipErrorInvalidValue;
  if (a.H == 4) return finish_f32_dispatch<4>(a, s);
  if (a.H == 8) return finish_f32_dispatch<8>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
