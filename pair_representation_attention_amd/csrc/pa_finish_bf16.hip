// The end of ring attention on the bf16 path, fused: for the query pairs x
// of R rows and the per-head outputs o assembled over every key shard,
//   out = (sigmoid(LN(x) W_g + b_g) * o) W_o + b_o
// in one pass.  The gate is computed where it is used and never stored.
//
// Every wave works on its own tiles of 32 query positions of one row, with
// no barrier in the tile loop (as in the projection kernel):
//   1. LayerNorm of the tile in registers (fp32 statistics; the affine map is
//      folded into the packed W_g operand image and its column constants);
//   2. per head b: the gate block out^T = W_g^T x^T on the matrix cores
//      (rows = the head's 32 channels, lane = position), sigmoid, times o,
//      rounded to fp16 into the wave's own LDS tile (position-major);
//   3. per 32 output channels: W_o^T x og^T on the matrix cores, + b_o,
//      bf16 store.
// The W_g image (HD x C_IN fp16) is copied into LDS once per workgroup;
// W_o operands are read from the cache at their MFMAs.
#include <atomic>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int C_IN, int H>
struct FinishShape {
  static constexpr int HD = H * 32, KS = C_IN / 16, OP = HD + 8, KO = HD / 16;
  static constexpr int WAVES = 4;
  static constexpr int WG_BYTES = HD * C_IN * 2;                 // W_g operand image
  static constexpr int OG_BYTES = WAVES * 32 * OP * 2;           // one gated-o tile per wave
  static constexpr int LDS = WG_BYTES + OG_BYTES + HD * 4;
  static constexpr bool FITS = LDS <= 160 * 1024;
};

template <int C_IN, int H>
__global__ __launch_bounds__(256) void finish_fused_kernel(
    const bf16* __restrict__ x, int64_t xs_r, int64_t xs_p, float eps, const f16* __restrict__ wimg,
    const float* __restrict__ cst, const float* __restrict__ o_part, const f16* __restrict__ woT,
    const bf16* __restrict__ b_o, bf16* __restrict__ out, int64_t os_r, int64_t os_p, int nrows, int P, int nbq) {
  using SH = FinishShape<C_IN, H>;
  constexpr int HD = SH::HD, KS = SH::KS, OP = SH::OP, KO = SH::KO, CBN = C_IN / 32;
  static_assert(SH::FITS, "finish operands exceed LDS");
  __shared__ __attribute__((aligned(1024))) char smem[SH::LDS];
  f16* wg_lds = reinterpret_cast<f16*>(smem);
  f16* og_all = reinterpret_cast<f16*>(smem + SH::WG_BYTES);
  float* cg = reinterpret_cast<float*>(smem + SH::WG_BYTES + SH::OG_BYTES);

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lq = lane & 31, g = lane >> 5;
  f16* og = og_all + wave * 32 * OP;

  // the gate columns are blocks [3 HD/32, 4 HD/32) of the packed q|k|v|g image
  {
    const f16x8* src = reinterpret_cast<const f16x8*>(wimg) + (int64_t)(3 * HD / 32) * KS * 64;
    f16x8* dst = reinterpret_cast<f16x8*>(wg_lds);
    for (int i = tid; i < HD / 32 * KS * 64; i += 256) dst[i] = src[i];
    for (int n = tid; n < HD; n += 256) cg[n] = cst[3 * HD + n];
  }
  __syncthreads();

  const int64_t ntiles = (int64_t)nrows * nbq;
  const int64_t stride = (int64_t)gridDim.x * SH::WAVES;
  auto load_tile = [&](int64_t tile, bf16x8* raw) {
    if (tile < ntiles) {
      const int r = (int)(tile / nbq), p = (int)(tile % nbq) * 32 + lq;
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

  int64_t tile = (int64_t)blockIdx.x * SH::WAVES + wave;
  bf16x8 pre[KS];
  load_tile(tile, pre);
  for (; tile < ntiles; tile += stride) {
    bf16x8 raw[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) raw[t] = pre[t];
    load_tile(tile + stride, pre);
    const int r = (int)(tile / nbq), p = (int)(tile % nbq) * 32 + lq;
    const bool valid = p < P;
    const float* orow = o_part + ((int64_t)r * P + (valid ? p : 0)) * HD;
    // at H = 4 the tile's o values (64 registers) are loaded before
    // LayerNorm, so that their latency hides behind it
    constexpr bool OPF = H == 4;
    f32x4 opre[OPF ? H : 1][OPF ? 4 : 1];
    if constexpr (OPF) {
#pragma unroll
      for (int b = 0; b < H; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          opre[b][jj] = valid ? *reinterpret_cast<const f32x4*>(orow + b * 32 + jj * 8 + g * 4) : f32x4{};
    }

    // ---- LayerNorm (two passes, fp32) ----
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
        const float dlt = bf2f(raw[t][e]) - mean;
        s2 += dlt * dlt;
      }
    s2 += __shfl_xor(s2, 32, 64);
    const float rstd = 1.0f / __builtin_sqrtf(s2 * (1.0f / C_IN) + eps);
    f16x8 X[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) X[t][e] = f2h_sat((bf2f(raw[t][e]) - mean) * rstd);

    // ---- per head: gate, times o, into the wave's LDS tile ----
#pragma unroll
    for (int b = 0; b < H; ++b) {
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KS; ++t)
        acc = mfma32(*reinterpret_cast<const f16x8*>(wg_lds + (b * KS + t) * 512 + lane * 8), X[t], acc);
      // register 4jj+e holds channel jj*8 + g*4 + e of head b for position p
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int ch = jj * 8 + g * 4;
        f32x4 ov = {};
        if constexpr (OPF) ov = opre[b][jj];
        else if (valid) ov = *reinterpret_cast<const f32x4*>(orow + b * 32 + ch);
        const f32x4 cc = *reinterpret_cast<const f32x4*>(cg + b * 32 + ch);
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gate = sigmoid_from_log2(acc[jj * 4 + e] + cc[e]);   // columns scaled by -log2(e)
          v[e] = f2h_sat(ov[e] * gate);
        }
        *reinterpret_cast<f16x4*>(og + lq * OP + b * 32 + ch) = v;
      }
    }

    // ---- output projection: rows = output channels, lane = position ----
#pragma unroll 2
    for (int cb = 0; cb < CBN; ++cb) {
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < KO; ++t)
        acc = mfma32(ld16(woT + (int64_t)(cb * 32 + lq) * HD + t * 16 + g * 8),
                     *reinterpret_cast<const f16x8*>(og + lq * OP + t * 16 + g * 8), acc);
      if (valid) {
        bf16* dst = out + (int64_t)r * os_r + (int64_t)p * os_p + cb * 32;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = jj * 8 + g * 4 + e;
            ov[e] = f2bf(acc[jj * 4 + e] + (b_o != nullptr ? bf2f(b_o[cb * 32 + c]) : 0.0f));
          }
          st8(dst + jj * 8 + g * 4, ov);
        }
      }
    }
  }
}

template <int C_IN, int H>
static hipError_t finish_fused_dispatch(const FinishFusedArgs& a, int num_cu, hipStream_t s) {
  using SH = FinishShape<C_IN, H>;
  if constexpr (!SH::FITS) {
    return hipErrorInvalidValue;
  } else {
    const int nbq = a.Pp / 32;
    if (nbq < 1 || a.Pp != nbq * 32 || a.P < 1 || a.P > a.Pp || a.nrows < 1) return hipErrorInvalidValue;
    static std::atomic<int> wg_cache{0};   // resident workgroups per CU, asked once per instance
    int per_cu = wg_cache.load(std::memory_order_relaxed);
    if (per_cu == 0) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, finish_fused_kernel<C_IN, H>, 256, 0) != hipSuccess ||
          n < 1)
        n = 1;
      per_cu = n;
      wg_cache.store(n, std::memory_order_relaxed);
    }
    const int64_t ntiles = (int64_t)a.nrows * nbq;
    const int64_t want = (ntiles + SH::WAVES - 1) / SH::WAVES;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)num_cu * per_cu));
    hipLaunchKernelGGL((finish_fused_kernel<C_IN, H>), dim3(grid), dim3(256), 0, s, (const bf16*)a.x, a.xs_r,
                       a.xs_p, a.eps, (const f16*)a.wimg, a.cst, a.o_part, (const f16*)a.woT, (const bf16*)a.b_o,
                       (bf16*)a.out, a.os_r, a.os_p, a.nrows, a.P, nbq);
    return hipGetLastError();
  }
}

bool finish_fused_bf16_supported(int c, int H) {
  switch (c) {
    case 64: return H == 4 ? FinishShape<64, 4>::FITS : H == 8 && FinishShape<64, 8>::FITS;
    case 128: return H == 4 ? FinishShape<128, 4>::FITS : H == 8 && FinishShape<128, 8>::FITS;
    case 256: return H == 4 ? FinishShape<256, 4>::FITS : H == 8 && FinishShape<256, 8>::FITS;
    default: return false;
  }
}

hipError_t launch_finish_fused_bf16(const FinishFusedArgs& a, int num_cu, hipStream_t s) {
  if (a.H == 4) {
    if (a.c == 64) return finish_fused_dispatch<64, 4>(a, num_cu, s);
    if (a.c == 128) return finish_fused_dispatch<128, 4>(a, num_cu, s);
    if (a.c == 256) return finish_fused_dispatch<256, 4>(a, num_cu, s);
  } else if (a.H == 8) {
    if (a.c == 64) return finish_fused_dispatch<64, 8>(a, num_cu, s);
    if (a.c == 128) return finish_fused_dispatch<128, 8>(a, num_cu, s);
    if (a.c == 256) return finish_fused_dispatch<256, 8>(a, num_cu, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
