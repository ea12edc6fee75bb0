// fp32 kernels for gated pair-biased attention on gfx950 (plain fp32 VALU
// arithmetic: no reduced-precision matrix mode anywhere on this path).
//
// Same row-attention formulation as the bf16 path.  Workspace layouts:
//   q, k, v, g [nrows][P][H*32] float (q scaled by 1/sqrt(d), g after sigmoid)
//   bias [H][P][P] float
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// LayerNorm of 32 positions into LDS (fp32, pitch c_in + 1), then every
// requested output column as a plain dot product in channel order.
// mode 0: q,k,v,g   1: q,k,v,g + bias   2: bias only
__global__ __launch_bounds__(256) void proj_f32_kernel(
    const float* __restrict__ x, int64_t xs_r, int64_t xs_p, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, const float* __restrict__ wq, const float* __restrict__ wk,
    const float* __restrict__ wv, const float* __restrict__ wg, const float* __restrict__ wb,
    const float* __restrict__ b_g, float q_scale, float* __restrict__ q_ws, float* __restrict__ k_ws,
    float* __restrict__ v_ws, float* __restrict__ g_ws, float* __restrict__ bias, float bias_scale, int c_in, int hd,
    int H, int nrows, int P, int mode) {
  extern __shared__ float xs[];   // [32][c_in + 1]
  const int pitch = c_in + 1;
  const int r = blockIdx.y;
  const int p0 = blockIdx.x * 32;
  const int tid = threadIdx.x;
  {
    const int pl = tid / 8, sub = tid % 8;   // 8 threads per position
    const int p = p0 + pl;
    const bool valid = p < P;
    const float* xp = x + (int64_t)r * xs_r + (int64_t)(valid ? p : 0) * xs_p;
    float s = 0.0f;
    for (int c = sub; c < c_in; c += 8) s += valid ? xp[c] : 0.0f;
    const float mean = group_sum<8>(s) / (float)c_in;
    float s2 = 0.0f;
    for (int c = sub; c < c_in; c += 8) {
      const float t = (valid ? xp[c] : 0.0f) - mean;
      s2 += t * t;
    }
    const float var = group_sum<8>(s2) / (float)c_in;
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int c = sub; c < c_in; c += 8)
      xs[pl * pitch + c] = valid ? (xp[c] - mean) * rstd * gamma[c] + beta[c] : 0.0f;
  }
  __syncthreads();
  const int nq = mode == 2 ? 0 : 4 * hd;
  const int nb = mode == 0 ? 0 : H;
  const int ncol = nq + nb;
  for (int idx = tid; idx < 32 * ncol; idx += blockDim.x) {
    const int pl = idx / ncol, col = idx % ncol;
    const int p = p0 + pl;
    if (p >= P) continue;
    const float* xr = xs + pl * pitch;
    if (col < nq) {
      const int t = col / hd, cc = col % hd;
      const float* w = t == 0 ? wq : t == 1 ? wk : t == 2 ? wv : wg;
      float acc = 0.0f;
      for (int k = 0; k < c_in; ++k) acc = fmaf(xr[k], w[(int64_t)k * hd + cc], acc);
      const int64_t o = ((int64_t)r * P + p) * hd + cc;
      if (t == 0) q_ws[o] = acc * q_scale;
      else if (t == 1) k_ws[o] = acc;
      else if (t == 2) v_ws[o] = acc;
      else g_ws[o] = 1.0f / (1.0f + expf(-(acc + (b_g != nullptr ? b_g[cc] : 0.0f))));
    } else {
      const int hh = col - nq;
      float acc = 0.0f;
      for (int k = 0; k < c_in; ++k) acc = fmaf(xr[k], wb[(int64_t)k * H + hh], acc);
      bias[((int64_t)hh * P + r) * P + p] = acc * bias_scale;
    }
  }
}

// One thread per (query, head): online softmax over all keys in fp32 with
// expf, then the gated output projection from LDS.
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q_ws, const float* __restrict__ k_ws, const float* __restrict__ v_ws,
    const float* __restrict__ g_ws, const float* __restrict__ bias, const uint8_t* __restrict__ mask,
    int64_t ms_r, int64_t ms_k, const float* __restrict__ wo, const float* __restrict__ b_o,
    float* __restrict__ out, int64_t os_r, int64_t os_p, int H, int c_out, int nrows, int P) {
  extern __shared__ float o_s[];   // [32][hd + 1]
  const int hd = H * 32;
  const int pitch = hd + 1;
  const int r = blockIdx.y;
  const int q0 = blockIdx.x * 32;
  const int qi = threadIdx.x % 32, h = threadIdx.x / 32;
  const int q = q0 + qi;
  const int qc = min(q, P - 1);
  float qv[32], o[32];
  const float* qp = q_ws + ((int64_t)r * P + qc) * hd + h * 32;
  for (int e = 0; e < 32; ++e) {
    qv[e] = qp[e];
    o[e] = 0.0f;
  }
  float m = -__builtin_inff(), l = 0.0f;
  const float* brow = bias + ((int64_t)h * P + qc) * P;
  for (int k = 0; k < P; ++k) {
    if (mask != nullptr && mask[(int64_t)r * ms_r + (int64_t)k * ms_k] == 0) continue;
    const float* kp = k_ws + ((int64_t)r * P + k) * hd + h * 32;
    float s = 0.0f;
    for (int e = 0; e < 32; ++e) s = fmaf(qv[e], kp[e], s);
    s += brow[k];
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);
    const float pw = expf(s - m_new);
    l = l * alpha + pw;
    const float* vp = v_ws + ((int64_t)r * P + k) * hd + h * 32;
    for (int e = 0; e < 32; ++e) o[e] = fmaf(pw, vp[e], o[e] * alpha);
    m = m_new;
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float* gp = g_ws + ((int64_t)r * P + qc) * hd + h * 32;
  for (int e = 0; e < 32; ++e) o_s[qi * pitch + h * 32 + e] = o[e] * inv * gp[e];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * c_out; idx += blockDim.x) {
    const int qq = idx / c_out, c = idx % c_out;
    const int p = q0 + qq;
    if (p >= P) continue;
    float acc = 0.0f;
    for (int k = 0; k < hd; ++k) acc = fmaf(o_s[qq * pitch + k], wo[(int64_t)k * c_out + c], acc);
    out[(int64_t)r * os_r + (int64_t)p * os_p + c] = acc + (b_o != nullptr ? b_o[c] : 0.0f);
  }
}

hipError_t launch_proj_f32(const ProjArgs& a, int mode, hipStream_t s) {
  dim3 grid((a.P + 31) / 32, a.nrows);
  const size_t lds = sizeof(float) * 32 * (a.c_in + 1);
  hipLaunchKernelGGL(proj_f32_kernel, grid, dim3(256), lds, s, (const float*)a.x, a.xs_r, a.xs_p,
                     (const float*)a.gamma, (const float*)a.beta, a.eps, (const float*)a.wq, (const float*)a.wk,
                     (const float*)a.wv, (const float*)a.wg, (const float*)a.wb, (const float*)a.b_g, a.q_scale,
                     (float*)a.q_ws, (float*)a.k_ws, (float*)a.v_ws, (float*)a.g_ws, a.bias, a.bias_scale, a.c_in,
                     a.hd, a.H, a.nrows, a.P, mode);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.P + 31) / 32, a.nrows);
  const size_t lds = sizeof(float) * 32 * (a.H * 32 + 1);
  hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(32 * a.H), lds, s, (const float*)a.q_ws, (const float*)a.k_ws,
                     (const float*)a.v_ws, (const float*)a.g_ws, (const float*)a.bias, a.mask, a.ms_r, a.ms_k, (const float*)a.wo,
                     (const float*)a.b_o, (float*)a.out, a.os_r, a.os_p, a.H, a.c_out, a.nrows, a.P);
  return hipGetLastError();
}

}  // namespace pa
