// Host-side argument bundles and launchers of the pair-attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

namespace pa {

struct PackArgs {
  const void *wq, *wk, *wv, *wg, *wo;  // natural layouts
  void *wT, *woT;                      // packed copies in the workspace
  int c_in, hd, c_out;
};

// LayerNorm + projection of nrows x P positions.  Element (r, p, c) of the
// input is x[r*xs_r + p*xs_p + c].
struct ProjArgs {
  const void* x;
  int64_t xs_r, xs_p;
  const void *gamma, *beta;
  float eps;
  const void* wT;                // bf16 path: packed q|k|v|g weights
  const void *wq, *wk, *wv, *wg; // fp32 path: natural layouts
  const void *wb, *b_g;          // both paths: w_b [c_in][H], gate bias [H*32]
  float q_scale;
  void *q_ws, *k_ws, *v_ws, *g_ws;
  float* bias;                   // pair bias output (rows = the projected rows r); fp16 when swizzled
  int bias_swizzled;             // 1: attention layout (fp16 operand order, Pp x Pp, zero padded); 0: [H][P][P] float
  float bias_scale;              // multiplies the stored bias (log2(e) for the attention layout)
  int c_in, hd, H, nrows, P, Pp;
};

struct AttnArgs {
  const void *q_ws, *k_ws, *v_ws, *g_ws;
  const void* bias;              // bf16 path: attention layout (fp16, log2 units); fp32 path: [H][P][P] float natural
  const uint8_t* mask;           // fp32 path: key kept iff mask[r*ms_r + k*ms_k] != 0 (NULL = all)
  int64_t ms_r, ms_k;
  const uint32_t* mask_bits;     // bf16 path: keep bits per (row, 32-key block), see launch_mask_bits
  const void *woT, *wo, *b_o;    // woT for bf16, wo (natural) for fp32
  void* out;                     // element (r, p, c) at out[r*os_r + p*os_p + c]
  int64_t os_r, os_p;
  int H, c_out, nrows, P, Pp;
};

hipError_t launch_pack_bf16(const PackArgs& a, hipStream_t s);
hipError_t launch_bias_to_attn_layout(const float* src, void* dst, int H, int P, int Pp, hipStream_t s);
// mode 0: q,k,v,g   1: q,k,v,g + bias   2: bias only
hipError_t launch_proj_bf16(const ProjArgs& a, int mode, int num_cu, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// keep bits [nrows][nkb] for the bf16 attention (mask may be NULL: all keys < P kept)
hipError_t launch_mask_bits(const uint8_t* mask, int64_t ms_r, int64_t ms_k, uint32_t* bits, int nrows, int P,
                            int nkb, hipStream_t s);

hipError_t launch_proj_f32(const ProjArgs& a, int mode, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

}  // namespace pa
