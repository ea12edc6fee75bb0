// Host-side argument bundles and launchers of the pair-attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

namespace pa {

struct PackArgs {
  const void *wq, *wk, *wv, *wg, *wo;  // natural layouts
  const void *gamma, *beta, *b_g;      // LayerNorm of the projected tensor, gate bias (may be NULL)
  void *wT, *woT;                      // packed images in the workspace: gamma o W (operand order), W_o^T
  float* cst;                          // [4*hd] column constants beta . W (+ b_g)
  int c_in, hd, c_out;
  // pair-bias operand (wb_img NULL: not built): w_b [b_c_in][H] with the
  // LayerNorm gamma / beta of the biased tensor; image of b_c_in/16 KB and
  // 8 constants, for ProjArgs.wb_img / wb_cst
  const void *wb = nullptr, *b_gamma = nullptr, *b_beta = nullptr;
  void* wb_img = nullptr;
  float* wb_cst = nullptr;
  int b_c_in = 0, H = 0;
  // keep bits and ranges of nrows mask rows (bits NULL: none; layout of
  // launch_mask_bits)
  const uint8_t* mask = nullptr;
  int64_t ms_r = 0, ms_k = 0;
  uint32_t* bits = nullptr;
  int nrows = 0, P = 0, nkb = 0;
};

// LayerNorm + projection of nrows x P positions.  Element (r, p, c) of the
// input is x[r*xs_r + p*xs_p + c].
struct ProjArgs {
  const void* x;
  int64_t xs_r, xs_p;
  const void *gamma, *beta;
  float eps;
  const void* wT;                // packed q|k|v|g operand image (launch_pack_bf16)
  const float* cst;              // its column constants
  const void* wb;                // w_b [c_in][H]
  void *q_ws, *k_ws, *v_ws, *g_ws;  // q and the gate from columns packed with their scales (column_scale)
  float* bias;                   // pair bias output (rows = the projected rows r); fp16 when swizzled
  int bias_swizzled;             // 1: attention layout (fp16 operand order, Pp x Pp, zero padded); 0: [H][P][P] float
  float bias_scale;              // multiplies the stored bias (log2(e) for the attention layout)
  int c_in, hd, H, nrows, P, Pp;
  // the pair-bias operand and constants from launch_pack_bf16 (NULL: each
  // workgroup builds them from wb, gamma and beta)
  const void* wb_img = nullptr;
  const float* wb_cst = nullptr;
};

struct AttnArgs {
  const void *q_ws, *k_ws, *v_ws, *g_ws;
  const void* bias;              // attention layout (fp16, log2 units)
  const uint32_t* mask_bits;     // keep bits per (row, 32-key block), see launch_mask_bits; NULL = no mask
  const int* mask_range;         // per row: first block with a kept key, one past the last (with mask_bits)
  const void *woT, *b_o;
  void* out;                     // element (r, p, c) at out[r*os_r + p*os_p + c]
  int64_t os_r, os_p;
  int H, c_out, nrows;
  int P, Pp;                     // queries (and keys in mode 0)
  // 0: one pass (gate, output projection, out); 1: one shard of Pk keys
  // (Ppk padded): its o and lse into o_part [nrows][P][H*32] / lse_part
  // [nrows][H][P]; 2: merged into the o_part / lse_part already there
  int mode;
  int Pk, Ppk;
  float *o_part, *lse_part;
};

hipError_t launch_pack_bf16(const PackArgs& a, hipStream_t s);
// caller bias [H][Pq][Pk] float (natural-log units) -> attention layout, Ppq x Ppk
hipError_t launch_bias_to_attn_layout(const float* src, void* dst, int H, int Pq, int Pk, int Ppq, int Ppk,
                                      hipStream_t s);
// mode 0: q,k,v,g   1: q,k,v,g + bias   2: bias only
hipError_t launch_proj_bf16(const ProjArgs& a, int mode, int num_cu, hipStream_t s);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
// exp2 issue-rate calibration: 2048 x 256 threads, 8 chains of `iters` exp2
// each, one float per thread into out
hipError_t launch_calib_exp2(float* out, int iters, hipStream_t s);
// gate (g_ws, layout of q), output projection and bf16 store of merged partial
// outputs o_part (fields g_ws, woT, b_o, out, os_r, os_p, H, c_out, nrows, P, Pp, o_part)
hipError_t launch_finish_bf16(const AttnArgs& a, hipStream_t s);
// keep bits [nrows][nkb] for the attention (mask may be NULL: all keys < P
// kept), followed by each row's key-block range [nrows][2] (mask_range_of)
hipError_t launch_mask_bits(const uint8_t* mask, int64_t ms_r, int64_t ms_k, uint32_t* bits, int nrows, int P,
                            int nkb, hipStream_t s);
// workspace bytes of the keep bits and the ranges, and where the ranges start
inline size_t mask_bits_bytes(int64_t nrows, int64_t nkb) {
  return (size_t)((nrows * nkb + 3) / 4 * 4) * 4 + (size_t)nrows * 8;
}
inline int* mask_range_of(uint32_t* bits, int64_t nrows, int64_t nkb) {
  return reinterpret_cast<int*>(bits + (nrows * nkb + 3) / 4 * 4);
}

// The fused end of the bf16 ring: out = (sigmoid(LN(x) W_g + b_g) * o) W_o + b_o
// for query pairs x (element (r, p, ch) at x[r*xs_r + p*xs_p + ch]) and the
// assembled per-head outputs o_part [nrows][P][H*32]; wimg / cst / woT come
// from launch_pack_bf16.  Supported where its LDS operands fit.
struct FinishFusedArgs {
  const void* x;
  int64_t xs_r, xs_p;
  float eps;
  const void* wimg;
  const float* cst;
  const float* o_part;
  const void *woT, *b_o;
  void* out;
  int64_t os_r, os_p;
  int c, H, nrows, P, Pp;
};
bool finish_fused_bf16_supported(int c, int H);
hipError_t launch_finish_fused_bf16(const FinishFusedArgs& a, int num_cu, hipStream_t s);

// ---- fp32 path (fp16-pair operands on the matrix cores) ----
// Packs the gamma-folded q|k|v|g projection operands (nqkvg blocks of 32
// columns) and, when wo != NULL, the W_o operand.
struct PackF32Args {
  const void *wq, *wk, *wv, *wg, *gamma, *beta, *b_g, *wo;
  void *w_hi, *w_lo;             // [nqkvg][c_in/16][64][8] fp16 each
  float* cst;                    // [nqkvg * 32]
  void *wo_hi, *wo_lo;           // [c_out/32][H][2][64][8] fp16 each
  int c_in, hd, H, nqkvg, c_out;
};
struct ProjF32Args {
  const void* x;
  int64_t xs_r, xs_p;
  float eps;
  const void *w_hi, *w_lo;       // packed q|k|v|g operands (launch_pack_f32)
  const float* cst;
  int b_first, nqkvg;            // q|k|v|g blocks [b_first, b_first + nqkvg) of the packed list
  int with_bias;                 // 1: also the pair bias, from wb with LayerNorm gamma and beta
  const void *wb, *gamma, *beta;
  int hd;
  float q_scale;
  void *q_hi, *q_lo, *k_hi, *k_lo, *v_hi, *v_lo;
  float* g_ws;
  float* bias;                   // tiled S^T image (log2 units via bias_scale) or, with bias_natural, [H][P][P]
  int bias_natural;
  float bias_scale;
  int c_in, H, nrows, P, Pp;
};
struct AttnF32Args {
  const void *q_hi, *q_lo, *k_hi, *k_lo, *v_hi, *v_lo;
  const float* g_ws;
  const float* bias;             // tiled S^T image, log2 units, -inf at padded keys
  const uint32_t* mask_bits;     // NULL = no mask
  const void *wo_hi, *wo_lo;
  const void* b_o;
  void* out;
  int64_t os_r, os_p;
  int H, c_out, nrows;
  int P, Pp;                     // queries (and keys when Pk = P)
  int Pk, Ppk;                   // keys
  // 0: one pass (gate, output projection, out); 1: this key shard's o and
  // lse into o_part [nrows][P][H*32] / lse_part [nrows][H][P]; 2: merged
  // into the o_part / lse_part already there
  int mode;
  float *o_part, *lse_part;
};
hipError_t launch_pack_f32(const PackF32Args& a, hipStream_t s);
hipError_t launch_proj_f32(const ProjF32Args& a, int num_cu, hipStream_t s);
hipError_t launch_bias_to_f32_layout(const float* src, float* dst, int H, int Pq, int Pk, int Ppq, int Ppk,
                                     hipStream_t s);
hipError_t launch_attn_f32(const AttnF32Args& a, hipStream_t s);
// gate (g_ws), output projection and store of merged partial outputs o_part
hipError_t launch_finish_f32(const AttnF32Args& a, hipStream_t s);

// Flag words of the debug build's index checks, one per source file: each
// call reads its file's word and clears it (0 in the release build).
hipError_t debug_take_attn(unsigned int* out);
hipError_t debug_take_bf16(unsigned int* out);

}  // namespace pa
