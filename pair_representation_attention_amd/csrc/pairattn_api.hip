// C ABI of the pair-attention library: argument checks, workspace carving and
// kernel launches.  Every entry point is declared and documented in
// include/pairattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "pa_launch.h"
#include "pairattn.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

constexpr size_t kAlign = 256;
constexpr size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline int64_t pad32(int64_t v) { return (v + 31) / 32 * 32; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_c(int64_t c) { return c == 64 || c == 128 || c == 256; }
bool supported_h(int64_t H) { return H == 4 || H == 8; }

// Largest attention-row count a launch grid can address (grid.y <= 65535
// with 4 rows per workgroup on the bf16 path, 1 row on the fp32 path).
constexpr int64_t kMaxRowsBf16 = 65535LL * 4;
constexpr int64_t kMaxRowsF32 = 65535LL;
constexpr int64_t kMaxPositions = 1LL << 20;

// ---- workspace layout -----------------------------------------------------
struct Layout {
  size_t wT = 0, woT = 0, q = 0, k = 0, v = 0, g = 0, bias = 0, bits = 0, total = 0;
};

// nrows x P positions, c_in input channels, c_out output channels.
Layout make_layout(int64_t nrows, int64_t P, int64_t c_in, int64_t c_out, int64_t H, int32_t dtype,
                   bool with_bias) {
  Layout L;
  const int64_t hd = H * 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  if (dtype == PAIRATTN_BF16) {
    const int64_t Pp = pad32(P);
    L.wT = take((size_t)4 * hd * c_in * 2);
    L.woT = take((size_t)c_out * hd * 2);
    L.q = take((size_t)nrows * H * Pp * 32 * 2);
    L.k = take((size_t)nrows * H * Pp * 32 * 2);
    L.v = take((size_t)nrows * H * 32 * Pp * 2);
    L.g = take((size_t)nrows * H * Pp * 32 * 2);   // gate in the layout of q
    // the attention reads the bias as fp16 in operand order, Pp x Pp, log2
    // units; a caller-provided bias (row block) is converted into it as well
    L.bias = take((size_t)H * Pp * Pp * 2);
    L.bits = take((size_t)nrows * (Pp / 32) * 4);
  } else {
    L.q = take((size_t)nrows * P * hd * 4);
    L.k = take((size_t)nrows * P * hd * 4);
    L.v = take((size_t)nrows * P * hd * 4);
    L.g = take((size_t)nrows * P * hd * 4);
    if (with_bias) L.bias = take((size_t)H * P * P * 4);
  }
  L.total = off;
  return L;
}

// ---- device check -----------------------------------------------------------
struct DevInfo {
  int state = 0;  // 0 unknown, 1 gfx950, -1 other
  int num_cu = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

int check_device(int* num_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(PAIRATTN_ERR_DEVICE, "no current HIP device");
  if (dev >= 64) return fail(PAIRATTN_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& d = g_dev[dev];
  if (d.state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(PAIRATTN_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    d.state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    d.num_cu = prop.multiProcessorCount;
    if (d.state < 0) {
      return fail(PAIRATTN_ERR_DEVICE, "device %d is %s; this library runs on gfx950 only", dev,
                  prop.gcnArchName);
    }
  }
  if (d.state < 0) return fail(PAIRATTN_ERR_DEVICE, "device %d is not gfx950", dev);
  *num_cu = d.num_cu;
  return PAIRATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PAIRATTN_OK;
  return fail(PAIRATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t elt_bytes(int32_t dtype) { return dtype == PAIRATTN_BF16 ? 2 : 4; }

// ---- shared parameter checks ---------------------------------------------------
int check_params(const pairattn_params* p, bool need_qkvgo, bool need_lnz) {
  if (p == nullptr) return fail(PAIRATTN_ERR_ARG, "params is NULL");
  if (p->dtype != PAIRATTN_F32 && p->dtype != PAIRATTN_BF16)
    return fail(PAIRATTN_ERR_ARG, "params->dtype %d is neither PAIRATTN_F32 nor PAIRATTN_BF16", p->dtype);
  if (!(p->ln_eps >= 0.0f) || !std::isfinite(p->ln_eps))
    return fail(PAIRATTN_ERR_ARG, "params->ln_eps must be finite and >= 0");
  struct {
    const void* ptr;
    const char* name;
    bool required;
  } items[] = {
      {p->ln_gamma, "ln_gamma", true},
      {p->ln_beta, "ln_beta", true},
      {p->w_b, "w_b", true},
      {p->w_q, "w_q", need_qkvgo},
      {p->w_k, "w_k", need_qkvgo},
      {p->w_v, "w_v", need_qkvgo},
      {p->w_g, "w_g", need_qkvgo},
      {p->w_o, "w_o", need_qkvgo},
      {p->b_g, "b_g", false},
      {p->b_o, "b_o", false},
      {p->lnz_gamma, "lnz_gamma", need_lnz},
      {p->lnz_beta, "lnz_beta", need_lnz},
  };
  for (auto& it : items) {
    if (it.required && it.ptr == nullptr) return fail(PAIRATTN_ERR_ARG, "params->%s is NULL", it.name);
    if (it.ptr != nullptr && !aligned16(it.ptr))
      return fail(PAIRATTN_ERR_ARG, "params->%s is not 16-byte aligned", it.name);
  }
  return PAIRATTN_OK;
}

int check_shape_common(int64_t I, int64_t c, int64_t H, int64_t d, int32_t dtype) {
  if (I < 1) return fail(PAIRATTN_ERR_ARG, "I must be >= 1 (got %lld)", (long long)I);
  if (c < 1 || H < 1 || d < 1) return fail(PAIRATTN_ERR_ARG, "channel, head and head-width sizes must be >= 1");
  if (d != 32) return fail(PAIRATTN_ERR_UNSUPPORTED, "head width d=%lld unsupported (only 32)", (long long)d);
  if (!supported_h(H)) return fail(PAIRATTN_ERR_UNSUPPORTED, "H=%lld unsupported (4 or 8)", (long long)H);
  if (!supported_c(c))
    return fail(PAIRATTN_ERR_UNSUPPORTED, "channel count %lld unsupported (64, 128 or 256)", (long long)c);
  if (I > kMaxPositions) return fail(PAIRATTN_ERR_UNSUPPORTED, "I=%lld exceeds 2^20", (long long)I);
  (void)dtype;
  return PAIRATTN_OK;
}

int check_rows_limit(int64_t nrows, int32_t dtype) {
  const int64_t lim = dtype == PAIRATTN_BF16 ? kMaxRowsBf16 : kMaxRowsF32;
  if (nrows > lim)
    return fail(PAIRATTN_ERR_UNSUPPORTED, "%lld attention rows exceed the launch limit %lld", (long long)nrows,
                (long long)lim);
  return PAIRATTN_OK;
}

int check_workspace(const pairattn_params* p, size_t need) {
  if (need == 0) return PAIRATTN_OK;
  if (p->workspace == nullptr) return fail(PAIRATTN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(p->workspace) & (kAlign - 1)) != 0)
    return fail(PAIRATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (p->workspace_bytes < need)
    return fail(PAIRATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", p->workspace_bytes, need);
  return PAIRATTN_OK;
}

#define PA_TRY(expr)              \
  do {                            \
    const int _st = (expr);       \
    if (_st != PAIRATTN_OK) return _st; \
  } while (0)

char* ws_at(const pairattn_params* p, size_t off) { return static_cast<char*>(p->workspace) + off; }

// ---- optional per-kernel timing (HIP events on the call's stream) ----------
constexpr int kMaxMarks = 8;
struct Timing {
  bool enabled = false;
  bool created = false;
  hipEvent_t ev[kMaxMarks];
  const char* name[kMaxMarks];
  int n = 0;
};
thread_local Timing g_tm;

void tm_begin(hipStream_t s) {
  Timing& t = g_tm;
  t.n = 0;
  if (!t.enabled) return;
  if (!t.created) {
    for (int i = 0; i < kMaxMarks; ++i) (void)hipEventCreate(&t.ev[i]);
    t.created = true;
  }
  (void)hipEventRecord(t.ev[0], s);
  t.name[0] = "";
  t.n = 1;
}

void tm_mark(hipStream_t s, const char* stage) {
  Timing& t = g_tm;
  if (!t.enabled || t.n == 0 || t.n >= kMaxMarks) return;
  (void)hipEventRecord(t.ev[t.n], s);
  t.name[t.n] = stage;
  ++t.n;
}

}  // namespace

// ============================================================================
extern "C" {

int pairattn_version(void) { return 10000; }

int pairattn_timing_enable(int enable) {
  const int prev = g_tm.enabled ? 1 : 0;
  g_tm.enabled = enable != 0;
  g_tm.n = 0;
  return prev;
}

int pairattn_timing_read(float* ms, const char** names, int cap) {
  Timing& t = g_tm;
  if (!t.enabled || t.n < 2) return 0;
  if (hipEventSynchronize(t.ev[t.n - 1]) != hipSuccess) return -PAIRATTN_ERR_HIP;
  int k = 0;
  for (int i = 1; i < t.n && k < cap; ++i, ++k) {
    float v = 0.0f;
    if (hipEventElapsedTime(&v, t.ev[i - 1], t.ev[i]) != hipSuccess) return -PAIRATTN_ERR_HIP;
    if (ms != nullptr) ms[k] = v;
    if (names != nullptr) names[k] = t.name[i];
  }
  return k;
}

const char* pairattn_status_string(int status) {
  switch (status) {
    case PAIRATTN_OK: return "ok";
    case PAIRATTN_ERR_ARG: return "invalid argument";
    case PAIRATTN_ERR_UNSUPPORTED: return "unsupported shape or option";
    case PAIRATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case PAIRATTN_ERR_DEVICE: return "device is not a gfx950 GPU";
    case PAIRATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pairattn_last_error(void) { return g_err; }

size_t pairattn_tri_workspace_bytes(int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || I < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_z) || I > kMaxPositions)
    return 0;
  return make_layout(I, I, c_z, c_z, H, dtype, true).total;
}

size_t pairattn_msa_workspace_bytes(int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H, int64_t d,
                                    int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || S < 1 || I < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_m) || !supported_c(c_z) || I > kMaxPositions)
    return 0;
  return make_layout(S, I, c_m, c_m, H, dtype, true).total;
}

size_t pairattn_rows_workspace_bytes(int64_t R, int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || R < 1 || I < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_z) || I > kMaxPositions)
    return 0;
  return make_layout(R, I, c_z, c_z, H, dtype, false).total;
}

int pairattn_validate_tri(const void* z, const uint8_t* mask, const pairattn_params* p, const void* out,
                          int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t orientation) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, false));
  if (z == nullptr || out == nullptr) return fail(PAIRATTN_ERR_ARG, "z and out must not be NULL");
  if (!aligned16(z) || !aligned16(out)) return fail(PAIRATTN_ERR_ARG, "z and out must be 16-byte aligned");
  if (orientation != PAIRATTN_START && orientation != PAIRATTN_END)
    return fail(PAIRATTN_ERR_ARG, "orientation %d is neither PAIRATTN_START nor PAIRATTN_END", orientation);
  PA_TRY(check_shape_common(I, c_z, H, d, p->dtype));
  PA_TRY(check_rows_limit(I, p->dtype));
  const size_t zbytes = (size_t)I * I * c_z * elt_bytes(p->dtype);
  if (overlaps(out, zbytes, z, zbytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps z");
  if (mask != nullptr && overlaps(out, zbytes, mask, (size_t)I * I)) return fail(PAIRATTN_ERR_ARG, "out overlaps mask");
  const size_t need = pairattn_tri_workspace_bytes(I, c_z, H, d, p->dtype);
  PA_TRY(check_workspace(p, need));
  if (overlaps(out, zbytes, p->workspace, p->workspace_bytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps the workspace");
  return PAIRATTN_OK;
}

int pairattn_validate_msa(const void* m, const void* z, const uint8_t* mask, const pairattn_params* p,
                          const void* out, int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H, int64_t d) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, true));
  if (m == nullptr || z == nullptr || out == nullptr) return fail(PAIRATTN_ERR_ARG, "m, z and out must not be NULL");
  if (!aligned16(m) || !aligned16(z) || !aligned16(out))
    return fail(PAIRATTN_ERR_ARG, "m, z and out must be 16-byte aligned");
  if (S < 1) return fail(PAIRATTN_ERR_ARG, "S must be >= 1 (got %lld)", (long long)S);
  PA_TRY(check_shape_common(I, c_m, H, d, p->dtype));
  if (c_z < 1) return fail(PAIRATTN_ERR_ARG, "c_z must be >= 1");
  if (!supported_c(c_z))
    return fail(PAIRATTN_ERR_UNSUPPORTED, "c_z=%lld unsupported (64, 128 or 256)", (long long)c_z);
  PA_TRY(check_rows_limit(S, p->dtype));
  PA_TRY(check_rows_limit(I, p->dtype));
  const size_t eb = elt_bytes(p->dtype);
  const size_t obytes = (size_t)S * I * c_m * eb;
  if (overlaps(out, obytes, m, obytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps m");
  if (overlaps(out, obytes, z, (size_t)I * I * c_z * eb)) return fail(PAIRATTN_ERR_ARG, "out overlaps z");
  if (mask != nullptr && overlaps(out, obytes, mask, (size_t)S * I)) return fail(PAIRATTN_ERR_ARG, "out overlaps mask");
  const size_t need = pairattn_msa_workspace_bytes(S, I, c_m, c_z, H, d, p->dtype);
  PA_TRY(check_workspace(p, need));
  if (overlaps(out, obytes, p->workspace, p->workspace_bytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps the workspace");
  return PAIRATTN_OK;
}

int pairattn_validate_rows(const void* z_rows, const float* bias, const uint8_t* mask_rows,
                           const pairattn_params* p, const void* out_rows, int64_t R, int64_t I, int64_t c_z,
                           int64_t H, int64_t d) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, false));
  if (z_rows == nullptr || bias == nullptr || out_rows == nullptr)
    return fail(PAIRATTN_ERR_ARG, "z_rows, bias and out_rows must not be NULL");
  if (!aligned16(z_rows) || !aligned16(bias) || !aligned16(out_rows))
    return fail(PAIRATTN_ERR_ARG, "z_rows, bias and out_rows must be 16-byte aligned");
  if (R < 1) return fail(PAIRATTN_ERR_ARG, "R must be >= 1 (got %lld)", (long long)R);
  PA_TRY(check_shape_common(I, c_z, H, d, p->dtype));
  PA_TRY(check_rows_limit(R, p->dtype));
  const size_t obytes = (size_t)R * I * c_z * elt_bytes(p->dtype);
  if (overlaps(out_rows, obytes, z_rows, obytes)) return fail(PAIRATTN_ERR_ARG, "out_rows overlaps z_rows");
  if (overlaps(out_rows, obytes, bias, (size_t)H * I * I * 4)) return fail(PAIRATTN_ERR_ARG, "out_rows overlaps bias");
  const size_t need = pairattn_rows_workspace_bytes(R, I, c_z, H, d, p->dtype);
  PA_TRY(check_workspace(p, need));
  if (overlaps(out_rows, obytes, p->workspace, p->workspace_bytes))
    return fail(PAIRATTN_ERR_ARG, "out_rows overlaps the workspace");
  return PAIRATTN_OK;
}

// ---------------------------------------------------------------------------
// One launch sequence for all three operations: (pack) -> projections of
// the attended tensor -> (pair bias of a separate tensor) -> attention.
// ---------------------------------------------------------------------------
static int run_row_attention(const pairattn_params* p, const Layout& L, hipStream_t s, int num_cu,
                             // attended tensor
                             const void* x, int64_t xs_r, int64_t xs_p, int64_t c, int64_t nrows, int64_t P, int64_t H,
                             // bias: computed in the projection (bias_in_proj), from a separate tensor (zb != NULL), or given
                             bool bias_in_proj, const void* zb, int64_t zb_c, const float* bias_given,
                             // mask and output addressing
                             const uint8_t* mask, int64_t ms_r, int64_t ms_k, void* out, int64_t os_r, int64_t os_p) {
  const int64_t hd = H * 32;
  const bool bf = p->dtype == PAIRATTN_BF16;
  const int Pp = (int)pad32(P);
  // bf16 path: the attention reads the workspace bias ([H][P][Pp], log2 units);
  // fp32 path: [H][P][P] natural units, the caller's own array for row blocks
  float* bias_ws = (bf || bias_given == nullptr) ? reinterpret_cast<float*>(ws_at(p, L.bias)) : nullptr;
  const void* bias = (bf || bias_given == nullptr) ? (const void*)bias_ws : (const void*)bias_given;
  const int bias_swz = bf ? 1 : 0;
  const float bias_scale = bf ? 1.4426950408889634f : 1.0f;

  pa::ProjArgs pj{};
  pj.x = x;
  pj.xs_r = xs_r;
  pj.xs_p = xs_p;
  pj.gamma = p->ln_gamma;
  pj.beta = p->ln_beta;
  pj.eps = p->ln_eps;
  pj.wq = p->w_q;
  pj.wk = p->w_k;
  pj.wv = p->w_v;
  pj.wg = p->w_g;
  pj.wb = p->w_b;
  pj.b_g = p->b_g;
  pj.q_ws = ws_at(p, L.q);
  pj.k_ws = ws_at(p, L.k);
  pj.v_ws = ws_at(p, L.v);
  pj.g_ws = ws_at(p, L.g);
  pj.bias = bias_ws;
  pj.bias_swizzled = bias_swz;
  pj.bias_scale = bias_scale;
  pj.c_in = (int)c;
  pj.hd = (int)hd;
  pj.H = (int)H;
  pj.nrows = (int)nrows;
  pj.P = (int)P;
  pj.Pp = Pp;
  const int mode = bias_in_proj ? 1 : 0;

  tm_begin(s);
  if (bf) {
    pa::PackArgs pk{p->w_q, p->w_k, p->w_v, p->w_g, p->w_o, ws_at(p, L.wT), ws_at(p, L.woT), (int)c, (int)hd, (int)c};
    PA_TRY(hip_status(pa::launch_pack_bf16(pk, s), "weight packing launch"));
    tm_mark(s, "pack");
    pj.wT = ws_at(p, L.wT);
    pj.q_scale = 1.4426950408889634f / std::sqrt(32.0f);
    PA_TRY(hip_status(pa::launch_proj_bf16(pj, mode, num_cu, s), "projection launch"));
  } else {
    pj.q_scale = 1.0f / std::sqrt(32.0f);
    PA_TRY(hip_status(pa::launch_proj_f32(pj, mode, s), "projection launch"));
  }
  tm_mark(s, "projection");

  if (zb != nullptr) {   // MSA: bias from the pair tensor with its own LayerNorm
    pa::ProjArgs pb{};
    pb.x = zb;
    pb.xs_r = P * zb_c;
    pb.xs_p = zb_c;
    pb.gamma = p->lnz_gamma;
    pb.beta = p->lnz_beta;
    pb.eps = p->ln_eps;
    pb.wb = p->w_b;
    pb.bias = bias_ws;
    pb.bias_swizzled = bias_swz;
    pb.bias_scale = bias_scale;
    pb.c_in = (int)zb_c;
    pb.hd = (int)hd;
    pb.H = (int)H;
    pb.nrows = (int)P;
    pb.P = (int)P;
    pb.Pp = Pp;
    if (bf) PA_TRY(hip_status(pa::launch_proj_bf16(pb, 2, num_cu, s), "pair-bias launch"));
    else PA_TRY(hip_status(pa::launch_proj_f32(pb, 2, s), "pair-bias launch"));
    tm_mark(s, "pair_bias");
  }
  if (bf && bias_given != nullptr) {   // row block: caller's bias -> attention layout
    PA_TRY(hip_status(pa::launch_bias_to_attn_layout(bias_given, bias_ws, (int)H, (int)P, Pp, s), "bias copy launch"));
    tm_mark(s, "bias_copy");
  }

  pa::AttnArgs at{};
  at.q_ws = pj.q_ws;
  at.k_ws = pj.k_ws;
  at.v_ws = pj.v_ws;
  at.g_ws = pj.g_ws;
  at.bias = bias;
  at.mask = mask;
  // bf16 path: keep bits only when there is a mask (without one the kernel
  // drops just the keys past P, which it computes)
  at.mask_bits = (bf && mask != nullptr) ? reinterpret_cast<const uint32_t*>(ws_at(p, L.bits)) : nullptr;
  at.ms_r = ms_r;
  at.ms_k = ms_k;
  at.woT = bf ? ws_at(p, L.woT) : nullptr;
  at.wo = p->w_o;
  at.b_o = p->b_o;
  at.out = out;
  at.os_r = os_r;
  at.os_p = os_p;
  at.H = (int)H;
  at.c_out = (int)c;
  at.nrows = (int)nrows;
  at.P = (int)P;
  at.Pp = Pp;
  if (bf && mask != nullptr) {
    PA_TRY(hip_status(pa::launch_mask_bits(mask, ms_r, ms_k, reinterpret_cast<uint32_t*>(ws_at(p, L.bits)),
                                           (int)nrows, (int)P, Pp / 32, s),
                      "mask bits launch"));
    tm_mark(s, "mask_bits");
  }
  if (bf) PA_TRY(hip_status(pa::launch_attn_bf16(at, s), "attention launch"));
  else PA_TRY(hip_status(pa::launch_attn_f32(at, s), "attention launch"));
  tm_mark(s, "attention");
  return PAIRATTN_OK;
}

int pairattn_tri_fwd(const void* z, const uint8_t* mask, const pairattn_params* p, void* out, int64_t I, int64_t c_z,
                     int64_t H, int64_t d, int32_t orientation, void* stream) {
  PA_TRY(pairattn_validate_tri(z, mask, p, out, I, c_z, H, d, orientation));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(I, I, c_z, c_z, H, p->dtype, true);
  const bool start = orientation == PAIRATTN_START;
  // START: row i, position j -> pair (i, j); END: row j, position i -> pair (i, j)
  const int64_t xs_r = start ? I * c_z : c_z;
  const int64_t xs_p = start ? c_z : I * c_z;
  const int64_t ms_r = start ? I : 1;
  const int64_t ms_k = start ? 1 : I;
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, z, xs_r, xs_p, c_z, I, I, H, true,
                           nullptr, 0, nullptr, mask, ms_r, ms_k, out, xs_r, xs_p);
}

int pairattn_msa_row_fwd(const void* m, const void* z, const uint8_t* mask, const pairattn_params* p, void* out,
                         int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_msa(m, z, mask, p, out, S, I, c_m, c_z, H, d));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(S, I, c_m, c_m, H, p->dtype, true);
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, m, I * c_m, c_m, c_m, S, I, H, false, z,
                           c_z, nullptr, mask, I, 1, out, I * c_m, c_m);
}

int pairattn_tri_bias(const void* z, const pairattn_params* p, float* bias, int64_t I, int64_t c_z, int64_t H,
                      int32_t orientation, void* stream) {
  g_err[0] = '\0';
  if (p == nullptr) return fail(PAIRATTN_ERR_ARG, "params is NULL");
  if (p->dtype != PAIRATTN_F32 && p->dtype != PAIRATTN_BF16)
    return fail(PAIRATTN_ERR_ARG, "params->dtype %d is neither PAIRATTN_F32 nor PAIRATTN_BF16", p->dtype);
  if (!(p->ln_eps >= 0.0f) || !std::isfinite(p->ln_eps)) return fail(PAIRATTN_ERR_ARG, "params->ln_eps must be finite and >= 0");
  if (p->ln_gamma == nullptr || p->ln_beta == nullptr || p->w_b == nullptr)
    return fail(PAIRATTN_ERR_ARG, "ln_gamma, ln_beta and w_b are required");
  if (!aligned16(p->ln_gamma) || !aligned16(p->ln_beta) || !aligned16(p->w_b))
    return fail(PAIRATTN_ERR_ARG, "ln_gamma, ln_beta and w_b must be 16-byte aligned");
  if (z == nullptr || bias == nullptr) return fail(PAIRATTN_ERR_ARG, "z and bias must not be NULL");
  if (!aligned16(z) || !aligned16(bias)) return fail(PAIRATTN_ERR_ARG, "z and bias must be 16-byte aligned");
  if (orientation != PAIRATTN_START && orientation != PAIRATTN_END)
    return fail(PAIRATTN_ERR_ARG, "orientation %d is neither PAIRATTN_START nor PAIRATTN_END", orientation);
  PA_TRY(check_shape_common(I, c_z, H, 32, p->dtype));
  PA_TRY(check_rows_limit(I, p->dtype));
  if (overlaps(bias, (size_t)H * I * I * 4, z, (size_t)I * I * c_z * elt_bytes(p->dtype)))
    return fail(PAIRATTN_ERR_ARG, "bias overlaps z");
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const bool start = orientation == PAIRATTN_START;
  pa::ProjArgs pb{};
  pb.x = z;
  pb.xs_r = start ? I * c_z : c_z;
  pb.xs_p = start ? c_z : I * c_z;
  pb.gamma = p->ln_gamma;
  pb.beta = p->ln_beta;
  pb.eps = p->ln_eps;
  pb.wb = p->w_b;
  pb.bias = bias;
  pb.bias_swizzled = 0;
  pb.bias_scale = 1.0f;
  pb.c_in = (int)c_z;
  pb.hd = (int)(H * 32);
  pb.H = (int)H;
  pb.nrows = (int)I;
  pb.P = (int)I;
  pb.Pp = (int)pad32(I);
  hipStream_t s = static_cast<hipStream_t>(stream);
  tm_begin(s);
  const int st = p->dtype == PAIRATTN_BF16 ? hip_status(pa::launch_proj_bf16(pb, 2, num_cu, s), "pair-bias launch")
                                           : hip_status(pa::launch_proj_f32(pb, 2, s), "pair-bias launch");
  tm_mark(s, "pair_bias");
  return st;
}

int pairattn_tri_rows_fwd(const void* z_rows, const float* bias, const uint8_t* mask_rows, const pairattn_params* p,
                          void* out_rows, int64_t R, int64_t I, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_rows(z_rows, bias, mask_rows, p, out_rows, R, I, c_z, H, d));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(R, I, c_z, c_z, H, p->dtype, false);
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, z_rows, I * c_z, c_z, c_z, R, I, H, false,
                           nullptr, 0, bias, mask_rows, I, 1, out_rows, I * c_z, c_z);
}

}  // extern "C"
