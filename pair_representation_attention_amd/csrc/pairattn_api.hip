// C ABI of the pair-attention library: argument checks, workspace carving and
// kernel launches.  Every entry point is declared and documented in
// include/pairattn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
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

// Largest attention-row count the launches address (the projection grid
// and the bf16 attention grid count rows in 4-row groups below 65536).
constexpr int64_t kMaxRows = 65535LL * 4;
constexpr int64_t kMaxPositions = 1LL << 20;

// ---- workspace layout -----------------------------------------------------
constexpr size_t kWbImgBytes = 256 / 16 * 1024;   // pair-bias operand image for up to 256 channels

struct Layout {
  // bf16 path
  size_t wT = 0, woT = 0, q = 0, k = 0, v = 0, g = 0, bias = 0, bits = 0, wb_img = 0;
  // fp32 path: hi/lo planes of q, k, v and of the packed weights
  size_t q_lo = 0, k_lo = 0, v_lo = 0, w_hi = 0, w_lo = 0, cst = 0, wo_hi = 0, wo_lo = 0;
  size_t total = 0;
};

// nrows x P positions, c_in input channels, c_out output channels.
Layout make_layout(int64_t nrows, int64_t P, int64_t c_in, int64_t c_out, int64_t H, int32_t dtype) {
  Layout L;
  const int64_t hd = H * 32;
  const int64_t Pp = pad32(P);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const size_t plane = (size_t)nrows * H * Pp * 32 * 2;   // one fp16 q/k/v plane
  if (dtype == PAIRATTN_BF16) {
    L.wT = take((size_t)4 * hd * c_in * 2);
    L.cst = take((size_t)4 * hd * 4);
    L.wb_img = take(kWbImgBytes + 8 * 4);   // pair-bias operand (c <= 256) and its 8 constants
    L.woT = take((size_t)c_out * hd * 2);
    L.q = take(plane);
    L.k = take(plane);
    L.v = take(plane);
    L.g = take(plane);   // gate in the layout of q
    // the attention reads the bias as fp16 in operand order, Pp x Pp, log2
    // units; a caller-provided bias (row block) is converted into it as well
    L.bias = take((size_t)H * Pp * Pp * 2);
  } else {
    const int64_t nblk = 4 * hd / 32;        // q|k|v|g column blocks
    L.w_hi = take((size_t)nblk * c_in * 64);   // (c_in/16) K-steps x 64 lanes x 8 fp16 per block
    L.w_lo = take((size_t)nblk * c_in * 64);
    L.cst = take((size_t)nblk * 32 * 4);
    L.wo_hi = take((size_t)c_out * hd * 2);
    L.wo_lo = take((size_t)c_out * hd * 2);
    L.q = take(plane);
    L.q_lo = take(plane);
    L.k = take(plane);
    L.k_lo = take(plane);
    L.v = take(plane);
    L.v_lo = take(plane);
    L.g = take(2 * plane);                     // float, O^T tile images
    L.bias = take((size_t)H * Pp * Pp * 4);    // float, S^T tile images
  }
  L.bits = take(pa::mask_bits_bytes(nrows, Pp / 32));
  L.total = off;
  return L;
}

// Partial attention: R rows of Jq query pairs against Kn key pairs.  Queries
// get q (and, for the finish, the gate); keys get k and v.
struct PartialLayout {
  size_t w_hi = 0, w_lo = 0, cst = 0, wo_hi = 0, wo_lo = 0, q = 0, q_lo = 0, k = 0, k_lo = 0, v = 0, v_lo = 0, g = 0,
         bias = 0, bits = 0, total = 0;
  size_t wT = 0, woT = 0;   // bf16 path: packed fp16 weights
};
PartialLayout make_partial_layout(int64_t R, int64_t Jq, int64_t Kn, int64_t c, int64_t H, int32_t dtype) {
  PartialLayout L;
  if (dtype == PAIRATTN_BF16) {
    const int64_t hd = H * 32;
    const int64_t Ppq = pad32(Jq), Ppk = pad32(Kn);
    size_t off = 0;
    auto take = [&](size_t bytes) {
      const size_t at = off;
      off += align_up(bytes);
      return at;
    };
    L.wT = take((size_t)4 * hd * c * 2);
    L.cst = take((size_t)4 * hd * 4);
    L.woT = take((size_t)c * hd * 2);
    const size_t qplane = (size_t)R * H * Ppq * 32 * 2, kplane = (size_t)R * H * Ppk * 32 * 2;
    L.q = take(qplane);
    L.g = take(qplane);
    L.k = take(kplane);
    L.v = take(kplane);
    L.bias = take((size_t)H * Ppq * Ppk * 2);   // fp16 operand order, log2 units
    L.bits = take(pa::mask_bits_bytes(R, Ppk / 32));
    L.total = off;
    return L;
  }
  const int64_t hd = H * 32;
  const int64_t Ppq = pad32(Jq), Ppk = pad32(Kn);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const int64_t nblk = 4 * hd / 32;
  L.w_hi = take((size_t)nblk * c * 64);
  L.w_lo = take((size_t)nblk * c * 64);
  L.cst = take((size_t)nblk * 32 * 4);
  L.wo_hi = take((size_t)c * hd * 2);
  L.wo_lo = take((size_t)c * hd * 2);
  const size_t qplane = (size_t)R * H * Ppq * 32 * 2, kplane = (size_t)R * H * Ppk * 32 * 2;
  L.q = take(qplane);
  L.q_lo = take(qplane);
  L.k = take(kplane);
  L.k_lo = take(kplane);
  L.v = take(kplane);
  L.v_lo = take(kplane);
  L.g = take(2 * qplane);
  L.bias = take((size_t)H * Ppq * Ppk * 4);
  L.bits = take(pa::mask_bits_bytes(R, Ppk / 32));
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
  (void)dtype;
  if (nrows > kMaxRows)
    return fail(PAIRATTN_ERR_UNSUPPORTED, "%lld attention rows exceed the launch limit %lld", (long long)nrows,
                (long long)kMaxRows);
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
// A pool of events per thread, created when timing is enabled; every call
// records a boundary and one event after each kernel, with no host wait, so
// that many calls can be timed back to back and read at once.
constexpr int kPool = 1024;
struct Timing {
  bool enabled = false;
  bool created = false;
  hipEvent_t ev[kPool];
  const char* name[kPool];   // nullptr: the start of a call
  int n = 0;
};
thread_local Timing g_tm;

void tm_begin(hipStream_t s) {
  Timing& t = g_tm;
  if (!t.enabled || !t.created || t.n >= kPool) return;
  (void)hipEventRecord(t.ev[t.n], s);
  t.name[t.n] = nullptr;
  ++t.n;
}

void tm_mark(hipStream_t s, const char* stage) {
  Timing& t = g_tm;
  if (!t.enabled || t.n == 0 || t.n >= kPool) return;
  (void)hipEventRecord(t.ev[t.n], s);
  t.name[t.n] = stage;
  ++t.n;
}

}  // namespace

// ---- static scratch of the allocation-free entry point ---------------------
// One array per device: the code object's global segment, allocated when the
// library's kernels load on that device and held until the process ends.  In
// host code `scratch` names a host-side stand-in, never passed to a kernel:
// its device address is looked up once per device (with that device current)
// and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = PAIRATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(PAIRATTN_ERR_DEVICE, "no current HIP device");
  if (dev >= 64) return fail(PAIRATTN_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* at = nullptr;
    const hipError_t e = hipGetSymbolAddress(&at, HIP_SYMBOL(scratch));
    if (e != hipSuccess || at == nullptr)
      return fail(PAIRATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    if ((reinterpret_cast<uintptr_t>(at) & (kAlign - 1)) != 0)
      return fail(PAIRATTN_ERR_HIP, "scratch of device %d is not 256-byte aligned", dev);
    g_scratch_ptr[dev] = at;
  }
  *ptr = g_scratch_ptr[dev];
  return PAIRATTN_OK;
}
}  // namespace

// ============================================================================
extern "C" {

int pairattn_version(void) { return 10100; }

int pairattn_timing_enable(int enable) {
  Timing& t = g_tm;
  const int prev = t.enabled ? 1 : 0;
  if (enable && !t.created) {
    for (int i = 0; i < kPool; ++i)
      if (hipEventCreate(&t.ev[i]) != hipSuccess) {
        for (int j = 0; j < i; ++j) (void)hipEventDestroy(t.ev[j]);
        return -PAIRATTN_ERR_HIP;
      }
    t.created = true;
  }
  t.enabled = enable != 0;
  t.n = 0;
  return prev;
}

int pairattn_timing_read(float* ms, const char** names, int cap) {
  Timing& t = g_tm;
  if (!t.enabled || t.n < 2) {
    t.n = 0;
    return 0;
  }
  if (hipEventSynchronize(t.ev[t.n - 1]) != hipSuccess) return -PAIRATTN_ERR_HIP;
  int k = 0;
  for (int i = 1; i < t.n && k < cap; ++i) {
    if (t.name[i] == nullptr) continue;   // the start of the next call
    float v = 0.0f;
    if (hipEventElapsedTime(&v, t.ev[i - 1], t.ev[i]) != hipSuccess) return -PAIRATTN_ERR_HIP;
    if (ms != nullptr) ms[k] = v;
    if (names != nullptr) names[k] = t.name[i];
    ++k;
  }
  t.n = 0;
  return k;
}

int pairattn_calibrate_exp2(float* out, int64_t iters, void* stream) {
  g_err[0] = '\0';
  if (out == nullptr || !aligned16(out)) return fail(PAIRATTN_ERR_ARG, "out must be a 16-byte aligned device pointer");
  if (iters < 1 || iters > (1LL << 24)) return fail(PAIRATTN_ERR_ARG, "iters must be in [1, 2^24]");
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  return hip_status(pa::launch_calib_exp2(out, (int)iters, static_cast<hipStream_t>(stream)), "exp2 calibration launch");
}

int pairattn_debug_status(uint32_t* flags, int32_t* checking) {
  g_err[0] = '\0';
  unsigned int a = 0, b = 0;
#ifdef PA_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return fail(PAIRATTN_ERR_HIP, "device synchronisation failed");
  if (pa::debug_take_attn(&a) != hipSuccess || pa::debug_take_bf16(&b) != hipSuccess)
    return fail(PAIRATTN_ERR_HIP, "reading the debug flag words failed");
#endif
  if (flags != nullptr) *flags = a | b;
#ifdef PA_DEBUG
  if (checking != nullptr) *checking = 1;
#else
  if (checking != nullptr) *checking = 0;
#endif
  return PAIRATTN_OK;
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
  return make_layout(I, I, c_z, c_z, H, dtype).total;
}

size_t pairattn_msa_workspace_bytes(int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H, int64_t d,
                                    int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || S < 1 || I < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_m) || !supported_c(c_z) || I > kMaxPositions)
    return 0;
  return make_layout(S, I, c_m, c_m, H, dtype).total;
}

size_t pairattn_rows_workspace_bytes(int64_t R, int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || R < 1 || I < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_z) || I > kMaxPositions)
    return 0;
  return make_layout(R, I, c_z, c_z, H, dtype).total;
}

}  // extern "C"

namespace {
// Everything pairattn_validate_tri checks except the workspace.
int validate_tri_args(const void* z, const uint8_t* mask, const pairattn_params* p, const void* out, int64_t I,
                      int64_t c_z, int64_t H, int64_t d, int32_t orientation) {
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
  return PAIRATTN_OK;
}
}  // namespace

extern "C" {

int pairattn_validate_tri(const void* z, const uint8_t* mask, const pairattn_params* p, const void* out,
                          int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t orientation) {
  g_err[0] = '\0';
  PA_TRY(validate_tri_args(z, mask, p, out, I, c_z, H, d, orientation));
  const size_t zbytes = (size_t)I * I * c_z * elt_bytes(p->dtype);
  const size_t need = pairattn_tri_workspace_bytes(I, c_z, H, d, p->dtype);
  PA_TRY(check_workspace(p, need));
  if (overlaps(out, zbytes, p->workspace, p->workspace_bytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps the workspace");
  return PAIRATTN_OK;
}

size_t pairattn_tri_chunked_workspace_bytes(int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t dtype,
                                            int64_t block) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || I < 1 || block < 1 || d != 32 || !supported_h(H) ||
      !supported_c(c_z) || I > kMaxPositions)
    return 0;
  // one block's projections and keep bits; the bias region covers the whole I x I
  return make_layout(std::min(block, I), I, c_z, c_z, H, dtype).total;
}

int pairattn_validate_tri_chunked(const void* z, const uint8_t* mask, const pairattn_params* p, const void* out,
                                  int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t orientation, int64_t block) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, false));
  if (z == nullptr || out == nullptr) return fail(PAIRATTN_ERR_ARG, "z and out must not be NULL");
  if (!aligned16(z) || !aligned16(out)) return fail(PAIRATTN_ERR_ARG, "z and out must be 16-byte aligned");
  if (orientation != PAIRATTN_START && orientation != PAIRATTN_END)
    return fail(PAIRATTN_ERR_ARG, "orientation %d is neither PAIRATTN_START nor PAIRATTN_END", orientation);
  if (block < 1) return fail(PAIRATTN_ERR_ARG, "block must be >= 1 (got %lld)", (long long)block);
  PA_TRY(check_shape_common(I, c_z, H, d, p->dtype));
  PA_TRY(check_rows_limit(I, p->dtype));
  const size_t zbytes = (size_t)I * I * c_z * elt_bytes(p->dtype);
  if (overlaps(out, zbytes, z, zbytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps z");
  if (mask != nullptr && overlaps(out, zbytes, mask, (size_t)I * I)) return fail(PAIRATTN_ERR_ARG, "out overlaps mask");
  const size_t need = pairattn_tri_chunked_workspace_bytes(I, c_z, H, d, p->dtype, block);
  PA_TRY(check_workspace(p, need));
  if (overlaps(out, zbytes, p->workspace, p->workspace_bytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps the workspace");
  return PAIRATTN_OK;
}

size_t pairattn_tri_partial_workspace_bytes(int64_t R, int64_t Jq, int64_t Kn, int64_t c_z, int64_t H, int64_t d,
                                            int32_t dtype) {
  if ((dtype != PAIRATTN_F32 && dtype != PAIRATTN_BF16) || R < 1 || Jq < 1 || Kn < 1 || d != 32 ||
      !supported_h(H) || !supported_c(c_z) || Jq > kMaxPositions || Kn > kMaxPositions)
    return 0;
  return make_partial_layout(R, Jq, Kn, c_z, H, dtype).total;
}

int pairattn_validate_tri_partial(const void* q_pairs, const void* kv_pairs, const float* bias, const uint8_t* mask,
                                  const pairattn_params* p, const float* o, const float* lse, int64_t R, int64_t Jq,
                                  int64_t Kn, int64_t c_z, int64_t H, int64_t d) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, false));
  if (q_pairs == nullptr || kv_pairs == nullptr || bias == nullptr || o == nullptr || lse == nullptr)
    return fail(PAIRATTN_ERR_ARG, "q_pairs, kv_pairs, bias, o and lse must not be NULL");
  if (!aligned16(q_pairs) || !aligned16(kv_pairs) || !aligned16(bias) || !aligned16(o) || !aligned16(lse))
    return fail(PAIRATTN_ERR_ARG, "q_pairs, kv_pairs, bias, o and lse must be 16-byte aligned");
  if (R < 1 || Jq < 1 || Kn < 1) return fail(PAIRATTN_ERR_ARG, "R, Jq and Kn must be >= 1");
  PA_TRY(check_shape_common(std::max(Jq, Kn), c_z, H, d, p->dtype));
  PA_TRY(check_rows_limit(R, p->dtype));
  const size_t obytes = (size_t)R * Jq * H * d * 4, lbytes = (size_t)R * H * Jq * 4;
  const size_t qbytes = (size_t)R * Jq * c_z * elt_bytes(p->dtype), kbytes = (size_t)R * Kn * c_z * elt_bytes(p->dtype);
  if (overlaps(o, obytes, lse, lbytes)) return fail(PAIRATTN_ERR_ARG, "o overlaps lse");
  for (const void* in : {q_pairs, kv_pairs, (const void*)bias}) {
    const size_t nb = in == q_pairs ? qbytes : in == kv_pairs ? kbytes : (size_t)H * Jq * Kn * 4;
    if (overlaps(o, obytes, in, nb) || overlaps(lse, lbytes, in, nb))
      return fail(PAIRATTN_ERR_ARG, "o or lse overlaps an input");
  }
  const size_t need = pairattn_tri_partial_workspace_bytes(R, Jq, Kn, c_z, H, d, p->dtype);
  PA_TRY(check_workspace(p, need));
  if (overlaps(o, obytes, p->workspace, p->workspace_bytes) || overlaps(lse, lbytes, p->workspace, p->workspace_bytes))
    return fail(PAIRATTN_ERR_ARG, "o or lse overlaps the workspace");
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
struct RowAttn {
  // attended tensor: element (row, position, channel) at x[row*xs_r + pos*xs_p + ch]
  const void* x;
  int64_t xs_r, xs_p, c, nrows, P, H;
  // bias: computed in the projection (bias_in_proj), from a separate tensor
  // (zb != NULL), given (bias_given), or none of these: already in the
  // workspace in the attention's layout (chunked calls)
  bool bias_in_proj;
  const void* zb;
  int64_t zb_c;
  const float* bias_given;
  // mask and output addressing
  const uint8_t* mask;
  int64_t ms_r, ms_k;
  void* out;
  int64_t os_r, os_p;
  // part of a longer launch sequence whose caller records the timing marks
  bool nested = false;
};

static int run_row_attention_bf16(const pairattn_params* p, const Layout& L, hipStream_t s, int num_cu,
                                  const RowAttn& ra) {
  const int64_t hd = ra.H * 32;
  const int Pp = (int)pad32(ra.P);
  // the attention reads the workspace bias (fp16 operand order, log2 units)
  float* bias_ws = reinterpret_cast<float*>(ws_at(p, L.bias));

  pa::ProjArgs pj{};
  pj.x = ra.x;
  pj.xs_r = ra.xs_r;
  pj.xs_p = ra.xs_p;
  pj.gamma = p->ln_gamma;
  pj.beta = p->ln_beta;
  pj.eps = p->ln_eps;
  pj.wb = p->w_b;
  pj.q_ws = ws_at(p, L.q);
  pj.k_ws = ws_at(p, L.k);
  pj.v_ws = ws_at(p, L.v);
  pj.g_ws = ws_at(p, L.g);
  pj.bias = bias_ws;
  pj.bias_swizzled = 1;
  pj.bias_scale = 1.4426950408889634f;
  pj.c_in = (int)ra.c;
  pj.hd = (int)hd;
  pj.H = (int)ra.H;
  pj.nrows = (int)ra.nrows;
  pj.P = (int)ra.P;
  pj.Pp = Pp;

  auto mark = [&](const char* stage) {
    if (!ra.nested) tm_mark(s, stage);
  };
  if (!ra.nested) tm_begin(s);
  pa::PackArgs pk{};
  pk.wq = p->w_q;
  pk.wk = p->w_k;
  pk.wv = p->w_v;
  pk.wg = p->w_g;
  pk.wo = p->w_o;
  pk.gamma = p->ln_gamma;
  pk.beta = p->ln_beta;
  pk.b_g = p->b_g;
  pk.wT = ws_at(p, L.wT);
  pk.woT = ws_at(p, L.woT);
  pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
  pk.c_in = (int)ra.c;
  pk.hd = (int)hd;
  pk.c_out = (int)ra.c;
  // the same launch builds the pair-bias operand (bias from the projected
  // tensor or from the pair tensor) and the keep bits of the mask
  void* wb_img = ws_at(p, L.wb_img);
  float* wb_cst = reinterpret_cast<float*>(static_cast<char*>(wb_img) + kWbImgBytes);
  if (ra.bias_in_proj || ra.zb != nullptr) {
    pk.wb = p->w_b;
    pk.b_gamma = ra.zb != nullptr ? p->lnz_gamma : p->ln_gamma;
    pk.b_beta = ra.zb != nullptr ? p->lnz_beta : p->ln_beta;
    pk.b_c_in = (int)(ra.zb != nullptr ? ra.zb_c : ra.c);
    pk.H = (int)ra.H;
    pk.wb_img = wb_img;
    pk.wb_cst = wb_cst;
  }
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws_at(p, L.bits));
  if (ra.mask != nullptr) {
    pk.mask = ra.mask;
    pk.ms_r = ra.ms_r;
    pk.ms_k = ra.ms_k;
    pk.bits = bits;
    pk.nrows = (int)ra.nrows;
    pk.P = (int)ra.P;
    pk.nkb = Pp / 32;
  }
  PA_TRY(hip_status(pa::launch_pack_bf16(pk, s), "weight packing launch"));
  mark("pack");
  pj.wT = ws_at(p, L.wT);
  pj.cst = reinterpret_cast<const float*>(ws_at(p, L.cst));
  if (ra.bias_in_proj) {
    pj.wb_img = wb_img;
    pj.wb_cst = wb_cst;
  }
  PA_TRY(hip_status(pa::launch_proj_bf16(pj, ra.bias_in_proj ? 1 : 0, num_cu, s), "projection launch"));
  mark("projection");

  if (ra.zb != nullptr) {   // MSA: bias from the pair tensor with its own LayerNorm
    pa::ProjArgs pb{};
    pb.x = ra.zb;
    pb.xs_r = ra.P * ra.zb_c;
    pb.xs_p = ra.zb_c;
    pb.gamma = p->lnz_gamma;
    pb.beta = p->lnz_beta;
    pb.eps = p->ln_eps;
    pb.wb = p->w_b;
    pb.bias = bias_ws;
    pb.bias_swizzled = 1;
    pb.bias_scale = 1.4426950408889634f;
    pb.c_in = (int)ra.zb_c;
    pb.hd = (int)hd;
    pb.H = (int)ra.H;
    pb.nrows = (int)ra.P;
    pb.P = (int)ra.P;
    pb.Pp = Pp;
    pb.wb_img = wb_img;
    pb.wb_cst = wb_cst;
    PA_TRY(hip_status(pa::launch_proj_bf16(pb, 2, num_cu, s), "pair-bias launch"));
    mark("pair_bias");
  }
  if (ra.bias_given != nullptr) {   // row block: caller's bias -> attention layout
    PA_TRY(hip_status(pa::launch_bias_to_attn_layout(ra.bias_given, bias_ws, (int)ra.H, (int)ra.P, (int)ra.P, Pp, Pp, s),
                      "bias copy launch"));
    mark("bias_copy");
  }

  pa::AttnArgs at{};
  at.q_ws = pj.q_ws;
  at.k_ws = pj.k_ws;
  at.v_ws = pj.v_ws;
  at.g_ws = pj.g_ws;
  at.bias = bias_ws;
  // keep bits only when there is a mask (without one the kernel drops just
  // the keys past P, which it computes); built by the preparation launch
  at.mask_bits = ra.mask != nullptr ? bits : nullptr;
  at.mask_range = ra.mask != nullptr ? pa::mask_range_of(bits, ra.nrows, Pp / 32) : nullptr;
  at.woT = ws_at(p, L.woT);
  at.b_o = p->b_o;
  at.out = ra.out;
  at.os_r = ra.os_r;
  at.os_p = ra.os_p;
  at.H = (int)ra.H;
  at.c_out = (int)ra.c;
  at.nrows = (int)ra.nrows;
  at.P = (int)ra.P;
  at.Pp = Pp;
  PA_TRY(hip_status(pa::launch_attn_bf16(at, s), "attention launch"));
  mark("attention");
  return PAIRATTN_OK;
}

static int run_row_attention_f32(const pairattn_params* p, const Layout& L, hipStream_t s, int num_cu,
                                 const RowAttn& ra) {
  const int64_t hd = ra.H * 32;
  const int Pp = (int)pad32(ra.P);
  const int nqkvg = (int)(4 * hd / 32);
  float* bias_ws = reinterpret_cast<float*>(ws_at(p, L.bias));

  auto mark = [&](const char* stage) {
    if (!ra.nested) tm_mark(s, stage);
  };
  if (!ra.nested) tm_begin(s);
  pa::PackF32Args pk{};
  pk.wq = p->w_q;
  pk.wk = p->w_k;
  pk.wv = p->w_v;
  pk.wg = p->w_g;
  pk.gamma = p->ln_gamma;
  pk.beta = p->ln_beta;
  pk.b_g = p->b_g;
  pk.wo = p->w_o;
  pk.w_hi = ws_at(p, L.w_hi);
  pk.w_lo = ws_at(p, L.w_lo);
  pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
  pk.wo_hi = ws_at(p, L.wo_hi);
  pk.wo_lo = ws_at(p, L.wo_lo);
  pk.c_in = (int)ra.c;
  pk.hd = (int)hd;
  pk.H = (int)ra.H;
  pk.nqkvg = nqkvg;
  pk.c_out = (int)ra.c;
  PA_TRY(hip_status(pa::launch_pack_f32(pk, s), "weight packing launch"));
  mark("pack");

  pa::ProjF32Args pj{};
  pj.x = ra.x;
  pj.xs_r = ra.xs_r;
  pj.xs_p = ra.xs_p;
  pj.eps = p->ln_eps;
  pj.w_hi = pk.w_hi;
  pj.w_lo = pk.w_lo;
  pj.cst = pk.cst;
  pj.b_first = 0;
  pj.nqkvg = nqkvg;
  pj.with_bias = ra.bias_in_proj ? 1 : 0;
  pj.wb = p->w_b;
  pj.gamma = p->ln_gamma;
  pj.beta = p->ln_beta;
  pj.hd = (int)hd;
  pj.q_scale = 1.4426950408889634f / std::sqrt(32.0f);
  pj.q_hi = ws_at(p, L.q);
  pj.q_lo = ws_at(p, L.q_lo);
  pj.k_hi = ws_at(p, L.k);
  pj.k_lo = ws_at(p, L.k_lo);
  pj.v_hi = ws_at(p, L.v);
  pj.v_lo = ws_at(p, L.v_lo);
  pj.g_ws = reinterpret_cast<float*>(ws_at(p, L.g));
  pj.bias = bias_ws;
  pj.bias_natural = 0;
  pj.bias_scale = 1.4426950408889634f;
  pj.c_in = (int)ra.c;
  pj.H = (int)ra.H;
  pj.nrows = (int)ra.nrows;
  pj.P = (int)ra.P;
  pj.Pp = Pp;
  PA_TRY(hip_status(pa::launch_proj_f32(pj, num_cu, s), "projection launch"));
  mark("projection");

  if (ra.zb != nullptr) {
    pa::ProjF32Args pb{};
    pb.x = ra.zb;
    pb.xs_r = ra.P * ra.zb_c;
    pb.xs_p = ra.zb_c;
    pb.eps = p->ln_eps;
    pb.nqkvg = 0;
    pb.with_bias = 1;
    pb.wb = p->w_b;
    pb.gamma = p->lnz_gamma;
    pb.beta = p->lnz_beta;
    pb.hd = (int)hd;
    pb.bias = bias_ws;
    pb.bias_natural = 0;
    pb.bias_scale = 1.4426950408889634f;
    pb.c_in = (int)ra.zb_c;
    pb.H = (int)ra.H;
    pb.nrows = (int)ra.P;
    pb.P = (int)ra.P;
    pb.Pp = Pp;
    PA_TRY(hip_status(pa::launch_proj_f32(pb, num_cu, s), "pair-bias launch"));
    mark("pair_bias");
  }
  if (ra.bias_given != nullptr) {
    PA_TRY(hip_status(pa::launch_bias_to_f32_layout(ra.bias_given, bias_ws, (int)ra.H, (int)ra.P, (int)ra.P, Pp,
                                                    Pp, s),
                      "bias copy launch"));
    mark("bias_copy");
  }

  uint32_t* bits = reinterpret_cast<uint32_t*>(ws_at(p, L.bits));
  if (ra.mask != nullptr) {
    PA_TRY(hip_status(pa::launch_mask_bits(ra.mask, ra.ms_r, ra.ms_k, bits, (int)ra.nrows, (int)ra.P, Pp / 32, s),
                      "mask bits launch"));
    mark("mask_bits");
  }
  pa::AttnF32Args at{};
  at.q_hi = pj.q_hi;
  at.q_lo = pj.q_lo;
  at.k_hi = pj.k_hi;
  at.k_lo = pj.k_lo;
  at.v_hi = pj.v_hi;
  at.v_lo = pj.v_lo;
  at.g_ws = pj.g_ws;
  at.bias = bias_ws;
  at.mask_bits = ra.mask != nullptr ? bits : nullptr;
  at.wo_hi = pk.wo_hi;
  at.wo_lo = pk.wo_lo;
  at.b_o = p->b_o;
  at.out = ra.out;
  at.os_r = ra.os_r;
  at.os_p = ra.os_p;
  at.H = (int)ra.H;
  at.c_out = (int)ra.c;
  at.nrows = (int)ra.nrows;
  at.P = (int)ra.P;
  at.Pp = Pp;
  at.Pk = (int)ra.P;
  at.Ppk = Pp;
  at.mode = 0;
  PA_TRY(hip_status(pa::launch_attn_f32(at, s), "attention launch"));
  mark("attention");
  return PAIRATTN_OK;
}

static int run_row_attention(const pairattn_params* p, const Layout& L, hipStream_t s, int num_cu, const RowAttn& ra) {
  return p->dtype == PAIRATTN_BF16 ? run_row_attention_bf16(p, L, s, num_cu, ra)
                                   : run_row_attention_f32(p, L, s, num_cu, ra);
}

int pairattn_tri_fwd(const void* z, const uint8_t* mask, const pairattn_params* p, void* out, int64_t I, int64_t c_z,
                     int64_t H, int64_t d, int32_t orientation, void* stream) {
  PA_TRY(pairattn_validate_tri(z, mask, p, out, I, c_z, H, d, orientation));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(I, I, c_z, c_z, H, p->dtype);
  const bool start = orientation == PAIRATTN_START;
  // START: row i, position j -> pair (i, j); END: row j, position i -> pair (i, j)
  const int64_t xs_r = start ? I * c_z : c_z;
  const int64_t xs_p = start ? c_z : I * c_z;
  const int64_t ms_r = start ? I : 1;
  const int64_t ms_k = start ? 1 : I;
  const RowAttn ra{z, xs_r, xs_p, c_z, I, I, H, true, nullptr, 0, nullptr, mask, ms_r, ms_k, out, xs_r, xs_p};
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, ra);
}

int pairattn_tri_fwd_noalloc(const void* z, const uint8_t* mask, const pairattn_params* p, void* out, int64_t I,
                             int64_t c_z, int64_t H, int64_t d, int32_t orientation, void* stream) {
  g_err[0] = '\0';
  // host checks first: arguments, then the size against the static scratch
  PA_TRY(validate_tri_args(z, mask, p, out, I, c_z, H, d, orientation));
  const size_t need = pairattn_tri_workspace_bytes(I, c_z, H, d, p->dtype);
  if (need > kScratchBytes)
    return fail(PAIRATTN_ERR_UNSUPPORTED,
                "I=%lld needs %zu bytes of scratch; the allocation-free call has %zu (pass a workspace to "
                "pairattn_tri_fwd instead)",
                (long long)I, need, kScratchBytes);
  void* ws = nullptr;
  PA_TRY(scratch_for_current_device(&ws));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  pairattn_params q = *p;
  q.workspace = ws;
  q.workspace_bytes = kScratchBytes;
  const Layout L = make_layout(I, I, c_z, c_z, H, q.dtype);
  const bool start = orientation == PAIRATTN_START;
  const int64_t xs_r = start ? I * c_z : c_z;
  const int64_t xs_p = start ? c_z : I * c_z;
  const int64_t ms_r = start ? I : 1;
  const int64_t ms_k = start ? 1 : I;
  RowAttn ra{z, xs_r, xs_p, c_z, I, I, H, true, nullptr, 0, nullptr, mask, ms_r, ms_k, out, xs_r, xs_p};
  ra.nested = true;
  return run_row_attention(&q, L, static_cast<hipStream_t>(stream), num_cu, ra);
}

int pairattn_msa_row_fwd(const void* m, const void* z, const uint8_t* mask, const pairattn_params* p, void* out,
                         int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_msa(m, z, mask, p, out, S, I, c_m, c_z, H, d));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(S, I, c_m, c_m, H, p->dtype);
  const RowAttn ra{m, I * c_m, c_m, c_m, S, I, H, false, z, c_z, nullptr, mask, I, 1, out, I * c_m, c_m};
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, ra);
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
  const int64_t xs_r = start ? I * c_z : c_z;
  const int64_t xs_p = start ? c_z : I * c_z;
  hipStream_t s = static_cast<hipStream_t>(stream);
  tm_begin(s);
  int st;
  if (p->dtype == PAIRATTN_BF16) {
    pa::ProjArgs pb{};
    pb.x = z;
    pb.xs_r = xs_r;
    pb.xs_p = xs_p;
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
    st = hip_status(pa::launch_proj_bf16(pb, 2, num_cu, s), "pair-bias launch");
  } else {
    pa::ProjF32Args pb{};
    pb.x = z;
    pb.xs_r = xs_r;
    pb.xs_p = xs_p;
    pb.eps = p->ln_eps;
    pb.nqkvg = 0;
    pb.with_bias = 1;
    pb.wb = p->w_b;
    pb.gamma = p->ln_gamma;
    pb.beta = p->ln_beta;
    pb.hd = (int)(H * 32);
    pb.bias = bias;
    pb.bias_natural = 1;
    pb.bias_scale = 1.0f;
    pb.c_in = (int)c_z;
    pb.H = (int)H;
    pb.nrows = (int)I;
    pb.P = (int)I;
    pb.Pp = (int)pad32(I);
    st = hip_status(pa::launch_proj_f32(pb, num_cu, s), "pair-bias launch");
  }
  tm_mark(s, "pair_bias");
  return st;
}

int pairattn_tri_chunked_fwd(const void* z, const uint8_t* mask, const pairattn_params* p, void* out, int64_t I,
                             int64_t c_z, int64_t H, int64_t d, int32_t orientation, int64_t block, void* stream) {
  PA_TRY(pairattn_validate_tri_chunked(z, mask, p, out, I, c_z, H, d, orientation, block));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  block = std::min(block, I);
  const Layout L = make_layout(block, I, c_z, c_z, H, p->dtype);
  const bool start = orientation == PAIRATTN_START;
  const bool bf = p->dtype == PAIRATTN_BF16;
  const int Pp = (int)pad32(I);
  const int64_t xs_r = start ? I * c_z : c_z;   // START: row i, position j; END: column j, position i
  const int64_t xs_p = start ? c_z : I * c_z;
  const int64_t ms_r = start ? I : 1;
  const int64_t ms_k = start ? 1 : I;
  hipStream_t s = static_cast<hipStream_t>(stream);
  tm_begin(s);

  // the pair bias of the whole Z, once, into the workspace in the attention's layout
  if (bf) {
    pa::ProjArgs pb{};
    pb.x = z;
    pb.xs_r = xs_r;
    pb.xs_p = xs_p;
    pb.gamma = p->ln_gamma;
    pb.beta = p->ln_beta;
    pb.eps = p->ln_eps;
    pb.wb = p->w_b;
    pb.bias = reinterpret_cast<float*>(ws_at(p, L.bias));
    pb.bias_swizzled = 1;
    pb.bias_scale = 1.4426950408889634f;
    pb.c_in = (int)c_z;
    pb.hd = (int)(H * 32);
    pb.H = (int)H;
    pb.nrows = (int)I;
    pb.P = (int)I;
    pb.Pp = Pp;
    PA_TRY(hip_status(pa::launch_proj_bf16(pb, 2, num_cu, s), "pair-bias launch"));
  } else {
    pa::ProjF32Args pb{};
    pb.x = z;
    pb.xs_r = xs_r;
    pb.xs_p = xs_p;
    pb.eps = p->ln_eps;
    pb.nqkvg = 0;
    pb.with_bias = 1;
    pb.wb = p->w_b;
    pb.gamma = p->ln_gamma;
    pb.beta = p->ln_beta;
    pb.hd = (int)(H * 32);
    pb.bias = reinterpret_cast<float*>(ws_at(p, L.bias));
    pb.bias_natural = 0;
    pb.bias_scale = 1.4426950408889634f;
    pb.c_in = (int)c_z;
    pb.H = (int)H;
    pb.nrows = (int)I;
    pb.P = (int)I;
    pb.Pp = Pp;
    PA_TRY(hip_status(pa::launch_proj_f32(pb, num_cu, s), "pair-bias launch"));
  }
  tm_mark(s, "pair_bias");

  // then blocks of rows (START) or columns (END): projections and attention
  // of `block` rows at a time against the bias above
  const size_t eb = elt_bytes(p->dtype);
  for (int64_t b0 = 0; b0 < I; b0 += block) {
    const int64_t n = std::min(block, I - b0);
    const int64_t xoff = start ? b0 * I * c_z : b0 * c_z;   // elements
    RowAttn ra{static_cast<const char*>(z) + xoff * eb, xs_r, xs_p, c_z, n, I, H, false, nullptr, 0, nullptr,
               mask != nullptr ? mask + (start ? b0 * I : b0) : nullptr, ms_r, ms_k,
               static_cast<char*>(out) + xoff * eb, xs_r, xs_p};
    ra.nested = true;
    PA_TRY(run_row_attention(p, L, s, num_cu, ra));
  }
  tm_mark(s, "blocks");
  return PAIRATTN_OK;
}

int pairattn_tri_partial_fwd(const void* q_pairs, const void* kv_pairs, const float* bias, const uint8_t* mask,
                             const pairattn_params* p, float* o, float* lse, int32_t accumulate, int64_t R, int64_t Jq,
                             int64_t Kn, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_tri_partial(q_pairs, kv_pairs, bias, mask, p, o, lse, R, Jq, Kn, c_z, H, d));
  if (accumulate & ~(PAIRATTN_PARTIAL_MERGE | PAIRATTN_PARTIAL_Q_READY))
    return fail(PAIRATTN_ERR_ARG, "accumulate %d has bits other than PAIRATTN_PARTIAL_MERGE and PAIRATTN_PARTIAL_Q_READY",
                accumulate);
  const bool merge = (accumulate & PAIRATTN_PARTIAL_MERGE) != 0;
  const bool q_ready = (accumulate & PAIRATTN_PARTIAL_Q_READY) != 0;
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const PartialLayout L = make_partial_layout(R, Jq, Kn, c_z, H, p->dtype);
  const int64_t hd = H * 32;
  const int Ppq = (int)pad32(Jq), Ppk = (int)pad32(Kn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  tm_begin(s);
  if (p->dtype == PAIRATTN_BF16) {
    pa::PackArgs pk{};
    pk.wq = p->w_q;
    pk.wk = p->w_k;
    pk.wv = p->w_v;
    pk.wg = p->w_g;
    pk.wo = p->w_o;
    pk.gamma = p->ln_gamma;
    pk.beta = p->ln_beta;
    pk.b_g = p->b_g;
    pk.wT = ws_at(p, L.wT);
    pk.woT = ws_at(p, L.woT);
    pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
    pk.c_in = (int)c_z;
    pk.hd = (int)hd;
    pk.c_out = (int)c_z;
    if (!q_ready) {
      PA_TRY(hip_status(pa::launch_pack_bf16(pk, s), "weight packing launch"));
      tm_mark(s, "pack");
    }
    // q of the query pairs (unless ready), k and v of the key pairs (the
    // other planes NULL)
    pa::ProjArgs pj{};
    pj.x = q_pairs;
    pj.xs_r = Jq * c_z;
    pj.xs_p = c_z;
    pj.gamma = p->ln_gamma;
    pj.beta = p->ln_beta;
    pj.eps = p->ln_eps;
    pj.wT = ws_at(p, L.wT);
    pj.cst = reinterpret_cast<const float*>(ws_at(p, L.cst));
    pj.q_ws = q_ready ? nullptr : ws_at(p, L.q);
    pj.c_in = (int)c_z;
    pj.hd = (int)hd;
    pj.H = (int)H;
    pj.nrows = (int)R;
    pj.P = (int)Jq;
    pj.Pp = Ppq;
    // the device's own shard (the query pairs' buffer): q, k and v in one pass
    const bool own = kv_pairs == q_pairs && Kn == Jq;
    if (own) {
      pj.k_ws = ws_at(p, L.k);
      pj.v_ws = ws_at(p, L.v);
    }
    if (own || !q_ready) PA_TRY(hip_status(pa::launch_proj_bf16(pj, 0, num_cu, s), "query projection launch"));
    if (!own) {
      pj.x = kv_pairs;
      pj.xs_r = Kn * c_z;
      pj.q_ws = nullptr;
      pj.k_ws = ws_at(p, L.k);
      pj.v_ws = ws_at(p, L.v);
      pj.P = (int)Kn;
      pj.Pp = Ppk;
      PA_TRY(hip_status(pa::launch_proj_bf16(pj, 0, num_cu, s), "key projection launch"));
    }
    tm_mark(s, "projection");
    void* bias_ws = ws_at(p, L.bias);
    PA_TRY(hip_status(pa::launch_bias_to_attn_layout(bias, bias_ws, (int)H, (int)Jq, (int)Kn, Ppq, Ppk, s),
                      "bias copy launch"));
    tm_mark(s, "bias_copy");
    uint32_t* bits = reinterpret_cast<uint32_t*>(ws_at(p, L.bits));
    if (mask != nullptr) {
      PA_TRY(hip_status(pa::launch_mask_bits(mask, Kn, 1, bits, (int)R, (int)Kn, Ppk / 32, s), "mask bits launch"));
      tm_mark(s, "mask_bits");
    }
    pa::AttnArgs at{};
    at.q_ws = ws_at(p, L.q);
    at.k_ws = ws_at(p, L.k);
    at.v_ws = ws_at(p, L.v);
    at.bias = bias_ws;
    at.mask_bits = mask != nullptr ? bits : nullptr;
    at.mask_range = mask != nullptr ? pa::mask_range_of(bits, R, Ppk / 32) : nullptr;
    at.H = (int)H;
    at.c_out = (int)c_z;
    at.nrows = (int)R;
    at.P = (int)Jq;
    at.Pp = Ppq;
    at.mode = merge ? 2 : 1;
    at.Pk = (int)Kn;
    at.Ppk = Ppk;
    at.o_part = o;
    at.lse_part = lse;
    PA_TRY(hip_status(pa::launch_attn_bf16(at, s), "attention launch"));
    tm_mark(s, "attention");
    return PAIRATTN_OK;
  }
  pa::PackF32Args pk{};
  pk.wq = p->w_q;
  pk.wk = p->w_k;
  pk.wv = p->w_v;
  pk.wg = p->w_g;
  pk.gamma = p->ln_gamma;
  pk.beta = p->ln_beta;
  pk.b_g = p->b_g;
  pk.w_hi = ws_at(p, L.w_hi);
  pk.w_lo = ws_at(p, L.w_lo);
  pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
  pk.c_in = (int)c_z;
  pk.hd = (int)hd;
  pk.H = (int)H;
  pk.nqkvg = (int)(4 * hd / 32);
  if (!q_ready) {
    PA_TRY(hip_status(pa::launch_pack_f32(pk, s), "weight packing launch"));
    tm_mark(s, "pack");
  }
  // q of the query pairs (blocks [0, hd/32); unless ready), k and v of the
  // key pairs (blocks [hd/32, 3*hd/32))
  pa::ProjF32Args pj{};
  pj.eps = p->ln_eps;
  pj.w_hi = pk.w_hi;
  pj.w_lo = pk.w_lo;
  pj.cst = pk.cst;
  pj.hd = (int)hd;
  pj.q_scale = 1.4426950408889634f / std::sqrt(32.0f);
  pj.q_hi = ws_at(p, L.q);
  pj.q_lo = ws_at(p, L.q_lo);
  pj.k_hi = ws_at(p, L.k);
  pj.k_lo = ws_at(p, L.k_lo);
  pj.v_hi = ws_at(p, L.v);
  pj.v_lo = ws_at(p, L.v_lo);
  pj.g_ws = reinterpret_cast<float*>(ws_at(p, L.g));
  pj.c_in = (int)c_z;
  pj.H = (int)H;
  pj.nrows = (int)R;
  pj.with_bias = 0;
  pj.x = q_pairs;
  pj.xs_r = Jq * c_z;
  pj.xs_p = c_z;
  pj.b_first = 0;
  // the device's own shard (the query pairs' buffer): q, k and v in one pass
  const bool own = kv_pairs == q_pairs && Kn == Jq;
  pj.b_first = q_ready ? (int)(hd / 32) : 0;
  pj.nqkvg = (int)((own ? 3 : 1) * hd / 32) - pj.b_first;
  pj.P = (int)Jq;
  pj.Pp = Ppq;
  if (pj.nqkvg > 0) PA_TRY(hip_status(pa::launch_proj_f32(pj, num_cu, s), "query projection launch"));
  if (!own) {
    pj.x = kv_pairs;
    pj.xs_r = Kn * c_z;
    pj.b_first = (int)(hd / 32);
    pj.nqkvg = (int)(2 * hd / 32);
    pj.P = (int)Kn;
    pj.Pp = Ppk;
    PA_TRY(hip_status(pa::launch_proj_f32(pj, num_cu, s), "key projection launch"));
  }
  tm_mark(s, "projection");
  float* bias_ws = reinterpret_cast<float*>(ws_at(p, L.bias));
  PA_TRY(hip_status(pa::launch_bias_to_f32_layout(bias, bias_ws, (int)H, (int)Jq, (int)Kn, Ppq, Ppk, s),
                    "bias copy launch"));
  tm_mark(s, "bias_copy");
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws_at(p, L.bits));
  if (mask != nullptr) {
    PA_TRY(hip_status(pa::launch_mask_bits(mask, Kn, 1, bits, (int)R, (int)Kn, Ppk / 32, s), "mask bits launch"));
    tm_mark(s, "mask_bits");
  }
  pa::AttnF32Args at{};
  at.q_hi = pj.q_hi;
  at.q_lo = pj.q_lo;
  at.k_hi = pj.k_hi;
  at.k_lo = pj.k_lo;
  at.v_hi = pj.v_hi;
  at.v_lo = pj.v_lo;
  at.bias = bias_ws;
  at.mask_bits = mask != nullptr ? bits : nullptr;
  at.H = (int)H;
  at.c_out = (int)c_z;
  at.nrows = (int)R;
  at.P = (int)Jq;
  at.Pp = Ppq;
  at.Pk = (int)Kn;
  at.Ppk = Ppk;
  at.mode = merge ? 2 : 1;
  at.o_part = o;
  at.lse_part = lse;
  PA_TRY(hip_status(pa::launch_attn_f32(at, s), "attention launch"));
  tm_mark(s, "attention");
  return PAIRATTN_OK;
}

size_t pairattn_tri_partial_finish_workspace_bytes(int64_t R, int64_t Jq, int64_t c_z, int64_t H, int64_t d,
                                                   int32_t dtype) {
  return pairattn_tri_partial_workspace_bytes(R, Jq, 1, c_z, H, d, dtype);
}

int pairattn_validate_tri_partial_finish(const void* q_pairs, const float* o, const pairattn_params* p,
                                         const void* out, int64_t R, int64_t Jq, int64_t c_z, int64_t H, int64_t d) {
  g_err[0] = '\0';
  PA_TRY(check_params(p, true, false));
  if (q_pairs == nullptr || o == nullptr || out == nullptr)
    return fail(PAIRATTN_ERR_ARG, "q_pairs, o and out must not be NULL");
  if (!aligned16(q_pairs) || !aligned16(o) || !aligned16(out))
    return fail(PAIRATTN_ERR_ARG, "q_pairs, o and out must be 16-byte aligned");
  if (R < 1 || Jq < 1) return fail(PAIRATTN_ERR_ARG, "R and Jq must be >= 1");
  PA_TRY(check_shape_common(Jq, c_z, H, d, p->dtype));
  PA_TRY(check_rows_limit(R, p->dtype));
  const size_t obytes = (size_t)R * Jq * c_z * elt_bytes(p->dtype);
  if (overlaps(out, obytes, q_pairs, obytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps q_pairs");
  if (overlaps(out, obytes, o, (size_t)R * Jq * H * d * 4)) return fail(PAIRATTN_ERR_ARG, "out overlaps o");
  PA_TRY(check_workspace(p, pairattn_tri_partial_finish_workspace_bytes(R, Jq, c_z, H, d, p->dtype)));
  if (overlaps(out, obytes, p->workspace, p->workspace_bytes)) return fail(PAIRATTN_ERR_ARG, "out overlaps the workspace");
  return PAIRATTN_OK;
}

int pairattn_tri_partial_finish(const void* q_pairs, const float* o, const pairattn_params* p, void* out, int64_t R,
                                int64_t Jq, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_tri_partial_finish(q_pairs, o, p, out, R, Jq, c_z, H, d));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const PartialLayout L = make_partial_layout(R, Jq, 1, c_z, H, p->dtype);
  const int64_t hd = H * 32;
  const int Ppq = (int)pad32(Jq);
  hipStream_t s = static_cast<hipStream_t>(stream);
  tm_begin(s);
  if (p->dtype == PAIRATTN_BF16) {
    pa::PackArgs pk{};
    pk.wq = p->w_q;
    pk.wk = p->w_k;
    pk.wv = p->w_v;
    pk.wg = p->w_g;
    pk.wo = p->w_o;
    pk.gamma = p->ln_gamma;
    pk.beta = p->ln_beta;
    pk.b_g = p->b_g;
    pk.wT = ws_at(p, L.wT);
    pk.woT = ws_at(p, L.woT);
    pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
    pk.c_in = (int)c_z;
    pk.hd = (int)hd;
    pk.c_out = (int)c_z;
    PA_TRY(hip_status(pa::launch_pack_bf16(pk, s), "weight packing launch"));
    tm_mark(s, "pack");
    if (pa::finish_fused_bf16_supported((int)c_z, (int)H)) {   // the gate computed where it is used
      pa::FinishFusedArgs fa{};
      fa.x = q_pairs;
      fa.xs_r = Jq * c_z;
      fa.xs_p = c_z;
      fa.eps = p->ln_eps;
      fa.wimg = ws_at(p, L.wT);
      fa.cst = reinterpret_cast<const float*>(ws_at(p, L.cst));
      fa.o_part = o;
      fa.woT = ws_at(p, L.woT);
      fa.b_o = p->b_o;
      fa.out = out;
      fa.os_r = Jq * c_z;
      fa.os_p = c_z;
      fa.c = (int)c_z;
      fa.H = (int)H;
      fa.nrows = (int)R;
      fa.P = (int)Jq;
      fa.Pp = Ppq;
      PA_TRY(hip_status(pa::launch_finish_fused_bf16(fa, num_cu, s), "finish launch"));
      tm_mark(s, "finish");
      return PAIRATTN_OK;
    }
    pa::ProjArgs pj{};   // the gate of the query pairs only
    pj.x = q_pairs;
    pj.xs_r = Jq * c_z;
    pj.xs_p = c_z;
    pj.gamma = p->ln_gamma;
    pj.beta = p->ln_beta;
    pj.eps = p->ln_eps;
    pj.wT = ws_at(p, L.wT);
    pj.cst = reinterpret_cast<const float*>(ws_at(p, L.cst));
    pj.g_ws = ws_at(p, L.g);
    pj.c_in = (int)c_z;
    pj.hd = (int)hd;
    pj.H = (int)H;
    pj.nrows = (int)R;
    pj.P = (int)Jq;
    pj.Pp = Ppq;
    PA_TRY(hip_status(pa::launch_proj_bf16(pj, 0, num_cu, s), "gate projection launch"));
    tm_mark(s, "projection");
    pa::AttnArgs at{};
    at.g_ws = pj.g_ws;
    at.woT = ws_at(p, L.woT);
    at.b_o = p->b_o;
    at.out = out;
    at.os_r = Jq * c_z;
    at.os_p = c_z;
    at.H = (int)H;
    at.c_out = (int)c_z;
    at.nrows = (int)R;
    at.P = (int)Jq;
    at.Pp = Ppq;
    at.o_part = const_cast<float*>(o);
    PA_TRY(hip_status(pa::launch_finish_bf16(at, s), "finish launch"));
    tm_mark(s, "finish");
    return PAIRATTN_OK;
  }
  pa::PackF32Args pk{};
  pk.wq = p->w_q;
  pk.wk = p->w_k;
  pk.wv = p->w_v;
  pk.wg = p->w_g;
  pk.gamma = p->ln_gamma;
  pk.beta = p->ln_beta;
  pk.b_g = p->b_g;
  pk.wo = p->w_o;
  pk.w_hi = ws_at(p, L.w_hi);
  pk.w_lo = ws_at(p, L.w_lo);
  pk.cst = reinterpret_cast<float*>(ws_at(p, L.cst));
  pk.wo_hi = ws_at(p, L.wo_hi);
  pk.wo_lo = ws_at(p, L.wo_lo);
  pk.c_in = (int)c_z;
  pk.hd = (int)hd;
  pk.H = (int)H;
  pk.nqkvg = (int)(4 * hd / 32);
  pk.c_out = (int)c_z;
  PA_TRY(hip_status(pa::launch_pack_f32(pk, s), "weight packing launch"));
  tm_mark(s, "pack");
  pa::ProjF32Args pj{};   // the gate of the query pairs: blocks [3*hd/32, 4*hd/32)
  pj.x = q_pairs;
  pj.xs_r = Jq * c_z;
  pj.xs_p = c_z;
  pj.eps = p->ln_eps;
  pj.w_hi = pk.w_hi;
  pj.w_lo = pk.w_lo;
  pj.cst = pk.cst;
  pj.b_first = (int)(3 * hd / 32);
  pj.nqkvg = (int)(hd / 32);
  pj.hd = (int)hd;
  pj.g_ws = reinterpret_cast<float*>(ws_at(p, L.g));
  pj.c_in = (int)c_z;
  pj.H = (int)H;
  pj.nrows = (int)R;
  pj.P = (int)Jq;
  pj.Pp = Ppq;
  PA_TRY(hip_status(pa::launch_proj_f32(pj, num_cu, s), "gate projection launch"));
  tm_mark(s, "projection");
  pa::AttnF32Args at{};
  at.g_ws = pj.g_ws;
  at.wo_hi = pk.wo_hi;
  at.wo_lo = pk.wo_lo;
  at.b_o = p->b_o;
  at.out = out;
  at.os_r = Jq * c_z;
  at.os_p = c_z;
  at.H = (int)H;
  at.c_out = (int)c_z;
  at.nrows = (int)R;
  at.P = (int)Jq;
  at.Pp = Ppq;
  at.o_part = const_cast<float*>(o);
  PA_TRY(hip_status(pa::launch_finish_f32(at, s), "finish launch"));
  tm_mark(s, "finish");
  return PAIRATTN_OK;
}

int pairattn_tri_rows_fwd(const void* z_rows, const float* bias, const uint8_t* mask_rows, const pairattn_params* p,
                          void* out_rows, int64_t R, int64_t I, int64_t c_z, int64_t H, int64_t d, void* stream) {
  PA_TRY(pairattn_validate_rows(z_rows, bias, mask_rows, p, out_rows, R, I, c_z, H, d));
  int num_cu = 0;
  PA_TRY(check_device(&num_cu));
  const Layout L = make_layout(R, I, c_z, c_z, H, p->dtype);
  const RowAttn ra{z_rows, I * c_z, c_z, c_z, R, I, H, false, nullptr, 0, bias, mask_rows, I, 1, out_rows, I * c_z, c_z};
  return run_row_attention(p, L, static_cast<hipStream_t>(stream), num_cu, ra);
}

}  // extern "C"
