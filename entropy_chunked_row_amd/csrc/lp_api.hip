// C ABI of liblp.so (declared in include/lp.h): argument validation, chunk /
// tile scheduling and stream-ordered launches.  Every check runs on the host
// before anything is launched; a rejected call touches no output.
#include <initializer_list>
#include <mutex>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/lp.h"
#include "lp_internal.hpp"

namespace {

thread_local char g_err[512] = {0};

lp_status fail(lp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lp_status ok() {
  g_err[0] = 0;
  return LP_OK;
}

lp_status hip_fail(hipError_t e, const char* where) {
  return fail(LP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// The launchers read hipGetLastError() after each launch; an error left
// pending on this thread by an earlier, unrelated runtime call (the caller's
// or another library's) would be reported as ours.  Clear it first.
void clear_pending_hip_error() { (void)hipGetLastError(); }

constexpr double kLog2eD = 1.44269504088896340736;
constexpr int64_t kMaxV = (int64_t(1) << 30);

bool temperature_applies(float t) { return t > 0.f && t != 1.f; }

// c = log2(e) / tau_effective, rounded once.
float exp2_scale(float temperature) {
  const double tau = temperature_applies(temperature) ? static_cast<double>(temperature) : 1.0;
  return static_cast<float>(kLog2eD / tau);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Every fp32 array argument (NULL allowed) must be 4-byte aligned.
bool f32_aligned(std::initializer_list<const float*> ps) {
  for (const float* p : ps)
    if (p && !aligned(p, 4)) return false;
  return true;
}

size_t dtype_bytes(int d) { return d == LP_FP32 ? 4 : 2; }

}  // namespace

// Scratch of lp_lm_head_logprobs_entropy_noalloc: one copy per GPU the
// library runs on, held until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address of each GPU's copy comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[LP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
hipError_t scratch_of_current_device(int* device, void** out) {
  hipError_t e = hipGetDevice(device);
  if (e != hipSuccess) return e;
  if (*device < 0 || *device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[*device]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[*device] = p;
  }
  *out = g_scratch_ptr[*device];
  return hipSuccess;
}

}  // namespace

extern "C" {

int lp_version(void) { return 100; }

const char* lp_status_string(int status) {
  switch (status) {
    case LP_OK: return "LP_OK";
    case LP_ERR_INVALID_ARGUMENT: return "LP_ERR_INVALID_ARGUMENT";
    case LP_ERR_UNSUPPORTED: return "LP_ERR_UNSUPPORTED";
    case LP_ERR_WORKSPACE_TOO_SMALL: return "LP_ERR_WORKSPACE_TOO_SMALL";
    case LP_ERR_HIP: return "LP_ERR_HIP";
    default: return "unknown status";
  }
}

const char* lp_last_error(void) { return g_err; }

static lp_status logprobs_entropy_impl(const void* logits, lp_dtype dtype, int64_t T, int64_t V, int64_t ld,
                                       const int64_t* targets, int64_t K, const uint8_t* mask, float temperature,
                                       int64_t chunk_rows, float* logprob, float* entropy, void* stream) {
  if (K < 1 || K > lp::kMaxTargets)
    return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: K must be in 1..%d", lp::kMaxTargets);
  if (dtype != LP_BF16 && dtype != LP_FP16 && dtype != LP_FP32)
    return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: unknown dtype %d", static_cast<int>(dtype));
  if (T < 0) return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: T < 0");
  if (V <= 0 || V > kMaxV) return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: V out of range (1..2^30)");
  if (ld < V) return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: ld < V");
  if (!isfinite(temperature)) return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: temperature not finite");
  if (T == 0) return ok();
  if (!logits || !targets || !logprob)
    return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: logits, targets and logprob are required");
  if (!aligned(logits, dtype_bytes(dtype)) || !aligned(logprob, 4) || (entropy && !aligned(entropy, 4)) ||
      !aligned(targets, 8))
    return fail(LP_ERR_INVALID_ARGUMENT, "lp_logprobs_entropy: misaligned pointer");
  // Chunks bound the rows whose fp32 copy exists at once in the page's
  // design; here no fp32 copy exists (rows are widened in registers), so all
  // chunks of the call run back to back in one launch, in row order: one
  // drain of the grid per call instead of one per chunk, and results that do
  // not depend on chunk_rows.
  (void)chunk_rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  lp::RowArgs a;
  a.x = logits;
  a.ld = ld;
  a.V = static_cast<int>(V);
  a.targets = targets;
  a.K = static_cast<int>(K);
  a.mask = mask;
  a.c = exp2_scale(temperature);
  a.logprob = logprob;
  a.entropy = entropy;
  a.row0 = 0;
  a.rows = T;
  clear_pending_hip_error();
  hipError_t e = lp::launch_logprobs_entropy(static_cast<int>(dtype), a, s);
  if (e != hipSuccess) return hip_fail(e, "lp_logprobs_entropy launch");
  return ok();
}

lp_status lp_logprobs_entropy(const void* logits, lp_dtype dtype, int64_t T, int64_t V, int64_t ld,
                              const int64_t* targets, const uint8_t* mask, float temperature,
                              int64_t chunk_rows, float* logprob, float* entropy, void* stream) {
  return logprobs_entropy_impl(logits, dtype, T, V, ld, targets, 1, mask, temperature, chunk_rows, logprob, entropy,
                               stream);
}

lp_status lp_logprobs_entropy_k(const void* logits, lp_dtype dtype, int64_t T, int64_t V, int64_t ld,
                                const int64_t* targets, int64_t K, const uint8_t* mask, float temperature,
                                int64_t chunk_rows, float* logprob, float* entropy, void* stream) {
  return logprobs_entropy_impl(logits, dtype, T, V, ld, targets, K, mask, temperature, chunk_rows, logprob, entropy,
                               stream);
}

int lp_lm_head_fast_tiles(int64_t T, int64_t h, int64_t V, int64_t ld_h, int64_t ld_w, int64_t tile_rows,
                          int backward) {
  if (T < 0 || h <= 0 || V <= 0 || V > kMaxV || h > kMaxV || ld_h < h || ld_w < h || tile_rows <= 0) return -1;
  return lp::lmhead_fast_tiles(T, h, V, ld_h, ld_w, tile_rows, backward ? 1 : 0) ? 1 : 0;
}

size_t lp_lm_head_workspace_bytes(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward) {
  lp::LMHeadWorkspace w;
  if (!lp::lmhead_workspace_layout(T, h, V, tile_rows, backward, &w)) return 0;
  return w.total;
}

// static_scratch: the call brings no workspace (the no-alloc form checks its
// own scratch), so `workspace` is not examined.
static lp_status check_lmhead(const char* fn, const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                              int64_t T, int64_t h, int64_t V, const int64_t* targets, float temperature,
                              int64_t tile_rows, void* workspace, size_t workspace_bytes, int backward,
                              lp::LMHeadWorkspace* w, bool static_scratch = false) {
  if (T < 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: T < 0", fn);
  if (h <= 0 || V <= 0 || V > kMaxV || h > kMaxV)
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: h and V must be in 1..2^30", fn);
  if (ld_h < h || ld_w < h) return fail(LP_ERR_INVALID_ARGUMENT, "%s: ld_h and ld_w must be >= h", fn);
  if (tile_rows <= 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: tile_rows must be > 0", fn);
  if (!isfinite(temperature)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: temperature not finite", fn);
  if (h % 8 || ld_h % 8 || ld_w % 8)
    return fail(LP_ERR_UNSUPPORTED, "%s: h, ld_h and ld_w must be multiples of 8", fn);
  if (T == 0) return LP_OK;
  if (!hidden || !weight || !targets) return fail(LP_ERR_INVALID_ARGUMENT, "%s: hidden, weight, targets required", fn);
  if (!aligned(hidden, 16) || !aligned(weight, 16))
    return fail(LP_ERR_UNSUPPORTED, "%s: hidden and weight must be 16-byte aligned", fn);
  if (!aligned(targets, 8)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned targets", fn);
  if (!lp::lmhead_workspace_layout(T, h, V, tile_rows, backward, w))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: sizes overflow the workspace layout", fn);
  if (!lp::lmhead_launches_fit(T, h, V, tile_rows, backward))
    return fail(LP_ERR_UNSUPPORTED, "%s: a launch would exceed 2^32-1 work-items; use a smaller tile_rows", fn);
  if (static_scratch) return LP_OK;
  if (!workspace || workspace_bytes < w->total)
    return fail(LP_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu", fn, w->total,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  return LP_OK;
}

static lp::LMHeadShape make_shape(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w, int64_t T,
                                  int64_t h, int64_t V, const int64_t* targets, int64_t K, const uint8_t* mask,
                                  float temperature, int64_t tile_rows) {
  lp::LMHeadShape sh;
  sh.hidden = static_cast<const uint16_t*>(hidden);
  sh.ld_h = ld_h;
  sh.weight = static_cast<const uint16_t*>(weight);
  sh.ld_w = ld_w;
  sh.T = T;
  sh.h = static_cast<int>(h);
  sh.V = static_cast<int>(V);
  sh.targets = targets;
  sh.K = static_cast<int>(K);
  sh.mask = mask;
  sh.c = exp2_scale(temperature);
  sh.inv_tau = temperature_applies(temperature) ? 1.0f / temperature : 1.0f;
  sh.tile_rows = tile_rows;
  return sh;
}

static lp_status lm_head_forward_impl(const char* fn, const void* hidden, int64_t ld_h, const void* weight,
                                      int64_t ld_w, int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                      int64_t K, const uint8_t* mask, float temperature, int64_t tile_rows,
                                      float* logprob, float* entropy, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (K < 1 || K > lp::kMaxTargets) return fail(LP_ERR_INVALID_ARGUMENT, "%s: K must be in 1..%d", fn, lp::kMaxTargets);
  lp::LMHeadWorkspace w;
  lp_status st = check_lmhead(fn, hidden, ld_h, weight, ld_w, T, h, V, targets, temperature, tile_rows,
                              workspace, workspace_bytes, 0, &w);
  if (st != LP_OK) return st;
  if (T == 0) return ok();
  if (!logprob) return fail(LP_ERR_INVALID_ARGUMENT, "%s: logprob is required", fn);
  if (!f32_aligned({logprob, entropy, lse})) return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned fp32 output", fn);
  lp::LMHeadShape sh = make_shape(hidden, ld_h, weight, ld_w, T, h, V, targets, K, mask, temperature, tile_rows);
  clear_pending_hip_error();
  hipError_t e = lp::launch_lmhead_forward(sh, logprob, entropy, lse, static_cast<char*>(workspace), w,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

lp_status lp_lm_head_logprobs_entropy(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                      int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                      const uint8_t* mask, float temperature, int64_t tile_rows,
                                      float* logprob, float* entropy, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return lm_head_forward_impl("lp_lm_head_logprobs_entropy", hidden, ld_h, weight, ld_w, T, h, V, targets, 1, mask,
                              temperature, tile_rows, logprob, entropy, lse, workspace, workspace_bytes, stream);
}

lp_status lp_lm_head_logprobs_entropy_k(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                        int64_t T, int64_t h, int64_t V, const int64_t* targets, int64_t K,
                                        const uint8_t* mask, float temperature, int64_t tile_rows, float* logprob,
                                        float* entropy, float* lse, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return lm_head_forward_impl("lp_lm_head_logprobs_entropy_k", hidden, ld_h, weight, ld_w, T, h, V, targets, K, mask,
                              temperature, tile_rows, logprob, entropy, lse, workspace, workspace_bytes, stream);
}

lp_status lp_lm_head_logprobs_entropy_noalloc(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                              int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                              const uint8_t* mask, float temperature, int64_t tile_rows,
                                              float* logprob, float* entropy, float* lse, void* stream) {
  const char* fn = "lp_lm_head_logprobs_entropy_noalloc";
  lp::LMHeadWorkspace w;
  lp_status st = check_lmhead(fn, hidden, ld_h, weight, ld_w, T, h, V, targets, temperature, tile_rows, nullptr, 0,
                              0, &w, true);
  if (st != LP_OK) return st;
  if (T == 0) return ok();
  if (w.total > LP_NOALLOC_SCRATCH_BYTES)
    return fail(LP_ERR_WORKSPACE_TOO_SMALL,
                "%s: this shape needs %zu bytes of scratch, the static scratch holds %zu; use a smaller tile_rows "
                "or the workspace form",
                fn, w.total, static_cast<size_t>(LP_NOALLOC_SCRATCH_BYTES));
  if (!logprob) return fail(LP_ERR_INVALID_ARGUMENT, "%s: logprob is required", fn);
  if (!f32_aligned({logprob, entropy, lse})) return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned fp32 output", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int device = 0;
  void* ws = nullptr;
  hipError_t e = scratch_of_current_device(&device, &ws);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (s) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(s, &sd);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (sd != device)
      return fail(LP_ERR_INVALID_ARGUMENT, "%s: the stream belongs to device %d, the current device is %d", fn,
                  static_cast<int>(sd), device);
  }
  lp::LMHeadShape sh = make_shape(hidden, ld_h, weight, ld_w, T, h, V, targets, 1, mask, temperature, tile_rows);
  clear_pending_hip_error();
  e = lp::launch_lmhead_forward(sh, logprob, entropy, lse, static_cast<char*>(ws), w, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

static lp_status lm_head_backward_impl(const char* fn, const void* hidden, int64_t ld_h, const void* weight,
                                       int64_t ld_w, int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                       int64_t K, const uint8_t* mask, float temperature, int64_t tile_rows,
                                       const float* lse, const float* entropy, const float* grad_logprob,
                                       const float* grad_entropy, float* grad_hidden, float* grad_weight,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (K < 1 || K > lp::kMaxTargets) return fail(LP_ERR_INVALID_ARGUMENT, "%s: K must be in 1..%d", fn, lp::kMaxTargets);
  lp::LMHeadWorkspace w;
  lp_status st = check_lmhead(fn, hidden, ld_h, weight, ld_w, T, h, V, targets, temperature, tile_rows,
                              workspace, workspace_bytes, 1, &w);
  if (st != LP_OK) return st;
  if (!f32_aligned({lse, entropy, grad_logprob, grad_entropy, grad_hidden, grad_weight}))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned fp32 argument", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    // no rows: the weight gradient is still defined (all zero)
    if (grad_weight) {
      clear_pending_hip_error();
      hipError_t e = lp::launch_zero_f32(grad_weight, V * h, s);
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
  }
  if (!lse || !entropy || !grad_logprob)
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: lse, entropy and grad_logprob are required", fn);
  lp::LMHeadShape sh = make_shape(hidden, ld_h, weight, ld_w, T, h, V, targets, K, mask, temperature, tile_rows);
  clear_pending_hip_error();
  hipError_t e = lp::launch_lmhead_backward(sh, lse, entropy, grad_logprob, grad_entropy, grad_hidden,
                                            grad_weight, static_cast<char*>(workspace), w, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

lp_status lp_lm_head_logprobs_entropy_backward(const void* hidden, int64_t ld_h, const void* weight,
                                               int64_t ld_w, int64_t T, int64_t h, int64_t V,
                                               const int64_t* targets, const uint8_t* mask,
                                               float temperature, int64_t tile_rows, const float* lse,
                                               const float* entropy, const float* grad_logprob,
                                               const float* grad_entropy, float* grad_hidden,
                                               float* grad_weight, void* workspace, size_t workspace_bytes,
                                               void* stream) {
  return lm_head_backward_impl("lp_lm_head_logprobs_entropy_backward", hidden, ld_h, weight, ld_w, T, h, V, targets,
                               1, mask, temperature, tile_rows, lse, entropy, grad_logprob, grad_entropy, grad_hidden,
                               grad_weight, workspace, workspace_bytes, stream);
}

lp_status lp_lm_head_logprobs_entropy_backward_k(const void* hidden, int64_t ld_h, const void* weight,
                                                 int64_t ld_w, int64_t T, int64_t h, int64_t V,
                                                 const int64_t* targets, int64_t K, const uint8_t* mask,
                                                 float temperature, int64_t tile_rows, const float* lse,
                                                 const float* entropy, const float* grad_logprob,
                                                 const float* grad_entropy, float* grad_hidden, float* grad_weight,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
  return lm_head_backward_impl("lp_lm_head_logprobs_entropy_backward_k", hidden, ld_h, weight, ld_w, T, h, V, targets,
                               K, mask, temperature, tile_rows, lse, entropy, grad_logprob, grad_entropy, grad_hidden,
                               grad_weight, workspace, workspace_bytes, stream);
}

size_t lp_lm_head_kl_workspace_bytes(int64_t T, int64_t h_student, int64_t V, int64_t tile_rows, int backward) {
  lp::LMHeadWorkspace w;
  if (!lp::lmhead_workspace_layout(T, h_student, V, tile_rows, backward ? 3 : 2, &w)) return 0;
  return w.total;
}

// Checks of one head's operands (T > 0).
static lp_status check_head(const char* fn, const char* who, const void* hidden, int64_t ld_h, const void* weight,
                            int64_t ld_w, int64_t h) {
  if (h <= 0 || h > kMaxV) return fail(LP_ERR_INVALID_ARGUMENT, "%s: %s h must be in 1..2^30", fn, who);
  if (ld_h < h || ld_w < h) return fail(LP_ERR_INVALID_ARGUMENT, "%s: %s ld_h and ld_w must be >= h", fn, who);
  if (h % 8 || ld_h % 8 || ld_w % 8)
    return fail(LP_ERR_UNSUPPORTED, "%s: %s h, ld_h and ld_w must be multiples of 8", fn, who);
  if (!hidden || !weight) return fail(LP_ERR_INVALID_ARGUMENT, "%s: %s hidden and weight are required", fn, who);
  if (!aligned(hidden, 16) || !aligned(weight, 16))
    return fail(LP_ERR_UNSUPPORTED, "%s: %s hidden and weight must be 16-byte aligned", fn, who);
  return LP_OK;
}

static lp_status check_kl_heads(const char* fn, const void* hs, int64_t ld_hs, const void* ws_, int64_t ld_ws,
                                int64_t h_s, const void* ht, int64_t ld_ht, const void* wt, int64_t ld_wt,
                                int64_t h_t, int64_t T, int64_t V, int64_t tile_rows, void* workspace,
                                size_t workspace_bytes, int backward, lp::LMHeadWorkspace* w) {
  if (T < 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: T < 0", fn);
  if (V <= 0 || V > kMaxV) return fail(LP_ERR_INVALID_ARGUMENT, "%s: V must be in 1..2^30", fn);
  if (h_s <= 0 || h_s > kMaxV || h_t <= 0 || h_t > kMaxV)
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: h_student and h_teacher must be in 1..2^30", fn);
  if (tile_rows <= 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: tile_rows must be > 0", fn);
  if (T == 0) return LP_OK;
  lp_status st = check_head(fn, "student", hs, ld_hs, ws_, ld_ws, h_s);
  if (st != LP_OK) return st;
  if ((st = check_head(fn, "teacher", ht, ld_ht, wt, ld_wt, h_t)) != LP_OK) return st;
  if (!lp::lmhead_workspace_layout(T, h_s, V, tile_rows, backward ? 3 : 2, w))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: sizes overflow the workspace layout", fn);
  if (!lp::lmhead_launches_fit(T, h_s > h_t ? h_s : h_t, V, tile_rows, backward ? 3 : 2))
    return fail(LP_ERR_UNSUPPORTED, "%s: a launch would exceed 2^32-1 work-items; use a smaller tile_rows", fn);
  if (!workspace || workspace_bytes < w->total)
    return fail(LP_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu", fn, w->total,
                workspace ? workspace_bytes : size_t(0));
  if (!aligned(workspace, 256)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  return LP_OK;
}

lp_status lp_lm_head_kl(const void* student_hidden, int64_t ld_hs, const void* student_weight, int64_t ld_ws,
                        int64_t h_student, const void* teacher_hidden, int64_t ld_ht, const void* teacher_weight,
                        int64_t ld_wt, int64_t h_teacher, int64_t T, int64_t V, const uint8_t* mask,
                        const int64_t* targets, const uint8_t* diff_mask, int64_t tile_rows, float* kl,
                        float* lp_student, float* lp_teacher, float* prob_diff, float* lse_student,
                        float* lse_teacher, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lp_lm_head_kl";
  lp::LMHeadWorkspace w;
  lp_status st = check_kl_heads(fn, student_hidden, ld_hs, student_weight, ld_ws, h_student, teacher_hidden, ld_ht,
                                teacher_weight, ld_wt, h_teacher, T, V, tile_rows, workspace, workspace_bytes, 0, &w);
  if (st != LP_OK) return st;
  if (!targets && (lp_student || lp_teacher || prob_diff))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: lp_student/lp_teacher/prob_diff need targets", fn);
  if (T == 0) return ok();
  if (!kl) return fail(LP_ERR_INVALID_ARGUMENT, "%s: kl is required", fn);
  if (targets && !aligned(targets, 8)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned targets", fn);
  if (!f32_aligned({kl, lp_student, lp_teacher, prob_diff, lse_student, lse_teacher}))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned fp32 output", fn);
  const lp::LMHeadShape su = make_shape(student_hidden, ld_hs, student_weight, ld_ws, T, h_student, V, targets, 1,
                                        mask, 1.0f, tile_rows);
  const lp::LMHeadShape te = make_shape(teacher_hidden, ld_ht, teacher_weight, ld_wt, T, h_teacher, V, targets, 1,
                                        mask, 1.0f, tile_rows);
  const lp::KLHeadOutputs out{kl, lp_student, lp_teacher, prob_diff, lse_student, lse_teacher};
  clear_pending_hip_error();
  hipError_t e = lp::launch_lmhead_kl_forward(su, te, targets, diff_mask, out, static_cast<char*>(workspace), w,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

lp_status lp_lm_head_kl_backward(const void* student_hidden, int64_t ld_hs, const void* student_weight,
                                 int64_t ld_ws, int64_t h_student, const void* teacher_hidden, int64_t ld_ht,
                                 const void* teacher_weight, int64_t ld_wt, int64_t h_teacher, int64_t T, int64_t V,
                                 const uint8_t* mask, int64_t tile_rows, const float* lse_student,
                                 const float* lse_teacher, const float* grad_kl, float* grad_hidden,
                                 float* grad_weight, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lp_lm_head_kl_backward";
  lp::LMHeadWorkspace w;
  lp_status st = check_kl_heads(fn, student_hidden, ld_hs, student_weight, ld_ws, h_student, teacher_hidden, ld_ht,
                                teacher_weight, ld_wt, h_teacher, T, V, tile_rows, workspace, workspace_bytes, 1, &w);
  if (st != LP_OK) return st;
  if (!f32_aligned({lse_student, lse_teacher, grad_kl, grad_hidden, grad_weight}))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned fp32 argument", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (grad_weight) {
      clear_pending_hip_error();
      hipError_t e = lp::launch_zero_f32(grad_weight, V * h_student, s);
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
  }
  if (!lse_student || !lse_teacher || !grad_kl)
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: lse_student, lse_teacher and grad_kl are required", fn);
  const lp::LMHeadShape su = make_shape(student_hidden, ld_hs, student_weight, ld_ws, T, h_student, V, nullptr, 1,
                                        mask, 1.0f, tile_rows);
  const lp::LMHeadShape te = make_shape(teacher_hidden, ld_ht, teacher_weight, ld_wt, T, h_teacher, V, nullptr, 1,
                                        mask, 1.0f, tile_rows);
  clear_pending_hip_error();
  hipError_t e = lp::launch_lmhead_kl_backward(su, te, lse_student, lse_teacher, grad_kl, grad_hidden, grad_weight,
                                               static_cast<char*>(workspace), w, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

lp_status lp_kl_full_vocab(const void* student, const void* teacher, lp_dtype dtype, int64_t T, int64_t V,
                           int64_t ld_s, int64_t ld_t, float* kl, const int64_t* targets,
                           const uint8_t* diff_mask, float* lp_student, float* lp_teacher, float* prob_diff,
                           void* stream) {
  const char* fn = "lp_kl_full_vocab";
  if (dtype != LP_BF16 && dtype != LP_FP16 && dtype != LP_FP32)
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: dtype must be LP_BF16, LP_FP16 or LP_FP32", fn);
  if (T < 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: T < 0", fn);
  if (V <= 0 || V > kMaxV) return fail(LP_ERR_INVALID_ARGUMENT, "%s: V out of range (1..2^30)", fn);
  if (ld_s < V || ld_t < V) return fail(LP_ERR_INVALID_ARGUMENT, "%s: ld_s and ld_t must be >= V", fn);
  if (!targets && (lp_student || lp_teacher || prob_diff))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: lp_student/lp_teacher/prob_diff need targets", fn);
  if (T == 0) return ok();
  if (T > 0x7fffffff) return fail(LP_ERR_UNSUPPORTED, "%s: more than 2^31-1 rows", fn);
  if (!student || !teacher || !kl) return fail(LP_ERR_INVALID_ARGUMENT, "%s: student, teacher, kl required", fn);
  if (!aligned(student, dtype_bytes(dtype)) || !aligned(teacher, dtype_bytes(dtype)) ||
      (targets && !aligned(targets, 8)) || !f32_aligned({kl, lp_student, lp_teacher, prob_diff}))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", fn);
  lp::KLArgs a;
  a.student = student;
  a.teacher = teacher;
  a.ld_s = ld_s;
  a.ld_t = ld_t;
  a.V = static_cast<int>(V);
  a.T = T;
  a.row0 = 0;
  a.c = static_cast<float>(kLog2eD);
  a.kl = kl;
  a.targets = targets;
  a.diff_mask = diff_mask;
  a.lp_student = lp_student;
  a.lp_teacher = lp_teacher;
  a.prob_diff = prob_diff;
  clear_pending_hip_error();
  hipError_t e = lp::launch_kl_full_vocab(static_cast<int>(dtype), a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

lp_status lp_prob_diff(const float* lp_a, const float* lp_b, const uint8_t* mask, int64_t n, float* out,
                       void* stream) {
  if (n < 0) return fail(LP_ERR_INVALID_ARGUMENT, "lp_prob_diff: n < 0");
  if (n == 0) return ok();
  if (!lp_a || !lp_b || !out) return fail(LP_ERR_INVALID_ARGUMENT, "lp_prob_diff: lp_a, lp_b, out required");
  if (!f32_aligned({lp_a, lp_b, out})) return fail(LP_ERR_INVALID_ARGUMENT, "lp_prob_diff: misaligned pointer");
  clear_pending_hip_error();
  hipError_t e = lp::launch_prob_diff(lp_a, lp_b, mask, n, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "lp_prob_diff");
  return ok();
}

size_t lp_prob_diff_stats_workspace_bytes(void) { return lp::prob_diff_stats_workspace_bytes(); }

lp_status lp_prob_diff_stats(const float* lp_a, const float* lp_b, const uint8_t* mask, int64_t n, double* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "lp_prob_diff_stats";
  if (n < 0) return fail(LP_ERR_INVALID_ARGUMENT, "%s: n < 0", fn);
  if (!out) return fail(LP_ERR_INVALID_ARGUMENT, "%s: out is required", fn);
  if (n > 0 && (!lp_a || !lp_b)) return fail(LP_ERR_INVALID_ARGUMENT, "%s: lp_a and lp_b are required", fn);
  if (!f32_aligned({lp_a, lp_b})) return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned lp_a or lp_b", fn);
  if (!workspace || workspace_bytes < lp::prob_diff_stats_workspace_bytes())
    return fail(LP_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes", fn, lp::prob_diff_stats_workspace_bytes());
  if (!aligned(workspace, 256) || !aligned(out, 8))
    return fail(LP_ERR_INVALID_ARGUMENT, "%s: misaligned workspace or out", fn);
  clear_pending_hip_error();
  hipError_t e = lp::launch_prob_diff_stats(lp_a, lp_b, mask, n, out, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, fn);
  return ok();
}

}  // extern "C"
