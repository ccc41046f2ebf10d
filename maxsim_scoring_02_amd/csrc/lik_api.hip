// C ABI of the gfx950 MaxSim scorer: argument checks, plans, dispatch.
//
// Every argument is checked on the host before any device work (the colpali
// pull request, section "Design", describes the same split: an "unsupported"
// answer for calls the kernel cannot run, while real kernel errors
// propagate).  No device memory is allocated here; scratch comes from the
// caller's workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "lik.h"
#include "lik_kernels.h"
#include "lik_plan.h"

// Fixed scratch of the allocation-free forward (lik_maxsim_fwd_noalloc):
// every device the library runs on holds one copy, at its own address, until
// the process ends.  In host code `scratch` only stands for the symbol; its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

lik_status fail(lik_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

lik_status ok() {
  g_last_error[0] = '\0';
  return LIK_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 56;

// a*b*c... without overflow, or -1
int64_t mul_ok(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > kMaxElems / x) return -1;
    r *= x;
  }
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }


std::atomic<int> g_dev_ok[64];   // 0 unknown, 1 gfx950, 2 other

lik_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(LIK_ERR_UNSUPPORTED, "no HIP device is available");
  if (dev < 64) {
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 1) return LIK_OK;
    if (st == 2) return fail(LIK_ERR_UNSUPPORTED, "device %d is not a gfx950 (MI355X) GPU", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(LIK_ERR_UNSUPPORTED, "cannot query HIP device %d", dev);
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(good ? 1 : 2, std::memory_order_relaxed);
  if (!good) return fail(LIK_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return LIK_OK;
}

// Common checks.  `D_rows` = number of document token rows, `pairs` = score count.
struct Shapes {
  int layout;
  int64_t nq_or_b, Lq, nd_or_n, Ld, dim;
  int64_t q_rows, d_rows, pairs, n_docs;
};

lik_status check_shapes(lik_dtype dtype, Shapes& s) {
  if (dtype != LIK_F16 && dtype != LIK_BF16 && dtype != LIK_F32 && dtype != LIK_F32_BF16X3)
    return fail(LIK_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (s.nq_or_b < 0 || s.Lq < 0 || s.nd_or_n < 0 || s.Ld < 0 || s.dim < 0)
    return fail(LIK_ERR_INVALID_ARG, "negative size");
  if (s.Lq > INT32_MAX || s.Ld > INT32_MAX || s.dim > 65536)
    return fail(LIK_ERR_INVALID_ARG, "size out of range");
  s.q_rows = mul_ok({s.nq_or_b, s.Lq});
  if (s.layout == lik::kAllPairs) {
    s.n_docs = s.nd_or_n;
    s.pairs = mul_ok({s.nq_or_b, s.nd_or_n});
  } else if (s.layout == lik::kPairwise) {
    s.n_docs = s.nq_or_b;
    s.pairs = s.nq_or_b;
  } else {
    s.n_docs = mul_ok({s.nq_or_b, s.nd_or_n});
    s.pairs = s.n_docs;
  }
  s.d_rows = s.n_docs < 0 ? -1 : mul_ok({s.n_docs, s.Ld});
  if (s.q_rows < 0 || s.pairs < 0 || s.n_docs < 0 || s.d_rows < 0 ||
      mul_ok({s.q_rows, s.dim, 4}) < 0 || mul_ok({s.d_rows, s.dim, 4}) < 0 ||
      mul_ok({s.pairs, s.Lq, 4}) < 0 || s.n_docs > INT32_MAX)
    return fail(LIK_ERR_INVALID_ARG, "sizes overflow");
  return LIK_OK;
}

lik_status check_supported(lik_dtype dtype, const Shapes& s) {
  (void)dtype;
  if (s.dim == 0 || !lik::fwd_dim_supported(s.dim))
    return fail(LIK_ERR_UNSUPPORTED, "embedding dim %lld has no kernel in this library (64, 128, 256)",
                (long long)s.dim);
  if (s.layout == lik::kAllPairs && (s.nd_or_n > lik::kApMaxDocIndex || s.Ld > lik::kApMaxLd))
    return fail(LIK_ERR_UNSUPPORTED, "all-pairs supports Nd <= %lld and Ld <= %lld (got %lld, %lld)",
                (long long)lik::kApMaxDocIndex, (long long)lik::kApMaxLd, (long long)s.nd_or_n,
                (long long)s.Ld);
  if (s.layout == lik::kAllPairs && s.Lq > 0 && s.nq_or_b > lik::kApMaxTokens / s.Lq)
    return fail(LIK_ERR_UNSUPPORTED, "all-pairs supports Nq * Lq <= %lld (got %lld x %lld)",
                (long long)lik::kApMaxTokens, (long long)s.nq_or_b, (long long)s.Lq);
  return LIK_OK;
}

// LIK_F32_BF16X3 on the all-pairs forward: the split copies of Q and D live
// in the workspace and are bounded.
lik_status check_split(lik_dtype dtype, const Shapes& s) {
  if (dtype != LIK_F32_BF16X3 || !lik::split_supported(s.layout, s.dim)) return LIK_OK;
  const int64_t need = lik::split_bytes(s.q_rows, s.d_rows, s.dim);
  if (need > lik::kSplitMaxBytes)
    return fail(LIK_ERR_UNSUPPORTED,
                "LIK_F32_BF16X3: the split copies of Q and D would take %lld bytes (at most %lld); "
                "use LIK_F32",
                (long long)need, (long long)lik::kSplitMaxBytes);
  return LIK_OK;
}

bool is_zero_problem(const Shapes& s) { return s.pairs == 0; }

lik_status forward_entry(int layout, const void* Q, const void* D, lik_dtype dtype, int64_t nq_or_b,
                         int64_t Lq, int64_t nd_or_n, int64_t Ld, int64_t dim,
                         const uint8_t* q_mask, const uint8_t* d_mask, float* scores,
                         int32_t* argmax, void* workspace, size_t ws_bytes, void* stream) {
  Shapes s{layout, nq_or_b, Lq, nd_or_n, Ld, dim, 0, 0, 0, 0};
  lik_status st = check_shapes(dtype, s);
  if (st != LIK_OK) return st;
  if (is_zero_problem(s)) return ok();
  if (s.q_rows > 0 && !Q) return fail(LIK_ERR_INVALID_ARG, "Q is NULL");
  if (s.d_rows > 0 && !D) return fail(LIK_ERR_INVALID_ARG, "D is NULL");
  if (!scores) return fail(LIK_ERR_INVALID_ARG, "scores is NULL");
  if (!aligned16(Q) || !aligned16(D) || !aligned16(scores) || !aligned16(argmax) ||
      !aligned16(workspace))
    return fail(LIK_ERR_INVALID_ARG, "Q, D, scores, argmax and workspace must be 16-byte aligned");
  st = check_supported(dtype, s);
  if (st == LIK_OK) st = check_split(dtype, s);
  if (st != LIK_OK) return st;
  lik::FwdPlan p = lik::make_fwd_plan(layout, (int)dtype, nq_or_b, Lq, nd_or_n, Ld, dim,
                                      d_mask != nullptr, argmax != nullptr, q_mask != nullptr);
  if (ws_bytes < p.fwd_bytes)
    return fail(LIK_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", ws_bytes,
                p.fwd_bytes);
  if (p.fwd_bytes > 0 && !workspace) return fail(LIK_ERR_INVALID_ARG, "workspace is NULL");
  st = check_device();
  if (st != LIK_OK) return st;
  hipError_t e = lik::run_forward(p, Q, D, q_mask, d_mask, scores, argmax,
                                  static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LIK_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return ok();
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of this device's scratch (the current device's copy).
lik_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(LIK_ERR_UNSUPPORTED, "no HIP device is available");
  if (dev >= 64) return fail(LIK_ERR_UNSUPPORTED, "device %d: the fixed scratch serves devices 0-63", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LIK_ERR_HIP, "cannot resolve the fixed scratch on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LIK_OK;
}

lik_status backward_entry(int layout, const void* Q, const void* D, lik_dtype dtype,
                          int64_t nq_or_b, int64_t Lq, int64_t nd_or_n, int64_t Ld, int64_t dim,
                          const uint8_t* q_mask, const uint8_t* d_mask, const float* grad_scores,
                          const int32_t* argmax, float* grad_Q, float* grad_D, void* workspace,
                          size_t ws_bytes, void* stream) {
  Shapes s{layout, nq_or_b, Lq, nd_or_n, Ld, dim, 0, 0, 0, 0};
  lik_status st = check_shapes(dtype, s);
  if (st != LIK_OK) return st;
  if (is_zero_problem(s)) return ok();
  if (!grad_Q && !grad_D) return ok();
  if (s.q_rows > 0 && !Q) return fail(LIK_ERR_INVALID_ARG, "Q is NULL");
  if (s.d_rows > 0 && !D) return fail(LIK_ERR_INVALID_ARG, "D is NULL");
  if (!grad_scores) return fail(LIK_ERR_INVALID_ARG, "grad_scores is NULL");
  if (!aligned16(Q) || !aligned16(D) || !aligned16(grad_Q) || !aligned16(grad_D) ||
      !aligned16(argmax) || !aligned16(workspace) || !aligned4(grad_scores))
    return fail(LIK_ERR_INVALID_ARG,
                "Q, D, argmax, gradients and workspace must be 16-byte aligned");
  st = check_supported(dtype, s);
  if (st == LIK_OK && !argmax) st = check_split(dtype, s);   // the recomputing forward
  if (st != LIK_OK) return st;
  lik::BwdPlan p = lik::make_bwd_plan(layout, (int)dtype, nq_or_b, Lq, nd_or_n, Ld, dim,
                                      d_mask != nullptr, argmax != nullptr, q_mask != nullptr);
  if (ws_bytes < p.total)
    return fail(LIK_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", ws_bytes,
                p.total);
  if (p.total > 0 && !workspace) return fail(LIK_ERR_INVALID_ARG, "workspace is NULL");
  st = check_device();
  if (st != LIK_OK) return st;
  hipError_t e = lik::run_backward(p, Q, D, q_mask, d_mask, grad_scores, argmax, grad_Q, grad_D,
                                   static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LIK_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace lik {
void profile_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_prof_start;
  *stop = g_prof_stop;
}
}  // namespace lik

extern "C" {

int lik_abi_version(void) { return LIK_ABI_VERSION; }

const char* lik_status_string(lik_status s) {
  switch (s) {
    case LIK_OK: return "ok";
    case LIK_ERR_INVALID_ARG: return "invalid argument";
    case LIK_ERR_UNSUPPORTED: return "unsupported";
    case LIK_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* lik_last_error(void) { return g_last_error; }

int lik_supported_dim(int64_t dim) { return lik::fwd_dim_supported(dim) ? 1 : 0; }

lik_status lik_set_profile_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(LIK_ERR_INVALID_ARG, "profile events: pass both or neither");
  g_prof_start = static_cast<hipEvent_t>(start_event);
  g_prof_stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

size_t lik_workspace_bytes(lik_op op, int64_t nq_or_b, int64_t lq, int64_t nd_or_n, int64_t ld,
                           int64_t dim, lik_dtype dtype, int flags) {
  if (nq_or_b < 0 || lq < 0 || nd_or_n < 0 || ld < 0 || dim < 0) return SIZE_MAX;
  int layout;
  bool bwd;
  switch (op) {
    case LIK_OP_FWD: layout = lik::kAllPairs; bwd = false; break;
    case LIK_OP_BWD: layout = lik::kAllPairs; bwd = true; break;
    case LIK_OP_PAIRWISE_FWD: layout = lik::kPairwise; bwd = false; break;
    case LIK_OP_PAIRWISE_BWD: layout = lik::kPairwise; bwd = true; break;
    case LIK_OP_KD_FWD: layout = lik::kKd; bwd = false; break;
    case LIK_OP_KD_BWD: layout = lik::kKd; bwd = true; break;
    default: return SIZE_MAX;
  }
  Shapes s{layout, nq_or_b, lq, nd_or_n, ld, dim, 0, 0, 0, 0};
  if (check_shapes(dtype == LIK_F32 || dtype == LIK_F16 || dtype == LIK_BF16 ||
                           dtype == LIK_F32_BF16X3
                       ? dtype
                       : LIK_BF16,
                   s) != LIK_OK)
    return SIZE_MAX;
  const bool has_dmask = (flags & 2) != 0;
  const bool arg = (flags & 1) != 0;
  const bool has_qmask = (flags & 4) != 0;
  if (!bwd)
    return lik::make_fwd_plan(layout, (int)dtype, nq_or_b, lq, nd_or_n, ld, dim, has_dmask, arg,
                              has_qmask)
        .fwd_bytes;
  return lik::make_bwd_plan(layout, (int)dtype, nq_or_b, lq, nd_or_n, ld, dim, has_dmask, arg,
                            has_qmask)
      .total;
}

namespace {
int64_t fwd_plan_value(const lik::FwdPlan& p, const char* key) {
  struct KV { const char* k; int64_t v; };
  const KV kv[] = {{"nb", p.NB},           {"upw", p.upw},         {"n_groups", p.n_groups},
                   {"n_sb", p.n_sb},       {"nchunks", p.nchunks}, {"tpc", p.tpc},
                   {"compact", p.compact}, {"partial", p.partial}, {"qpw", p.qpw},
                   {"n_units", p.n_units}, {"n_cg", p.n_cg},       {"split", p.elem == 3}};
  for (const KV& e : kv)
    if (std::strcmp(key, e.k) == 0) return e.v;
  return -1;
}
}  // namespace

int64_t lik_plan_value(lik_op op, int64_t nq_or_b, int64_t lq, int64_t nd_or_n, int64_t ld,
                       int64_t dim, lik_dtype dtype, int flags, const char* key) {
  if (!key) return -1;
  const size_t ws = lik_workspace_bytes(op, nq_or_b, lq, nd_or_n, ld, dim, dtype, flags);
  if (ws == SIZE_MAX) return -1;
  if (std::strcmp(key, "workspace") == 0) return (int64_t)ws;
  const int layout = (op == LIK_OP_FWD || op == LIK_OP_BWD)                   ? lik::kAllPairs
                     : (op == LIK_OP_PAIRWISE_FWD || op == LIK_OP_PAIRWISE_BWD) ? lik::kPairwise
                                                                                : lik::kKd;
  const bool bwd = op == LIK_OP_BWD || op == LIK_OP_PAIRWISE_BWD || op == LIK_OP_KD_BWD;
  const bool has_dmask = (flags & 2) != 0, arg = (flags & 1) != 0, has_qmask = (flags & 4) != 0;
  if (!bwd)
    return fwd_plan_value(lik::make_fwd_plan(layout, (int)dtype, nq_or_b, lq, nd_or_n, ld, dim,
                                             has_dmask, arg, has_qmask),
                          key);
  const lik::BwdPlan b = lik::make_bwd_plan(layout, (int)dtype, nq_or_b, lq, nd_or_n, ld, dim,
                                            has_dmask, arg, has_qmask);
  struct KV { const char* k; int64_t v; };
  const KV kv[] = {{"gd_mode", b.gd_mode},     {"gd_parts", b.gd_parts}, {"gs_split", b.gs_split},
                   {"gs_sw", b.gs_sw},         {"gq_ap", b.gq_ap},       {"gq_slices", b.gq_slices},
                   {"recompute", b.recompute}, {"gs_lds", (int64_t)b.gs_lds},
                   {"sort_batch", b.sort_batch}};
  for (const KV& e : kv)
    if (std::strcmp(key, e.k) == 0) return e.v;
  return fwd_plan_value(b.fwd, key);
}

lik_status lik_maxsim_fwd(const void* Q, const void* D, lik_dtype dtype, int64_t Nq, int64_t Lq,
                          int64_t Nd, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                          const uint8_t* d_mask, float* scores, int32_t* argmax, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return forward_entry(lik::kAllPairs, Q, D, dtype, Nq, Lq, Nd, Ld, dim, q_mask, d_mask, scores,
                       argmax, workspace, workspace_bytes, stream);
}

lik_status lik_maxsim_fwd_noalloc(const void* Q, const void* D, lik_dtype dtype, int64_t Nq,
                                  int64_t Lq, int64_t Nd, int64_t Ld, int64_t dim,
                                  const uint8_t* q_mask, const uint8_t* d_mask, float* scores,
                                  int32_t* argmax, void* stream) {
  Shapes s{lik::kAllPairs, Nq, Lq, Nd, Ld, dim, 0, 0, 0, 0};
  lik_status st = check_shapes(dtype, s);
  if (st != LIK_OK) return st;
  if (is_zero_problem(s)) return ok();
  const size_t need = lik::make_fwd_plan(lik::kAllPairs, (int)dtype, Nq, Lq, Nd, Ld, dim,
                                         d_mask != nullptr, argmax != nullptr, q_mask != nullptr)
                          .fwd_bytes;
  if (need > kScratchBytes)
    return fail(LIK_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch; the fixed scratch holds %zu (use "
                "lik_maxsim_fwd with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = check_device();
    if (st != LIK_OK) return st;
    st = scratch_address(&ws);
    if (st != LIK_OK) return st;
  }
  return forward_entry(lik::kAllPairs, Q, D, dtype, Nq, Lq, Nd, Ld, dim, q_mask, d_mask, scores,
                       argmax, ws, need, stream);
}

lik_status lik_maxsim_bwd(const void* Q, const void* D, lik_dtype dtype, int64_t Nq, int64_t Lq,
                          int64_t Nd, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                          const uint8_t* d_mask, const float* grad_scores, const int32_t* argmax,
                          float* grad_Q, float* grad_D, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return backward_entry(lik::kAllPairs, Q, D, dtype, Nq, Lq, Nd, Ld, dim, q_mask, d_mask,
                        grad_scores, argmax, grad_Q, grad_D, workspace, workspace_bytes, stream);
}

lik_status lik_maxsim_pairwise_fwd(const void* Q, const void* D, lik_dtype dtype, int64_t B,
                                   int64_t Lq, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                                   const uint8_t* d_mask, float* scores, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return forward_entry(lik::kPairwise, Q, D, dtype, B, Lq, 1, Ld, dim, q_mask, d_mask, scores,
                       argmax, workspace, workspace_bytes, stream);
}

lik_status lik_maxsim_pairwise_bwd(const void* Q, const void* D, lik_dtype dtype, int64_t B,
                                   int64_t Lq, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                                   const uint8_t* d_mask, const float* grad_scores,
                                   const int32_t* argmax, float* grad_Q, float* grad_D,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return backward_entry(lik::kPairwise, Q, D, dtype, B, Lq, 1, Ld, dim, q_mask, d_mask,
                        grad_scores, argmax, grad_Q, grad_D, workspace, workspace_bytes, stream);
}

lik_status lik_maxsim_kd_fwd(const void* Q, const void* D, lik_dtype dtype, int64_t B, int64_t Lq,
                             int64_t N, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                             const uint8_t* d_mask, float* scores, int32_t* argmax,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return forward_entry(lik::kKd, Q, D, dtype, B, Lq, N, Ld, dim, q_mask, d_mask, scores, argmax,
                       workspace, workspace_bytes, stream);
}

lik_status lik_maxsim_kd_bwd(const void* Q, const void* D, lik_dtype dtype, int64_t B, int64_t Lq,
                             int64_t N, int64_t Ld, int64_t dim, const uint8_t* q_mask,
                             const uint8_t* d_mask, const float* grad_scores,
                             const int32_t* argmax, float* grad_Q, float* grad_D,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return backward_entry(lik::kKd, Q, D, dtype, B, Lq, N, Ld, dim, q_mask, d_mask, grad_scores,
                        argmax, grad_Q, grad_D, workspace, workspace_bytes, stream);
}

lik_status lik_ce_rows(const float* scores, int64_t R, int64_t C, const int32_t* labels,
                       float scale, float* row_loss, float* loss, float* grad_scores,
                       void* stream) {
  if (R < 0 || C < 0) return fail(LIK_ERR_INVALID_ARG, "negative size (R %lld, C %lld)",
                                  (long long)R, (long long)C);
  if (mul_ok({R, C}) < 0) return fail(LIK_ERR_INVALID_ARG, "R x C overflows");
  if (R == 0) return ok();
  if (C == 0) return fail(LIK_ERR_INVALID_ARG, "rows have no columns (C == 0)");
  if (!labels && C < R)
    return fail(LIK_ERR_INVALID_ARG, "diagonal targets need C >= R (got R %lld, C %lld)",
                (long long)R, (long long)C);
  if (!scores) return fail(LIK_ERR_INVALID_ARG, "scores is NULL");
  if (!row_loss) return fail(LIK_ERR_INVALID_ARG, "row_loss is NULL");
  if (!loss) return fail(LIK_ERR_INVALID_ARG, "loss is NULL");
  if (!(scale == scale) || scale == 0.0f || scale > 3.4e38f || scale < -3.4e38f)
    return fail(LIK_ERR_INVALID_ARG, "scale must be finite and non-zero");
  if (!aligned4(scores) || !aligned4(labels) || !aligned4(row_loss) || !aligned4(loss) ||
      !aligned4(grad_scores))
    return fail(LIK_ERR_INVALID_ARG, "scores, labels, losses and gradient must be 4-byte aligned");
  if (R > (int64_t(1) << 32)) return fail(LIK_ERR_UNSUPPORTED, "R > 2^32 rows");
  lik_status st = check_device();
  if (st != LIK_OK) return st;
  hipError_t e = lik::run_ce_rows(scores, R, C, labels, scale, row_loss, loss, grad_scores,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(LIK_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
