// C ABI of libw8mp: argument validation, workspace carve-up, kernel dispatch.
// Declarations and contracts: include/w8mp.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "launch.h"
#include "w8mp.h"


namespace {

thread_local std::string g_last_error;

w8_status fail(w8_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

w8_status ok() {
  g_last_error.clear();
  return W8_OK;
}

w8_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(W8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest dimension the kernels index with 32-bit row counters.
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

#define W8_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

w8_status check_mk(int64_t M, int64_t K, int64_t maxK) {
  W8_REQUIRE(M >= 1 && M <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "M must be in [1, 2^31): got %lld", (long long)M);
  W8_REQUIRE(K >= 16 && K % 16 == 0, W8_ERR_INVALID_ARGUMENT, "K must be a positive multiple of 16: got %lld",
             (long long)K);
  W8_REQUIRE(K <= maxK, W8_ERR_UNSUPPORTED, "K=%lld exceeds the supported maximum %lld", (long long)K,
             (long long)maxK);
  W8_REQUIRE(M * K < (int64_t{1} << 46), W8_ERR_UNSUPPORTED, "M*K too large");
  return W8_OK;
}

// Compute units of the current device (cached per device); the GEMM plan
// depends on it, so workspace sizes are per device. Threads may race to fill
// an entry; they all store the same value, and the atomics keep that defined.
int cu_count() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

namespace w8 {
// Error and device queries for the other translation units of the library.
int report_status(int status, const char* detail) {
  g_last_error = detail ? detail : "";
  return status;
}
int device_cus() { return cu_count(); }
}  // namespace w8

namespace {

// Workspace layout of int8_mixed_linear (offsets from the 256-aligned base).
// flags and cnt are the bookkeeping that every call leaves zero again.
struct Int8Ws {
  size_t q, sx, rstd, flags, cnt, nO, O, XO, WO, part, total;
  w8::GemmPlan plan;
};

Int8Ws int8_layout(int64_t M, int64_t N, int64_t K) {
  Int8Ws w{};
  w.plan = w8::plan_int8_gemm(M, N, K, cu_count());
  const size_t P = static_cast<size_t>((K + 31) / 32 * 32);  // worst case: every column is an outlier
  size_t off = 0;
  w.q = off;     off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;    off = up(off + 4 * static_cast<size_t>(M));
  w.rstd = off;  off = up(off + 4 * static_cast<size_t>(M));
  w.flags = off; off = up(off + static_cast<size_t>(K));
  w.cnt = off;   off = up(off + 4 * static_cast<size_t>(w.plan.counters()));
  w.nO = off;    off = up(off + 4);
  w.O = off;     off = up(off + 4 * static_cast<size_t>(K));
  w.XO = off;    off = up(off + 2 * static_cast<size_t>(M) * P);
  w.WO = off;    off = up(off + 2 * static_cast<size_t>(N) * P);
  w.part = off;  off = up(off + w.plan.partial_bytes());
  w.total = off;
  return w;
}

// Magnitude bits (bits & 0x7FFF) of the largest value of the 16-bit format
// that is <= t: |x| > t exactly when x's magnitude bits exceed it.
uint32_t threshold_bits(float t, bool bf16) {
  if (bf16) {
    uint32_t u;
    std::memcpy(&u, &t, 4);
    return std::min<uint32_t>(u >> 16, 0x7F80u);   // truncation = round toward zero for t >= 0
  }
  auto f16_value = [](uint32_t h) -> double {        // h: magnitude bits of a non-NaN half
    const int e = static_cast<int>(h >> 10), m = static_cast<int>(h & 0x3FF);
    if (e == 31) return INFINITY;
    return e == 0 ? std::ldexp(static_cast<double>(m), -24) : std::ldexp(1024.0 + m, e - 25);
  };
  uint32_t lo = 0, hi = 0x7C00;                        // f16_value(lo) <= t always (t >= 0)
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    if (f16_value(mid) <= static_cast<double>(t)) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Workspace of the int8 GEMM parity export: counters, then partials.
struct GemmWs {
  size_t cnt, part, total;
  w8::GemmPlan plan;
};

// tail: 0 the linear's own plan; 1 leftover tiles as `split` 256x256 slices
// (split 1: every tile whole); 2 as `split` slices of 128x128 quarters.
GemmWs gemm_layout(int64_t M, int64_t N, int64_t K, int tail = 0, int split = 1) {
  GemmWs w{};
  w.plan = tail == 0 ? w8::plan_int8_gemm(M, N, K, cu_count())
                     : w8::plan_int8_gemm_forced(M, N, cu_count(), tail == 2, split);
  size_t off = 0;
  w.cnt = off;  off = up(off + 4 * static_cast<size_t>(w.plan.counters()));
  w.part = off; off = up(off + w.plan.partial_bytes());
  w.total = off;
  return w;
}

// Workspace layout of fp8_w8a8_linear: codes, scales, then the GEMM's split-K
// counters (left zero by every call) and partials.
struct Fp8Ws {
  size_t xq, sx, cnt, part, total;
  w8::GemmPlan plan;
};

Fp8Ws fp8_layout(int64_t M, int64_t N, int64_t K) {
  Fp8Ws w{};
  w.plan = w8::plan_fp8_gemm(M, N, K, cu_count());
  size_t off = 0;
  w.xq = off;   off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;   off = up(off + 4 * static_cast<size_t>(M));
  w.cnt = off;  off = up(off + 4 * static_cast<size_t>(w.plan.counters()));
  w.part = off; off = up(off + w.plan.partial_bytes());
  w.total = off;
  return w;
}

// Grid of the FP8 GEMM parity export: the linear's own plan (split 0) or the
// given block size and K-slicing.
w8::GemmPlan fp8_debug_plan(int64_t M, int64_t N, int64_t K, int split, int tile) {
  return split == 0 ? w8::plan_fp8_gemm(M, N, K, cu_count())
                    : w8::plan_fp8_gemm_split(M, N, split, tile == 128 ? 128 : 256);
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

w8_status check_ws(void* ws, size_t bytes, size_t need) {
  W8_REQUIRE(ws != nullptr, W8_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  W8_REQUIRE((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0, W8_ERR_WORKSPACE,
             "workspace must be 256-byte aligned");
  W8_REQUIRE(bytes >= need, W8_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", bytes, need);
  return W8_OK;
}

// Measurement hook state (see w8_profile_start in w8mp.h).
struct Profile {
  bool on = false;
  int cap = 0, n = 0;
  std::vector<hipEvent_t> ev;  // 4 per call: start, after row pass, after fix-up, after GEMM
} g_prof;

// Record boundary `b` (0..3) of the current call; a no-op unless profiling.
void mark(int b, hipStream_t s) {
  if (!g_prof.on || g_prof.n >= g_prof.cap) return;
  (void)hipEventRecord(g_prof.ev[4 * g_prof.n + b], s);
  if (b == 3) ++g_prof.n;
}

}  // namespace

extern "C" {

w8_status w8_profile_start(int max_calls) {
  W8_REQUIRE(max_calls >= 1, W8_ERR_INVALID_ARGUMENT, "max_calls must be >= 1");
  double unused[3];
  int n;
  if (g_prof.on) w8_profile_stop(unused, &n);
  g_prof.ev.assign(4 * static_cast<size_t>(max_calls), nullptr);
  for (auto& e : g_prof.ev) {
    if (hipEventCreate(&e) != hipSuccess) return fail(W8_ERR_HIP, "hipEventCreate failed");
  }
  g_prof.cap = max_calls;
  g_prof.n = 0;
  g_prof.on = true;
  return ok();
}

w8_status w8_profile_stop(double* stage_ms, int* n_calls) {
  W8_REQUIRE(stage_ms && n_calls, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  stage_ms[0] = stage_ms[1] = stage_ms[2] = 0.0;
  *n_calls = 0;
  if (!g_prof.on) return ok();
  w8_status st = W8_OK;
  for (int c = 0; c < g_prof.n; ++c) {
    hipEvent_t* e = &g_prof.ev[4 * static_cast<size_t>(c)];
    if (hipEventSynchronize(e[3]) != hipSuccess) st = W8_ERR_HIP;
    for (int k = 0; k < 3; ++k) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, e[k], e[k + 1]) != hipSuccess) st = W8_ERR_HIP;
      stage_ms[k] += ms;
    }
  }
  *n_calls = g_prof.n;
  for (auto& e : g_prof.ev)
    if (e) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on = false;
  g_prof.cap = g_prof.n = 0;
  return st == W8_OK ? ok() : fail(st, "reading profile events failed");
}

const char* w8_status_string(int status) {
  switch (status) {
    case W8_OK: return "W8_OK";
    case W8_ERR_INVALID_ARGUMENT: return "W8_ERR_INVALID_ARGUMENT";
    case W8_ERR_UNSUPPORTED: return "W8_ERR_UNSUPPORTED";
    case W8_ERR_WORKSPACE: return "W8_ERR_WORKSPACE";
    case W8_ERR_HIP: return "W8_ERR_HIP";
    default: return "W8_UNKNOWN_STATUS";
  }
}

const char* w8_last_error(void) { return g_last_error.c_str(); }

w8_status quantize_weight_rowwise(const void* W, int w_dt, int64_t N, int64_t K, int fmt, void* Wq, float* sw,
                                  void* stream) {
  W8_REQUIRE(W && Wq && sw, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(w_dt == W8_DT_F16 || w_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "weights must be f16 or bf16");
  W8_REQUIRE(fmt == W8_Q_INT8 || fmt == W8_Q_FP8_E4M3 || fmt == W8_Q_INT4_G128, W8_ERR_UNSUPPORTED,
             "unknown weight format %d", fmt);
  if (w8_status st = check_mk(N, K, fmt == W8_Q_INT8 ? W8_INT8_MAX_K : 65536); st != W8_OK) return st;
  W8_REQUIRE(fmt != W8_Q_INT4_G128 || K % 128 == 0, W8_ERR_UNSUPPORTED, "int4 groups need K %% 128 == 0");
  W8_REQUIRE(aligned16(W) && aligned16(Wq) && aligned16(sw), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = w_dt == W8_DT_BF16;
  if (fmt == W8_Q_INT8)
    w8::launch_int8_rows(W, bf, N, (int)K, 0x7F80u, static_cast<int8_t*>(Wq), sw, nullptr, w8::kProdNone,
                         w8::ProdArgs{}, s);
  else if (fmt == W8_Q_INT4_G128)
    w8::launch_int4_weights(W, bf, N, (int)K, static_cast<uint8_t*>(Wq), sw, s);
  else
    w8::launch_fp8_rows(W, bf, N, (int)K, nullptr, static_cast<uint8_t*>(Wq), sw, 2, s);
  return check_launch("quantize_weight_rowwise");
}

size_t int8_mixed_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return int8_layout(M, N, K).total;
}

static w8_status int8_common_checks(const void* X, int x_dt, int64_t M, int64_t K, float threshold) {
  W8_REQUIRE(X != nullptr, W8_ERR_INVALID_ARGUMENT, "X is NULL");
  W8_REQUIRE(x_dt == W8_DT_F16 || x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  if (w8_status st = check_mk(M, K, W8_INT8_MAX_K); st != W8_OK) return st;
  W8_REQUIRE(!std::isnan(threshold) && threshold >= 0.0f, W8_ERR_INVALID_ARGUMENT,
             "threshold must be >= 0 (+inf allowed), got %g", (double)threshold);
  W8_REQUIRE(aligned16(X), W8_ERR_INVALID_ARGUMENT, "X must be 16-byte aligned");
  return W8_OK;
}

// Producer descriptor -> kernel arguments; NULL means none.
static w8_status producer_args(const w8_producer* p, int64_t K, int* kind, w8::ProdArgs* pa) {
  *kind = w8::kProdNone;
  *pa = w8::ProdArgs{nullptr, nullptr, nullptr, 0.0f, nullptr};
  if (!p || p->kind == W8_PRODUCER_NONE) return W8_OK;
  W8_REQUIRE(p->kind == W8_PRODUCER_RMSNORM || p->kind == W8_PRODUCER_GELU_TANH, W8_ERR_INVALID_ARGUMENT,
             "unknown producer kind %d", p->kind);
  W8_REQUIRE(K <= 16384, W8_ERR_UNSUPPORTED, "a producer needs K <= 16384, got %lld", (long long)K);
  if (p->kind == W8_PRODUCER_RMSNORM) {
    W8_REQUIRE(std::isfinite(p->eps) && p->eps >= 0.0f, W8_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    W8_REQUIRE(aligned16(p->gamma) && aligned16(p->scale) && aligned16(p->shift), W8_ERR_INVALID_ARGUMENT,
               "gamma, scale and shift must be 16-byte aligned");
    *kind = w8::kProdRms;
    *pa = w8::ProdArgs{p->gamma, p->scale, p->shift, p->eps, nullptr};
  } else {
    *kind = w8::kProdGelu;
  }
  return W8_OK;
}

static w8_status int8_linear_impl(const void* X, int x_dt, int64_t M, int64_t K, const w8_producer* producer,
                                  const int8_t* Wq, const float* sw, const float* bias, int64_t N, float threshold,
                                  void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream,
                                  const char* what) {
  if (w8_status st = int8_common_checks(X, x_dt, M, K, threshold); st != W8_OK) return st;
  W8_REQUIRE(Wq && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED, "Y must be f16 or f32");
  W8_REQUIRE(aligned16(Wq) && aligned16(sw) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  int kind = 0;
  w8::ProdArgs pa{};
  if (w8_status st = producer_args(producer, K, &kind, &pa); st != W8_OK) return st;
  const Int8Ws L = int8_layout(M, N, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, L.total); st != W8_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = x_dt == W8_DT_BF16;
  int8_t* q = at<int8_t>(workspace, L.q);
  float* sx = at<float>(workspace, L.sx);
  uint8_t* flags = at<uint8_t>(workspace, L.flags);
  int* nO = at<int>(workspace, L.nO);
  int* O = at<int>(workspace, L.O);
  uint16_t* XO = at<uint16_t>(workspace, L.XO);
  uint16_t* WO = at<uint16_t>(workspace, L.WO);
  int* cnt = at<int>(workspace, L.cnt);
  int* part = at<int>(workspace, L.part);
  pa.rstd = at<float>(workspace, L.rstd);

  mark(0, s);
  const uint32_t tb = threshold_bits(threshold, bf);
  w8::launch_int8_rows(X, bf, M, (int)K, tb, q, sx, flags, kind, pa, s);
  mark(1, s);
  w8::launch_outlier_fixup(X, bf, M, (int)K, tb, flags, q, sx, O, nO, XO, Wq, N, WO, kind, pa, s);
  mark(2, s);
  w8::launch_int8_gemm(q, Wq, M, N, K, sx, sw, nO, XO, WO, bf, bias, Y, y_dt == W8_DT_F16 ? 1 : 2, L.plan, part,
                       cnt, reinterpret_cast<uint32_t*>(flags), static_cast<int>(K / 4), s);
  mark(3, s);
  return check_launch(what);
}

w8_status int8_mixed_linear(const void* X, int x_dt, int64_t M, int64_t K, const int8_t* Wq, const float* sw,
                            int64_t N, float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return int8_linear_impl(X, x_dt, M, K, nullptr, Wq, sw, nullptr, N, threshold, Y, y_dt, workspace,
                          workspace_bytes, stream, "int8_mixed_linear");
}

w8_status int8_mixed_linear_fused(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                  const int8_t* Wq, const float* sw, const float* bias, int64_t N, float threshold,
                                  void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  return int8_linear_impl(H, h_dt, M, K, producer, Wq, sw, bias, N, threshold, Y, y_dt, workspace, workspace_bytes,
                          stream, "int8_mixed_linear_fused");
}

size_t fp8_w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return fp8_layout(M, N, K).total;
}

w8_status fp8_w8a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                          int64_t N, const float* act_scale, void* Y, int y_dt, void* workspace,
                          size_t workspace_bytes, void* stream) {
  W8_REQUIRE(X && Wq8 && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(x_dt == W8_DT_F16 || x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  W8_REQUIRE(y_dt == W8_DT_BF16 || y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED,
             "Y must be bf16, f16 or f32");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(aligned16(X) && aligned16(Wq8) && aligned16(sw) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  const Fp8Ws L = fp8_layout(M, N, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, L.total); st != W8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* sx = at<float>(workspace, L.sx);
  mark(0, s);
  w8::launch_fp8_rows(X, x_dt == W8_DT_BF16, M, (int)K, act_scale, xq, sx, act_scale ? 1 : 0, s);
  mark(1, s);
  mark(2, s);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_fp8_gemm(xq, Wq8, M, N, K, sx, sw, Y, ydt, L.plan, at<float>(workspace, L.part),
                      at<int>(workspace, L.cnt), s);
  mark(3, s);
  return check_launch("fp8_w8a8_linear");
}

}  // extern "C"

namespace {

// FP8 weight-only: split-K counters and partials of the plan (at least one
// aligned unit, so a workspace is always passed).
struct W16Ws {
  size_t cnt, part, total;
  w8::GemmPlan plan;
};

W16Ws w16_layout(const w8::GemmPlan& plan) {
  W16Ws w{};
  w.plan = plan;
  size_t off = 0;
  w.cnt = off;  off = up(off + 4 * static_cast<size_t>(plan.counters()));
  w.part = off; off = up(off + plan.partial_bytes());
  w.total = std::max<size_t>(off, kAlign);
  return w;
}

w8::GemmPlan w16_plan(int64_t M, int64_t N, int64_t K, int split, int tile) {
  return split == 0 ? w8::plan_w8a16_gemm(M, N, K, cu_count())
                    : w8::plan_w8a16_gemm_split(M, N, split, tile == 128 ? 128 : 256);
}

}  // namespace

extern "C" {

static w8_status w16_checks(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                            int64_t N, void* Y, int y_dt) {
  W8_REQUIRE(X && Wq8 && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be bf16 (the weight-only path computes in bf16)");
  W8_REQUIRE(y_dt == W8_DT_BF16 || y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED,
             "Y must be bf16, f16 or f32");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(K % 64 == 0, W8_ERR_UNSUPPORTED, "K must be a multiple of 64, got %lld", (long long)K);
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(aligned16(X) && aligned16(Wq8) && aligned16(sw) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  return W8_OK;
}

static w8_status w16_run(const void* X, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw, int64_t N,
                         void* Y, int y_dt, const W16Ws& L, void* workspace, size_t workspace_bytes, void* stream,
                         const char* what) {
  if (w8_status st = check_ws(workspace, workspace_bytes, L.total); st != W8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  mark(0, s);
  mark(1, s);
  mark(2, s);
  w8::launch_w8a16_gemm(static_cast<const uint16_t*>(X), Wq8, M, N, K, sw, Y, ydt, L.plan,
                        at<float>(workspace, L.part), at<int>(workspace, L.cnt), s);
  mark(3, s);
  return check_launch(what);
}

size_t fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return w16_layout(w16_plan(M, N, K, 0, 0)).total;
}

w8_status fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                           int64_t N, void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w16_checks(X, x_dt, M, K, Wq8, sw, N, Y, y_dt); st != W8_OK) return st;
  return w16_run(X, M, K, Wq8, sw, N, Y, y_dt, w16_layout(w16_plan(M, N, K, 0, 0)), workspace, workspace_bytes,
                 stream, "fp8_w8a16_linear");
}

}  // extern "C"

namespace {

// W4A8: activation codes and row scales, split-K counters and partials.
struct W4Ws {
  size_t q, sx, cnt, part, total;
  w8::GemmPlan plan;
};

W4Ws w4_layout(int64_t M, int64_t N, int64_t K, int split) {
  W4Ws w{};
  w.plan = split == 0 ? w8::plan_w4a8_gemm(M, N, K, cu_count()) : w8::plan_w4a8_gemm_split(M, N, split);
  size_t off = 0;
  w.q = off;    off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;   off = up(off + 4 * static_cast<size_t>(M));
  w.cnt = off;  off = up(off + 4 * static_cast<size_t>(w.plan.counters()));
  w.part = off; off = up(off + w.plan.partial_bytes());
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

static w8_status w4_checks(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4,
                           int64_t N, void* Y, int y_dt) {
  W8_REQUIRE(X && Wq4 && sw4 && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(x_dt == W8_DT_F16 || x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  W8_REQUIRE(y_dt == W8_DT_BF16 || y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED,
             "Y must be bf16, f16 or f32");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(K % 128 == 0, W8_ERR_UNSUPPORTED, "K must be a multiple of 128 (the int4 group), got %lld",
             (long long)K);
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(M * K < (int64_t(1) << 32) && N * (K / 2) < (int64_t(1) << 32), W8_ERR_UNSUPPORTED,
             "X codes and packed weights must each be smaller than 4 GiB");
  W8_REQUIRE(aligned16(X) && aligned16(Wq4) && aligned16(sw4) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  return W8_OK;
}

static w8_status w4_run(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4,
                        int64_t N, void* Y, int y_dt, const W4Ws& L, void* workspace, size_t workspace_bytes,
                        void* stream, const char* what) {
  if (w8_status st = check_ws(workspace, workspace_bytes, L.total); st != W8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* q = at<int8_t>(workspace, L.q);
  float* sx = at<float>(workspace, L.sx);
  mark(0, s);
  // per-token absmax int8 codes: the int8 row pass with no outlier columns
  w8::launch_int8_rows(X, x_dt == W8_DT_BF16, M, (int)K, 0x7F80u, q, sx, nullptr, w8::kProdNone, w8::ProdArgs{}, s);
  mark(1, s);
  mark(2, s);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_w4a8_gemm(q, Wq4, M, N, K, sx, sw4, Y, ydt, L.plan, at<float>(workspace, L.part),
                       at<int>(workspace, L.cnt), s);
  mark(3, s);
  return check_launch(what);
}

size_t w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return w4_layout(M, N, K, 0).total;
}

w8_status w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4, int64_t N,
                      void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w4_checks(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt); st != W8_OK) return st;
  return w4_run(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt, w4_layout(M, N, K, 0), workspace, workspace_bytes, stream,
                "w4a8_linear");
}

// ---- parity exports ---------------------------------------------------------

size_t w8dbg_w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  return w4_layout(M, N, K, split).total;
}

w8_status w8dbg_w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4,
                            int64_t N, int split, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (w8_status st = w4_checks(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt); st != W8_OK) return st;
  W8_REQUIRE(split >= 0, W8_ERR_INVALID_ARGUMENT, "split must be >= 0");
  W8_REQUIRE(split <= K / 128, W8_ERR_UNSUPPORTED, "split %d needs at most K / 128 slices", split);
  return w4_run(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt, w4_layout(M, N, K, split), workspace, workspace_bytes, stream,
                "w8dbg_w4a8_linear");
}


size_t w8dbg_fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  return w16_layout(w16_plan(M, N, K, split, tile)).total;
}

w8_status w8dbg_fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8,
                                 const float* sw, int64_t N, int split, int tile, void* Y, int y_dt,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w16_checks(X, x_dt, M, K, Wq8, sw, N, Y, y_dt); st != W8_OK) return st;
  W8_REQUIRE(split >= 0, W8_ERR_INVALID_ARGUMENT, "split must be >= 0");
  W8_REQUIRE(tile == 0 || tile == 128 || tile == 256, W8_ERR_INVALID_ARGUMENT, "tile must be 0, 128 or 256");
  W8_REQUIRE(split <= K / 64, W8_ERR_UNSUPPORTED, "split %d needs at most K / 64 slices", split);
  return w16_run(X, M, K, Wq8, sw, N, Y, y_dt, w16_layout(w16_plan(M, N, K, split, tile)), workspace,
                 workspace_bytes, stream, "w8dbg_fp8_w8a16_linear");
}


size_t w8dbg_int8_quantize_activations_workspace_size(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return up(static_cast<size_t>(K)) + up(4 * static_cast<size_t>(M));
}

w8_status w8dbg_int8_quantize_activations(const void* X, int x_dt, int64_t M, int64_t K,
                                          const w8_producer* producer, float threshold, int8_t* q, float* sx,
                                          int32_t* outlier_idx, int32_t* n_outliers, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  if (w8_status st = int8_common_checks(X, x_dt, M, K, threshold); st != W8_OK) return st;
  W8_REQUIRE(q && sx && outlier_idx && n_outliers, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(aligned16(q) && aligned16(sx), W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  int kind = 0;
  w8::ProdArgs pa{};
  if (w8_status st = producer_args(producer, K, &kind, &pa); st != W8_OK) return st;
  const size_t need = w8dbg_int8_quantize_activations_workspace_size(M, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, need); st != W8_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = x_dt == W8_DT_BF16;
  uint8_t* flags = at<uint8_t>(workspace, 0);
  pa.rstd = at<float>(workspace, up(static_cast<size_t>(K)));
  const uint32_t tb = threshold_bits(threshold, bf);
  w8::launch_int8_rows(X, bf, M, (int)K, tb, q, sx, flags, kind, pa, s);
  w8::launch_outlier_fixup(X, bf, M, (int)K, tb, flags, q, sx, outlier_idx, n_outliers, nullptr, nullptr, 0, nullptr,
                           kind, pa, s);
  w8::launch_clear_words(reinterpret_cast<uint32_t*>(flags), static_cast<int>(K / 4), s);
  return check_launch("w8dbg_int8_quantize_activations");
}

size_t w8dbg_int8_gemm_i32_workspace_size(int64_t M, int64_t N, int64_t K, int tail, int split) {
  if (M < 1 || N < 1 || K < 1 || tail < 0 || tail > 2 || split < 1) return 0;
  return gemm_layout(M, N, K, tail, split).total;
}

w8_status w8dbg_int8_gemm_i32(const int8_t* q, const int8_t* Wq, int64_t M, int64_t N, int64_t K, int tail,
                              int split, int32_t* acc, void* workspace, size_t workspace_bytes, void* stream) {
  W8_REQUIRE(q && Wq && acc, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (w8_status st = check_mk(M, K, W8_INT8_MAX_K); st != W8_OK) return st;
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(tail >= 0 && tail <= 2 && split >= 1, W8_ERR_INVALID_ARGUMENT, "tail must be 0..2 and split >= 1");
  W8_REQUIRE(tail == 0 || (tail == 1 && split == 1) || (K % 64 == 0 && split <= K / 64), W8_ERR_UNSUPPORTED,
             "this tail treatment needs K %% 64 == 0 and split <= K / 64");
  W8_REQUIRE(aligned16(q) && aligned16(Wq) && aligned16(acc), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  const GemmWs L = gemm_layout(M, N, K, tail, split);
  if (L.total > 0) {
    if (w8_status st = check_ws(workspace, workspace_bytes, L.total); st != W8_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* cnt = L.total > 0 ? at<int>(workspace, L.cnt) : nullptr;
  int* part = L.total > 0 ? at<int>(workspace, L.part) : nullptr;
  w8::launch_int8_gemm(q, Wq, M, N, K, nullptr, nullptr, nullptr, nullptr, nullptr, true, nullptr, acc, 0, L.plan,
                       part, cnt,
                       nullptr, 0, s);
  return check_launch("w8dbg_int8_gemm_i32");
}

size_t w8dbg_fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  const w8::GemmPlan plan = fp8_debug_plan(M, N, K, split, tile);
  return up(4 * static_cast<size_t>(plan.counters())) + up(plan.partial_bytes());
}

w8_status w8dbg_fp8_gemm(const uint8_t* xq, const float* sx, const uint8_t* Wq8, const float* sw, int64_t M,
                         int64_t N, int64_t K, int split, int tile, void* Y, int y_dt, void* workspace,
                         size_t workspace_bytes, void* stream) {
  W8_REQUIRE(xq && sx && Wq8 && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(y_dt == W8_DT_BF16 || y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED,
             "Y must be bf16, f16 or f32");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(split >= 0, W8_ERR_INVALID_ARGUMENT, "split must be >= 0");
  W8_REQUIRE(tile == 0 || tile == 128 || tile == 256, W8_ERR_INVALID_ARGUMENT, "tile must be 0, 128 or 256");
  W8_REQUIRE(split == 0 || tile == 0 || K % 64 == 0, W8_ERR_UNSUPPORTED, "a tile size needs K %% 64 == 0");
  W8_REQUIRE(split <= 1 || (K % 64 == 0 && split <= K / 64), W8_ERR_UNSUPPORTED,
             "split %d needs K %% 64 == 0 and at most K / 64 slices", split);
  W8_REQUIRE(aligned16(xq) && aligned16(sx) && aligned16(Wq8) && aligned16(sw) && aligned16(Y),
             W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  const w8::GemmPlan plan = fp8_debug_plan(M, N, K, split, tile);
  const size_t cnt_bytes = up(4 * static_cast<size_t>(plan.counters()));
  const size_t need = cnt_bytes + up(plan.partial_bytes());
  if (need > 0) {
    if (w8_status st = check_ws(workspace, workspace_bytes, need); st != W8_OK) return st;
  }
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_fp8_gemm(xq, Wq8, M, N, K, sx, sw, Y, ydt, plan, need > 0 ? at<float>(workspace, cnt_bytes) : nullptr,
                      need > 0 ? at<int>(workspace, 0) : nullptr, static_cast<hipStream_t>(stream));
  return check_launch("w8dbg_fp8_gemm");
}

w8_status w8dbg_produce(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer, void* X,
                        void* stream) {
  W8_REQUIRE(H && X, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(h_dt == W8_DT_F16 || h_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "H must be f16 or bf16");
  if (w8_status st = check_mk(M, K, W8_INT8_MAX_K); st != W8_OK) return st;
  W8_REQUIRE(aligned16(H) && aligned16(X), W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  int kind = 0;
  w8::ProdArgs pa{};
  if (w8_status st = producer_args(producer, K, &kind, &pa); st != W8_OK) return st;
  w8::launch_produce(H, h_dt == W8_DT_BF16, M, (int)K, kind, pa, X, static_cast<hipStream_t>(stream));
  return check_launch("w8dbg_produce");
}

w8_status w8dbg_fp8_quantize_activations(const void* X, int x_dt, int64_t M, int64_t K, const float* act_scale,
                                         uint8_t* xq, float* sx, void* stream) {
  W8_REQUIRE(X && xq && sx, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(x_dt == W8_DT_F16 || x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(aligned16(X) && aligned16(xq) && aligned16(sx), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  w8::launch_fp8_rows(X, x_dt == W8_DT_BF16, M, (int)K, act_scale, xq, sx, act_scale ? 1 : 0,
                      static_cast<hipStream_t>(stream));
  return check_launch("w8dbg_fp8_quantize_activations");
}

}  // extern "C"
