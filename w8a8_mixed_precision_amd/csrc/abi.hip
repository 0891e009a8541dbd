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

// Compute units of the current device (cached per device); the GEMM plans
// depend on it. Threads may race to fill an entry; they all store the same
// value, and the atomics keep that defined.
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

// Every workspace starts with the same two regions, at fixed offsets whatever
// the shape of the call, so that one workspace can serve calls of different
// shapes one after another:
//  * kCntCap split-K arrival counters, zero between calls (each tile's last
//    slice resets its counter);
//  * the outlier-column flag words of the int8 linears, one per column up to
//    W8_INT8_MAX_K. A call marks its outlier columns with a stamp of its own
//    (never 0), so flags are never cleared and a flag left by an earlier or a
//    failed call does not match.
// Shape-dependent regions follow. Sizes are planned for kPlanCus compute
// units (MI355X); a device whose GEMM plan needs more split-K partials or
// counters than a workspace holds runs the plan without K-slicing instead.
using w8::kCntBytes;
using w8::kCntCap;
using w8::kFlagBytes;
using w8::kFront;
static_assert(kFlagBytes >= 4 * static_cast<size_t>(W8_INT8_MAX_K), "a flag word per column");
static_assert(kFront % kAlign == 0, "aligned front");
constexpr int kPlanCus = 256;

// The next call stamp (process-wide, thread-safe, skips 0). A stale flag can
// match again only after 2^32 - 1 further int8 calls.
uint32_t next_stamp() {
  static std::atomic<uint32_t> counter{0};
  uint32_t s = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  while (s == 0) s = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  return s;
}

// The plan when it fits the workspace's partials and the counter region,
// else the same grid without K-slicing (`whole`).
w8::GemmPlan fit_plan(const w8::GemmPlan& p, size_t part_bytes_avail, const w8::GemmPlan& whole) {
  if (p.counters() <= kCntCap && p.partial_bytes() <= part_bytes_avail) return p;
  return whole;
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

// Workspace layout of int8_mixed_linear (offsets from the 256-aligned base):
// the common front (counters, flags), then nO, the outlier list O [K], the
// codes q [M,K], sx [M], the RMSNorm rstd [M] of the fused path, the staged
// outlier operands XO [M, kOutCap] and WO [N, kOutCap], and the split-K
// partials of the plan.
struct Int8Ws {
  size_t cnt, flags, nO, O, q, sx, rstd, XO, WO, part, base;
};

Int8Ws int8_layout(int64_t M, int64_t N, int64_t K) {
  Int8Ws w{};
  size_t off = 0;
  w.cnt = off;   off += kCntBytes;
  w.flags = off; off += kFlagBytes;
  w.nO = off;    off = up(off + 4);
  w.O = off;     off = up(off + 4 * static_cast<size_t>(K));
  w.q = off;     off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;    off = up(off + 4 * static_cast<size_t>(M));
  w.rstd = off;  off = up(off + 4 * static_cast<size_t>(M));
  w.XO = off;    off = up(off + 2 * static_cast<size_t>(M) * w8::kOutCap);
  w.WO = off;    off = up(off + 2 * static_cast<size_t>(N) * w8::kOutCap);
  w.part = off;
  w.base = off;
  return w;
}

size_t int8_ws_size(int64_t M, int64_t N, int64_t K) {
  const w8::GemmPlan p = w8::plan_int8_gemm(M, N, K, kPlanCus);
  const size_t part = p.counters() <= kCntCap ? p.partial_bytes() : 0;
  return int8_layout(M, N, K).base + up(part);
}

// The int8 GEMM plan of this device that fits `avail` bytes of partials.
w8::GemmPlan int8_plan(int64_t M, int64_t N, int64_t K, size_t avail) {
  return fit_plan(w8::plan_int8_gemm(M, N, K, cu_count()), avail,
                  w8::plan_int8_gemm_forced(M, N, cu_count(), true, 1));
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

// Grid of the int8 GEMM parity export. tail: 0 the linear's own plan; 1
// leftover tiles as `split` 256x256 slices (split 1: every tile whole); 2 as
// `split` slices of 128x128 quarters. Workspace: the front, then partials.
w8::GemmPlan int8_debug_plan(int64_t M, int64_t N, int64_t K, int tail, int split, int cus) {
  if (tail == 3) return w8::plan_int8_gemm_streamk(M, N, cus);
  return tail == 0 ? w8::plan_int8_gemm(M, N, K, cus) : w8::plan_int8_gemm_forced(M, N, cus, tail == 2, split);
}

// Workspace layout of fp8_w8a8_linear: the front, codes [M,K], scales [M],
// split-K partials.
struct Fp8Ws {
  size_t xq, sx, part, base;
};

Fp8Ws fp8_layout(int64_t M, int64_t K) {
  Fp8Ws w{};
  size_t off = kFront;
  w.xq = off;   off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;   off = up(off + 4 * static_cast<size_t>(M));
  w.part = off;
  w.base = off;
  return w;
}

size_t plan_part(const w8::GemmPlan& p) { return p.counters() <= kCntCap ? up(p.partial_bytes()) : 0; }

w8::GemmPlan fp8_plan(int64_t M, int64_t N, int64_t K, size_t avail) {
  const w8::GemmPlan p = w8::plan_fp8_gemm(M, N, K, cu_count());
  return fit_plan(p, avail, w8::plan_fp8_gemm_split(M, N, 1, p.bm));
}

// Grid of the FP8 GEMM parity export: the linear's own plan (split 0) or the
// given block size and K-slicing.
w8::GemmPlan fp8_debug_plan(int64_t M, int64_t N, int64_t K, int split, int tile, int cus) {
  if (split == 0) return w8::plan_fp8_gemm(M, N, K, cus);
  if (tile == 129 || tile == 192) return w8::plan_fp8_gemm_rect(M, N, split, tile == 192 ? 192 : 128);
  return w8::plan_fp8_gemm_split(M, N, split, tile == 128 ? 128 : 256);
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

// Records event `b` (0..3) of a parity-export call on its stream: events[0]
// before the first kernel, then one after each stage (row pass, fix-up,
// GEMM). Product calls pass no events.
void mark(void* const* events, int b, hipStream_t s) {
  if (events && events[b]) (void)hipEventRecord(static_cast<hipEvent_t>(events[b]), s);
}

}  // namespace

extern "C" {

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
    w8::launch_int8_rows(W, bf, N, (int)K, 0x7F80u, static_cast<int8_t*>(Wq), sw, nullptr, 0u, w8::kProdNone,
                         w8::ProdArgs{}, s);
  else if (fmt == W8_Q_INT4_G128)
    w8::launch_int4_weights(W, bf, N, (int)K, static_cast<uint8_t*>(Wq), sw, s);
  else
    w8::launch_fp8_rows(W, bf, N, (int)K, nullptr, static_cast<uint8_t*>(Wq), sw, 2, s);
  return check_launch("quantize_weight_rowwise");
}

size_t int8_mixed_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return int8_ws_size(M, N, K);
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

// The three kernels of one int8 call on a validated workspace. `events`: the
// parity export's stage events (NULL for product calls).
static w8_status int8_linear_impl(const void* X, int x_dt, int64_t M, int64_t K, const w8_producer* producer,
                                  const int8_t* Wq, const float* sw, const float* bias, int64_t N, float threshold,
                                  void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events, const char* what, size_t need = 0,
                                  long long* timeline = nullptr, const w8::GemmPlan* forced = nullptr) {
  if (w8_status st = int8_common_checks(X, x_dt, M, K, threshold); st != W8_OK) return st;
  W8_REQUIRE(Wq && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED, "Y must be f16 or f32");
  W8_REQUIRE(aligned16(Wq) && aligned16(sw) && aligned16(Y) && aligned16(bias), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  int kind = 0;
  w8::ProdArgs pa{};
  if (w8_status st = producer_args(producer, K, &kind, &pa); st != W8_OK) return st;
  const Int8Ws L = int8_layout(M, N, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, need ? need : int8_ws_size(M, N, K)); st != W8_OK)
    return st;
  const w8::GemmPlan plan = forced ? *forced : int8_plan(M, N, K, workspace_bytes - L.base);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = x_dt == W8_DT_BF16;
  int8_t* q = at<int8_t>(workspace, L.q);
  float* sx = at<float>(workspace, L.sx);
  uint32_t* flags = at<uint32_t>(workspace, L.flags);
  int* nO = at<int>(workspace, L.nO);
  int* O = at<int>(workspace, L.O);
  uint16_t* XO = at<uint16_t>(workspace, L.XO);
  uint16_t* WO = at<uint16_t>(workspace, L.WO);
  int* cnt = at<int>(workspace, L.cnt);
  int* part = at<int>(workspace, L.part);
  pa.rstd = at<float>(workspace, L.rstd);
  const uint32_t stamp = next_stamp();
  const w8::SideSrc src{static_cast<const uint16_t*>(X), Wq, O, static_cast<int>(K), kind, pa};

  mark(events, 0, s);
  const uint32_t tb = threshold_bits(threshold, bf);
  w8::launch_int8_rows(X, bf, M, (int)K, tb, q, sx, flags, stamp, kind, pa, s);
  mark(events, 1, s);
  w8::launch_outlier_fixup(X, bf, M, (int)K, tb, flags, stamp, q, sx, O, nO, XO, Wq, N, WO, kind, pa, s);
  mark(events, 2, s);
  w8::launch_int8_gemm(q, Wq, M, N, K, sx, sw, nO, XO, WO, bf, bias, Y, y_dt == W8_DT_F16 ? 1 : 2, plan, part, cnt,
                       src, s, timeline);
  mark(events, 3, s);
  return check_launch(what);
}

w8_status int8_mixed_linear(const void* X, int x_dt, int64_t M, int64_t K, const int8_t* Wq, const float* sw,
                            int64_t N, float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return int8_linear_impl(X, x_dt, M, K, nullptr, Wq, sw, nullptr, N, threshold, Y, y_dt, workspace,
                          workspace_bytes, stream, nullptr, "int8_mixed_linear");
}

w8_status int8_mixed_linear_fused(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                  const int8_t* Wq, const float* sw, const float* bias, int64_t N, float threshold,
                                  void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  return int8_linear_impl(H, h_dt, M, K, producer, Wq, sw, bias, N, threshold, Y, y_dt, workspace, workspace_bytes,
                          stream, nullptr, "int8_mixed_linear_fused");
}

}  // extern "C"

// Scratch of int8_mixed_linear_noalloc: its workspace, in the library's own
// device memory. Each device holds its own copy from the time the library's
// code is loaded on it until the process ends, zero at load. In host code the
// name is only a stand-in: the address a kernel can use comes from
// hipGetSymbolAddress, once per device, kept in g_scratch_ptr.
static constexpr size_t kNoAllocBytes = size_t{96} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {

std::atomic<void*> g_scratch_ptr[64];

// The device address of this device's scratch (null if it cannot be found).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);   // racing threads store the same address
  return p;
}

}  // namespace

extern "C" {

w8_status int8_mixed_linear_noalloc(const void* X, int x_dt, int64_t M, int64_t K, const int8_t* Wq, const float* sw,
                                    int64_t N, float threshold, void* Y, int y_dt, void* stream) {
  // every argument check of int8_mixed_linear, before the device is touched
  if (w8_status st = int8_common_checks(X, x_dt, M, K, threshold); st != W8_OK) return st;
  W8_REQUIRE(Wq && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED, "Y must be f16 or f32");
  W8_REQUIRE(aligned16(Wq) && aligned16(sw) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  const size_t need = int8_layout(M, N, K).base;
  W8_REQUIRE(need <= kNoAllocBytes, W8_ERR_UNSUPPORTED,
             "M=%lld N=%lld K=%lld needs %zu bytes of scratch; int8_mixed_linear_noalloc has %zu (use "
             "int8_mixed_linear with a workspace)", (long long)M, (long long)N, (long long)K, need, kNoAllocBytes);
  void* ws = scratch_ptr();
  W8_REQUIRE(ws != nullptr, W8_ERR_HIP, "hipGetSymbolAddress of the no-allocation scratch failed");
  return int8_linear_impl(X, x_dt, M, K, nullptr, Wq, sw, nullptr, N, threshold, Y, y_dt, ws, kNoAllocBytes, stream,
                          nullptr, "int8_mixed_linear_noalloc", need);
}

size_t fp8_w8a8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return fp8_layout(M, K).base + plan_part(w8::plan_fp8_gemm(M, N, K, kPlanCus));
}

static w8_status fp8_impl(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                          int64_t N, const float* act_scale, void* Y, int y_dt, void* workspace,
                          size_t workspace_bytes, void* stream, void* const* events, const char* what) {
  W8_REQUIRE(X && Wq8 && sw && Y, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(x_dt == W8_DT_F16 || x_dt == W8_DT_BF16, W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  W8_REQUIRE(y_dt == W8_DT_BF16 || y_dt == W8_DT_F16 || y_dt == W8_DT_F32, W8_ERR_UNSUPPORTED,
             "Y must be bf16, f16 or f32");
  if (w8_status st = check_mk(M, K, 65536); st != W8_OK) return st;
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(aligned16(X) && aligned16(Wq8) && aligned16(sw) && aligned16(Y), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  const Fp8Ws L = fp8_layout(M, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, fp8_w8a8_linear_workspace_size(M, N, K)); st != W8_OK)
    return st;
  const w8::GemmPlan plan = fp8_plan(M, N, K, workspace_bytes - L.base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* xq = at<uint8_t>(workspace, L.xq);
  float* sx = at<float>(workspace, L.sx);
  mark(events, 0, s);
  w8::launch_fp8_rows(X, x_dt == W8_DT_BF16, M, (int)K, act_scale, xq, sx, act_scale ? 1 : 0, s);
  mark(events, 1, s);
  mark(events, 2, s);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_fp8_gemm(xq, Wq8, M, N, K, sx, sw, Y, ydt, plan, at<float>(workspace, L.part), at<int>(workspace, 0), s);
  mark(events, 3, s);
  return check_launch(what);
}

w8_status fp8_w8a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                          int64_t N, const float* act_scale, void* Y, int y_dt, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return fp8_impl(X, x_dt, M, K, Wq8, sw, N, act_scale, Y, y_dt, workspace, workspace_bytes, stream, nullptr,
                  "fp8_w8a8_linear");
}

}  // extern "C"

namespace {

// FP8 weight-only: the front, then the plan's split-K partials.
w8::GemmPlan w16_plan(int64_t M, int64_t N, int64_t K, int split, int tile, int cus) {
  return split == 0 ? w8::plan_w8a16_gemm(M, N, K, cus)
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

// `plan`: the grid to run; `whole`: the same grid unsliced, taken when the
// plan's partials do not fit the workspace.
static w8_status w16_run(const void* X, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw, int64_t N,
                         void* Y, int y_dt, const w8::GemmPlan& want, const w8::GemmPlan& whole, void* workspace,
                         size_t workspace_bytes, void* stream, const char* what) {
  if (w8_status st = check_ws(workspace, workspace_bytes, kFront); st != W8_OK) return st;
  const w8::GemmPlan plan = fit_plan(want, workspace_bytes - kFront, whole);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_w8a16_gemm(static_cast<const uint16_t*>(X), Wq8, M, N, K, sw, Y, ydt, plan, at<float>(workspace, kFront),
                        at<int>(workspace, 0), s);
  return check_launch(what);
}

size_t fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return kFront + plan_part(w16_plan(M, N, K, 0, 0, kPlanCus));
}

w8_status fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8, const float* sw,
                           int64_t N, void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w16_checks(X, x_dt, M, K, Wq8, sw, N, Y, y_dt); st != W8_OK) return st;
  if (w8_status st = check_ws(workspace, workspace_bytes, fp8_w8a16_linear_workspace_size(M, N, K)); st != W8_OK)
    return st;
  const w8::GemmPlan p = w16_plan(M, N, K, 0, 0, cu_count());
  return w16_run(X, M, K, Wq8, sw, N, Y, y_dt, p, w8::plan_w8a16_gemm_split(M, N, 1, p.bm), workspace,
                 workspace_bytes, stream, "fp8_w8a16_linear");
}

}  // extern "C"

namespace {

// W4A8: the front, activation codes [M,K], row scales [M], split-K partials.
struct W4Ws {
  size_t q, sx, part, base;
};

W4Ws w4_layout(int64_t M, int64_t K) {
  W4Ws w{};
  size_t off = kFront;
  w.q = off;    off = up(off + static_cast<size_t>(M) * K);
  w.sx = off;   off = up(off + 4 * static_cast<size_t>(M));
  w.part = off;
  w.base = off;
  return w;
}

w8::GemmPlan w4_plan(int64_t M, int64_t N, int64_t K, int split, int cus) {
  return split == 0 ? w8::plan_w4a8_gemm(M, N, K, cus) : w8::plan_w4a8_gemm_split(M, N, split);
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
                        int64_t N, void* Y, int y_dt, const w8::GemmPlan& want, void* workspace,
                        size_t workspace_bytes, void* stream, const char* what) {
  const W4Ws L = w4_layout(M, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, L.base); st != W8_OK) return st;
  const w8::GemmPlan plan = fit_plan(want, workspace_bytes - L.base, w8::plan_w4a8_gemm_split(M, N, 1));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* q = at<int8_t>(workspace, L.q);
  float* sx = at<float>(workspace, L.sx);
  // per-token absmax int8 codes: the int8 row pass with no outlier columns
  w8::launch_int8_rows(X, x_dt == W8_DT_BF16, M, (int)K, 0x7F80u, q, sx, nullptr, 0u, w8::kProdNone, w8::ProdArgs{},
                       s);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_w4a8_gemm(q, Wq4, M, N, K, sx, sw4, Y, ydt, plan, at<float>(workspace, L.part), at<int>(workspace, 0), s);
  return check_launch(what);
}

size_t w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  return w4_layout(M, K).base + plan_part(w4_plan(M, N, K, 0, kPlanCus));
}

w8_status w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4, int64_t N,
                      void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w4_checks(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt); st != W8_OK) return st;
  if (w8_status st = check_ws(workspace, workspace_bytes, w4a8_linear_workspace_size(M, N, K)); st != W8_OK)
    return st;
  return w4_run(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt, w4_plan(M, N, K, 0, cu_count()), workspace, workspace_bytes,
                stream, "w4a8_linear");
}

// ---- parity exports ---------------------------------------------------------

w8_status w8dbg_int8_mixed_linear_events(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                         const int8_t* Wq, const float* sw, const float* bias, int64_t N,
                                         float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                                         void* const* events, void* stream) {
  return int8_linear_impl(H, h_dt, M, K, producer, Wq, sw, bias, N, threshold, Y, y_dt, workspace, workspace_bytes,
                          stream, events, "w8dbg_int8_mixed_linear_events");
}

w8_status w8dbg_int8_gemm_timeline(const void* X, int x_dt, int64_t M, int64_t K, const int8_t* Wq, const float* sw,
                                    int64_t N, float threshold, void* Y, int y_dt, void* workspace,
                                    size_t workspace_bytes, long long* stamps, size_t stamps_len, int* grid,
                                    void* stream) {
  W8_REQUIRE(grid, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(M >= 1 && N >= 1 && K >= 1, W8_ERR_INVALID_ARGUMENT, "M, N, K must be >= 1");
  const Int8Ws L = int8_layout(M, N, K);
  W8_REQUIRE(workspace_bytes >= L.base, W8_ERR_WORKSPACE, "workspace smaller than its fixed regions");
  const w8::GemmPlan plan = int8_plan(M, N, K, workspace_bytes - L.base);
  grid[0] = plan.grid();
  grid[1] = plan.dp_tiles;
  grid[2] = K % 64 == 0 ? 1 : 0;                // the timeline is recorded by the 64-byte-step kernel only
  grid[3] = plan.streamk ? 2 : (plan.small ? 1 : 0);
  if (!stamps) return ok();
  W8_REQUIRE(grid[2] == 1, W8_ERR_UNSUPPORTED, "the timeline needs K %% 64 == 0");
  W8_REQUIRE(stamps_len >= 8 * static_cast<size_t>(grid[0]), W8_ERR_INVALID_ARGUMENT,
             "stamps holds %zu words; the launch needs 8 per block (%d blocks)", stamps_len, grid[0]);
  return int8_linear_impl(X, x_dt, M, K, nullptr, Wq, sw, nullptr, N, threshold, Y, y_dt, workspace, workspace_bytes,
                          stream, nullptr, "w8dbg_int8_gemm_timeline", 0, stamps);
}

size_t w8dbg_int8_mixed_linear_plan_workspace_size(int64_t M, int64_t N, int64_t K, int cus) {
  if (M < 1 || N < 1 || K < 1 || cus < 1 || cus > 4096) return 0;
  return int8_layout(M, N, K).base + plan_part(w8::plan_int8_gemm(M, N, K, cus));
}

w8_status w8dbg_int8_mixed_linear_plan(const void* H, int h_dt, int64_t M, int64_t K, const w8_producer* producer,
                                       const int8_t* Wq, const float* sw, const float* bias, int64_t N,
                                       float threshold, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                                       int cus, void* stream) {
  W8_REQUIRE(M >= 1 && N >= 1 && K >= 1, W8_ERR_INVALID_ARGUMENT, "M, N, K must be >= 1");
  W8_REQUIRE(cus >= 1 && cus <= 4096, W8_ERR_INVALID_ARGUMENT, "cus must be in [1, 4096]");
  const w8::GemmPlan plan = w8::plan_int8_gemm(M, N, K, cus);
  W8_REQUIRE(plan.counters() <= kCntCap, W8_ERR_UNSUPPORTED, "too many split tiles (%d > %d)", plan.counters(),
             kCntCap);
  return int8_linear_impl(H, h_dt, M, K, producer, Wq, sw, bias, N, threshold, Y, y_dt, workspace, workspace_bytes,
                          stream, nullptr, "w8dbg_int8_mixed_linear_plan",
                          w8dbg_int8_mixed_linear_plan_workspace_size(M, N, K, cus), nullptr, &plan);
}

w8_status w8dbg_fp8_w8a8_linear_events(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8,
                                       const float* sw, int64_t N, const float* act_scale, void* Y, int y_dt,
                                       void* workspace, size_t workspace_bytes, void* const* events, void* stream) {
  return fp8_impl(X, x_dt, M, K, Wq8, sw, N, act_scale, Y, y_dt, workspace, workspace_bytes, stream, events,
                  "w8dbg_fp8_w8a8_linear_events");
}

w8_status w8dbg_int8_workspace_layout(int64_t M, int64_t N, int64_t K, size_t* offsets) {
  W8_REQUIRE(offsets, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  W8_REQUIRE(M >= 1 && N >= 1 && K >= 1, W8_ERR_INVALID_ARGUMENT, "M, N, K must be >= 1");
  const Int8Ws L = int8_layout(M, N, K);
  const size_t v[11] = {L.cnt, L.flags, L.nO, L.O, L.q, L.sx, L.rstd, L.XO, L.WO, L.part,
                        static_cast<size_t>(w8::kOutCap)};
  std::memcpy(offsets, v, sizeof v);
  return ok();
}

size_t w8dbg_w4a8_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  return w4_layout(M, K).base + up(w4_plan(M, N, K, split, cu_count()).partial_bytes());
}

w8_status w8dbg_w4a8_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq4, const float* sw4,
                            int64_t N, int split, void* Y, int y_dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (w8_status st = w4_checks(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt); st != W8_OK) return st;
  W8_REQUIRE(split >= 0, W8_ERR_INVALID_ARGUMENT, "split must be >= 0");
  W8_REQUIRE(split <= K / 128, W8_ERR_UNSUPPORTED, "split %d needs at most K / 128 slices", split);
  const w8::GemmPlan p = w4_plan(M, N, K, split, cu_count());
  W8_REQUIRE(p.counters() <= kCntCap, W8_ERR_UNSUPPORTED, "too many split tiles (%d > %d)", p.counters(), kCntCap);
  const W4Ws L = w4_layout(M, K);
  if (w8_status st = check_ws(workspace, workspace_bytes, L.base + up(p.partial_bytes())); st != W8_OK) return st;
  return w4_run(X, x_dt, M, K, Wq4, sw4, N, Y, y_dt, p, workspace, workspace_bytes, stream, "w8dbg_w4a8_linear");
}

size_t w8dbg_fp8_w8a16_linear_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  return kFront + up(w16_plan(M, N, K, split, tile, cu_count()).partial_bytes());
}

w8_status w8dbg_fp8_w8a16_linear(const void* X, int x_dt, int64_t M, int64_t K, const uint8_t* Wq8,
                                 const float* sw, int64_t N, int split, int tile, void* Y, int y_dt,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (w8_status st = w16_checks(X, x_dt, M, K, Wq8, sw, N, Y, y_dt); st != W8_OK) return st;
  W8_REQUIRE(split >= 0, W8_ERR_INVALID_ARGUMENT, "split must be >= 0");
  W8_REQUIRE(tile == 0 || tile == 128 || tile == 256, W8_ERR_INVALID_ARGUMENT, "tile must be 0, 128 or 256");
  W8_REQUIRE(split <= K / 64, W8_ERR_UNSUPPORTED, "split %d needs at most K / 64 slices", split);
  const w8::GemmPlan p = w16_plan(M, N, K, split, tile, cu_count());
  W8_REQUIRE(p.counters() <= kCntCap, W8_ERR_UNSUPPORTED, "too many split tiles (%d > %d)", p.counters(), kCntCap);
  if (w8_status st = check_ws(workspace, workspace_bytes, kFront + up(p.partial_bytes())); st != W8_OK) return st;
  return w16_run(X, M, K, Wq8, sw, N, Y, y_dt, p, p, workspace, workspace_bytes, stream, "w8dbg_fp8_w8a16_linear");
}

size_t w8dbg_int8_quantize_activations_workspace_size(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return kFront + up(4 * static_cast<size_t>(M));
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
  uint32_t* flags = at<uint32_t>(workspace, kCntBytes);
  pa.rstd = at<float>(workspace, kFront);
  const uint32_t stamp = next_stamp();
  const uint32_t tb = threshold_bits(threshold, bf);
  w8::launch_int8_rows(X, bf, M, (int)K, tb, q, sx, flags, stamp, kind, pa, s);
  w8::launch_outlier_fixup(X, bf, M, (int)K, tb, flags, stamp, q, sx, outlier_idx, n_outliers, nullptr, nullptr, 0,
                           nullptr, kind, pa, s);
  return check_launch("w8dbg_int8_quantize_activations");
}

size_t w8dbg_int8_gemm_i32_workspace_size(int64_t M, int64_t N, int64_t K, int tail, int split) {
  if (M < 1 || N < 1 || K < 1 || tail < 0 || tail > 3 || split < 1) return 0;
  return kFront + up(int8_debug_plan(M, N, K, tail, split, cu_count()).partial_bytes());
}

w8_status w8dbg_int8_gemm_i32(const int8_t* q, const int8_t* Wq, int64_t M, int64_t N, int64_t K, int tail,
                              int split, int32_t* acc, void* workspace, size_t workspace_bytes, void* stream) {
  W8_REQUIRE(q && Wq && acc, W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (w8_status st = check_mk(M, K, W8_INT8_MAX_K); st != W8_OK) return st;
  W8_REQUIRE(N >= 1 && N <= kMaxDim, W8_ERR_INVALID_ARGUMENT, "N must be in [1, 2^31)");
  W8_REQUIRE(tail >= 0 && tail <= 3 && split >= 1, W8_ERR_INVALID_ARGUMENT, "tail must be 0..3 and split >= 1");
  W8_REQUIRE(tail != 3 || split == 1, W8_ERR_INVALID_ARGUMENT, "stream-K (tail 3) takes split = 1");
  W8_REQUIRE(tail == 0 || (tail == 1 && split == 1) || (K % 64 == 0 && split <= K / 64), W8_ERR_UNSUPPORTED,
             "this tail treatment needs K %% 64 == 0 and split <= K / 64");
  W8_REQUIRE(aligned16(q) && aligned16(Wq) && aligned16(acc), W8_ERR_INVALID_ARGUMENT,
             "pointers must be 16-byte aligned");
  const w8::GemmPlan plan = int8_debug_plan(M, N, K, tail, split, cu_count());
  W8_REQUIRE(plan.counters() <= kCntCap, W8_ERR_UNSUPPORTED, "too many split tiles (%d > %d)", plan.counters(),
             kCntCap);
  if (w8_status st = check_ws(workspace, workspace_bytes, kFront + up(plan.partial_bytes())); st != W8_OK) return st;
  const w8::SideSrc none{nullptr, nullptr, nullptr, 0, w8::kProdNone, w8::ProdArgs{}};
  w8::launch_int8_gemm(q, Wq, M, N, K, nullptr, nullptr, nullptr, nullptr, nullptr, true, nullptr, acc, 0, plan,
                       at<int>(workspace, kFront), at<int>(workspace, 0), none, static_cast<hipStream_t>(stream));
  return check_launch("w8dbg_int8_gemm_i32");
}

size_t w8dbg_fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  return kFront + up(fp8_debug_plan(M, N, K, split, tile, cu_count()).partial_bytes());
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
  W8_REQUIRE(tile == 0 || tile == 128 || tile == 256 || tile == 129 || tile == 192, W8_ERR_INVALID_ARGUMENT,
             "tile must be 0, 128, 129, 192 or 256");
  W8_REQUIRE(split == 0 || tile == 0 || K % 64 == 0, W8_ERR_UNSUPPORTED, "a tile size needs K %% 64 == 0");
  W8_REQUIRE(split == 0 || (tile != 129 && tile != 192) || (K % 128 == 0 && split <= K / 128), W8_ERR_UNSUPPORTED,
             "128-byte K steps need K %% 128 == 0 and at most K / 128 slices");
  W8_REQUIRE(split <= 1 || (K % 64 == 0 && split <= K / 64), W8_ERR_UNSUPPORTED,
             "split %d needs K %% 64 == 0 and at most K / 64 slices", split);
  W8_REQUIRE(aligned16(xq) && aligned16(sx) && aligned16(Wq8) && aligned16(sw) && aligned16(Y),
             W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  const w8::GemmPlan plan = fp8_debug_plan(M, N, K, split, tile, cu_count());
  W8_REQUIRE(plan.counters() <= kCntCap, W8_ERR_UNSUPPORTED, "too many split tiles (%d > %d)", plan.counters(),
             kCntCap);
  if (w8_status st = check_ws(workspace, workspace_bytes, kFront + up(plan.partial_bytes())); st != W8_OK) return st;
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  w8::launch_fp8_gemm(xq, Wq8, M, N, K, sx, sw, Y, ydt, plan, at<float>(workspace, kFront), at<int>(workspace, 0),
                      static_cast<hipStream_t>(stream));
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
