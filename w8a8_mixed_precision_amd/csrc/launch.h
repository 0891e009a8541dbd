// Host-side launchers of the libw8mp kernels (internal to the library).
#pragma once
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "producer.h"

namespace w8 {

// Sets the detail w8_last_error() returns on this thread; returns `status`.
int report_status(int status, const char* detail);
// Compute units of the current device (0 if it cannot be queried).
int device_cus();

// Grid of the tiled GEMMs: dp_tiles whole tiles of bm x bm outputs, then
// sk_tiles tiles cut into `split` K-slices each (split == 1: none). The int8
// GEMM uses bm = 256, and with `small` runs each of the sk_tiles leftover
// tiles as four 128x128 blocks (each cut into `split` slices); the FP8 GEMM
// and the FP8 weight-only GEMMs use bm = 256 or 128, the W4A8 GEMM 128.
// Tiles past dp_tiles (sk_tiles of them) run as `split` K-slices of whole
// tiles, as `split` K-slices of 128x128 quarters (small), or (streamk, int8
// only) as sk_blocks blocks that share their K steps evenly.
//
// rect (FP8 GEMM, K % 128 == 0): blocks of bm = 128 rows x bn = 128 or 192
// columns on 128-byte K steps.
struct GemmPlan {
  int tiles_m, tiles_n, dp_tiles, split, sk_tiles;
  int bm = 256;
  bool small = false;
  bool streamk = false;
  int sk_blocks = 0;
  bool rect = false;
  int bn = 0;                                    // block columns when rect (else bm)
  bool tail_first = false;                       // int8 quarters: launched before the whole tiles
  int units() const { return small ? 4 * sk_tiles : sk_tiles; }       // blocks per K-slice past dp_tiles
  int grid() const { return dp_tiles + (streamk ? sk_blocks : units() * split); }
  size_t partial_bytes() const {
    if (streamk) return size_t(2) * sk_blocks * bm * bm * 4;           // two slots per stream-K block
    const size_t b = small ? 128 * 128 * 4 : size_t(bm) * (rect ? bn : bm) * 4;
    return split > 1 ? size_t(units()) * split * b : 0;
  }
  int counters() const { return streamk ? sk_tiles : (split > 1 ? units() : 0); }
};
GemmPlan plan_int8_gemm(int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_int8_gemm_forced(int64_t M, int64_t N, int cus, bool small, int split);
// Stream-K over the last round of whole tiles and the leftover ones (all
// tiles when there are fewer than two rounds): `cus` blocks share their K
// steps evenly. K % 64 == 0.
GemmPlan plan_int8_gemm_streamk(int64_t M, int64_t N, int cus);

// The front of every workspace (abi.hip): kCntCap split-K arrival counters
// (zero between calls), then the int8 outlier-column flag words, one per
// column up to the largest int8 K, 133144 (stamped per call, never cleared).
// Shape-dependent regions follow it.
constexpr int kCntCap = 4096;
constexpr size_t kCntBytes = 4 * static_cast<size_t>(kCntCap);
constexpr size_t kFlagBytes = (4 * static_cast<size_t>(133144) + 255) / 256 * 256;
constexpr size_t kFront = kCntBytes + kFlagBytes;

// Outlier columns whose 16-bit values the fix-up stages for the GEMM (XO
// [M, kOutCap], WO [N, kOutCap] in the workspace); a call with more gathers
// them in the GEMM's epilogue instead.
constexpr int kOutCap = 256;

// Where the GEMM epilogue gathers the outlier columns when they do not fit
// the staging: X is made from H [M, K] by the producer `prod` (pa.rstd: the
// row pass's RMSNorm rstd), the weights come from Wq [N, K], the columns from
// the ascending list O.
struct SideSrc {
  const uint16_t* H;
  const int8_t* Wq;
  const int* O;
  int K;
  int prod;
  ProdArgs pa;
};

// prod: producer of X from H (kProdNone / kProdRms / kProdGelu of producer.h;
// rows with a producer need K <= 16384); pa: its parameters. flags: one word
// per column, set to `stamp` where some |x| > t (null: weight pass).
void launch_int8_rows(const void* X, bool bf16, int64_t rows, int K, uint32_t tbits, int8_t* q, float* sx,
                      uint32_t* flags, uint32_t stamp, int prod, const ProdArgs& pa, hipStream_t s);
size_t outlier_fixup_lds_bytes(int K);
void launch_outlier_fixup(const void* X, bool bf16, int64_t M, int K, uint32_t tbits, const uint32_t* colflag,
                          uint32_t stamp, int8_t* q, float* sx, int* O, int* nO, uint16_t* XO, const int8_t* Wq,
                          int64_t N, uint16_t* WO, int prod, const ProdArgs& pa, hipStream_t s);
void launch_produce(const void* H, bool bf16, int64_t M, int K, int prod, const ProdArgs& pa, void* X,
                    hipStream_t s);
void launch_fp8_rows(const void* X, bool bf16, int64_t rows, int K, const float* act_scale, uint8_t* xq, float* sx,
                     int mode, hipStream_t s);
void launch_int8_gemm(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                      const float* sw, const int* nO, const uint16_t* XO, const uint16_t* WO, bool xbf16,
                      const float* bias, void* Y, int mode, const GemmPlan& plan, int* part, int* cnt,
                      const SideSrc& src, hipStream_t s, long long* timeline = nullptr);
GemmPlan plan_fp8_gemm(int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_fp8_gemm_split(int64_t M, int64_t N, int split, int bm);
// 128 x bn blocks (bn = 128 or 192) on 128-byte K steps, `split` K-slices
// each (K % 128 == 0).
GemmPlan plan_fp8_gemm_rect(int64_t M, int64_t N, int split, int bn);
void launch_fp8_gemm(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                     const float* sw, void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s);
// W4A8: int4 weight codes packed two per byte with one fp32 scale per group of
// kW4Group values of K (group-major scales sw[g, n]).
constexpr int kW4Group = 128;
void launch_int4_weights(const void* W, bool bf16, int64_t N, int K, uint8_t* packed, float* sw, hipStream_t s);
GemmPlan plan_w4a8_gemm(int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_w4a8_gemm_split(int64_t M, int64_t N, int split);
void launch_w4a8_gemm(const int8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                      const float* sw, void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s);
GemmPlan plan_w8a16_gemm(int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_w8a16_gemm_split(int64_t M, int64_t N, int split, int bm);
void launch_w8a16_gemm(const uint16_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sw,
                       void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s);
// Plain 16-bit linear (X and W both bf16 or both f16), K % 64 == 0, on the
// weight-only kernel: plan_linear16 (the device's own choice), or
// plan_linear16_tail (256x256 blocks, the leftover tiles of the last partial
// wave in `split` K-slices) / plan_w8a16_gemm_split(.., 128).
GemmPlan plan_linear16(int64_t M, int64_t N, int64_t K, int cus);
GemmPlan plan_linear16_tail(int64_t M, int64_t N, int split, int cus);
void launch_linear16(const uint16_t* A, const uint16_t* B, bool bf16, int64_t M, int64_t N, int64_t K, void* Y,
                     int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s);

}  // namespace w8
