// Block driver: one DiT block's quantized linears chained on the caller's
// stream, with the fp16 exclusion policy for a massive-activation writer.
//
//   qkv = int8_mixed_linear_fused(X, RMSNorm1, Wqkv, bqkv)        fp16 [M, 3D]
//   a   = qkv[:, 2D:3D]                                            attention stub
//   o   = int8_mixed_linear_fused(a, none, Wo, bo)                 fp16 [M, D]
//   h   = X + o                                                    fp16
//   u   = int8_mixed_linear_fused(h, RMSNorm2, Wup, bup)           fp16 [M, F]
//   d   = int8_mixed_linear_fused(u, GELU, Wdown, bdown)           fp16 [M, D]
//         or, excluded: GELU(u) W16down^T (+ bdown) in 16 bit      fp32 [M, D]
//   Y   = h + d                                                    fp16
//
// The "Image21-INT8" card (section "Quantization") quantizes a block's linears
// with LLM.int8 at threshold 6.0; the "Image21-Turbo-OrbitQuant-W4A4" card
// (section "What 4-bit breaks here and what stays in fp16") keeps the MLP
// output projections that write the near-9000 text-token values in fp16.
// Attention is not part of the quantized path: the stub passes each token's
// value vector through, as if every token attended only to itself.
#include <algorithm>
#include <cstdarg>
#include <cstdio>

#include <hip/hip_runtime.h>

#include "common.h"
#include "launch.h"
#include "w8mp.h"

namespace w8 {

// a[m, c] = qkv[m, 2D + c], 16-byte chunks (D % 8 == 0).
__global__ __launch_bounds__(256) void k_take_value(const uint16_t* __restrict__ qkv, int64_t M, int D,
                                                    uint16_t* __restrict__ a) {
  const int cpr = D / 8;                        // chunks per row
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * cpr) return;
  const int64_t m = i / cpr;
  const int c = static_cast<int>(i % cpr);
  reinterpret_cast<uint4*>(a + m * D)[c] = reinterpret_cast<const uint4*>(qkv + m * 3 * D + 2 * D)[c];
}

// y = rne16(fl32(h) + fl32(d + bias)) per element; d fp16 (F32D false) or
// fp32, bias fp32 [D] or null. 8 elements per thread (D % 8 == 0).
template <bool F32D>
__global__ __launch_bounds__(256) void k_residual(const uint16_t* __restrict__ h, const void* __restrict__ d,
                                                  const float* __restrict__ bias, int64_t M, int D,
                                                  uint16_t* __restrict__ y) {
#pragma clang fp contract(off)
  const int cpr = D / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= M * cpr) return;
  const int c = static_cast<int>(i % cpr);
  float hv[8], dv[8];
  unpack8<false>(reinterpret_cast<const uint4*>(h)[i], hv);
  if constexpr (F32D) {
    const float4 a = reinterpret_cast<const float4*>(d)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(d)[2 * i + 1];
    dv[0] = a.x; dv[1] = a.y; dv[2] = a.z; dv[3] = a.w;
    dv[4] = b.x; dv[5] = b.y; dv[6] = b.z; dv[7] = b.w;
  } else {
    unpack8<false>(reinterpret_cast<const uint4*>(d)[i], dv);
  }
  if (bias) {
    const float4 a = reinterpret_cast<const float4*>(bias)[2 * c];
    const float4 b = reinterpret_cast<const float4*>(bias)[2 * c + 1];
    const float bv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) dv[e] = dv[e] + bv[e];
  }
  uint32_t o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32_to_f16_bits(hv[e] + dv[e]);
  reinterpret_cast<uint4*>(y)[i] = make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                                              o[6] | (o[7] << 16));
}

static void launch_take_value(const uint16_t* qkv, int64_t M, int D, uint16_t* a, hipStream_t s) {
  const int64_t n = M * (D / 8);
  k_take_value<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(qkv, M, D, a);
}

static void launch_residual(const uint16_t* h, const void* d, bool f32d, const float* bias, int64_t M, int D,
                            uint16_t* y, hipStream_t s) {
  const int64_t n = M * (D / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  if (f32d) k_residual<true><<<grid, block, 0, s>>>(h, d, bias, M, D, y);
  else k_residual<false><<<grid, block, 0, s>>>(h, d, bias, M, D, y);
}

}  // namespace w8

namespace {

constexpr size_t kAlignB = 256;
size_t upb(size_t x) { return (x + kAlignB - 1) / kAlignB * kAlignB; }

int block_cus() { return std::max(w8::device_cus(), 1); }

// Block workspace: one int8 linear workspace, shared by the four linears
// (its front and int8 layout serve calls of any shape in turn), then the
// intermediates, then the 16-bit down-projection's split-K partials (its
// counters are the front's).
struct BlockWs {
  size_t ws8, qkv, a, o, h, u, g, d, part16, total;
  size_t n8;
  w8::GemmPlan plan16;
};

BlockWs block_layout(int64_t M, int64_t D, int64_t F) {
  BlockWs w{};
  w.n8 = std::max({int8_mixed_linear_workspace_size(M, 3 * D, D), int8_mixed_linear_workspace_size(M, D, D),
                   int8_mixed_linear_workspace_size(M, F, D), int8_mixed_linear_workspace_size(M, D, F)});
  // sized for a 256-CU device; forward() runs this device's plan when it fits
  w.plan16 = w8::plan_linear16(M, D, F, 256);
  if (w.plan16.counters() > w8::kCntCap) w.plan16 = w8::plan_linear16_tail(M, D, 1, 256);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = upb(off + bytes); return at; };
  w.ws8 = take(w.n8);
  w.qkv = take(2 * static_cast<size_t>(M) * 3 * D);
  w.a = take(2 * static_cast<size_t>(M) * D);
  w.o = take(2 * static_cast<size_t>(M) * D);
  w.h = take(2 * static_cast<size_t>(M) * D);
  w.u = take(2 * static_cast<size_t>(M) * F);
  w.g = take(2 * static_cast<size_t>(M) * F);
  w.d = take(4 * static_cast<size_t>(M) * D);
  w.part16 = take(w.plan16.partial_bytes());
  w.total = off;
  return w;
}

w8_status block_fail(w8_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return static_cast<w8_status>(w8::report_status(st, buf));
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

size_t w8_dit_block_workspace_size(int64_t M, int64_t D, int64_t F) {
  if (M < 1 || D < 1 || F < 1) return 0;
  return block_layout(M, D, F).total;
}

w8_status w8_dit_block_forward(const w8_dit_block* blk, const void* X, int64_t M, void* Y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!blk || !X || !Y) return block_fail(W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  const int64_t D = blk->D, F = blk->F;
  if (M < 1 || D < 64 || F < 64 || D % 64 != 0 || F % 64 != 0 || D > 16384 || F > 16384)
    return block_fail(W8_ERR_INVALID_ARGUMENT, "need M >= 1 and D, F multiples of 64 in [64, 16384]");
  if (!blk->w_qkv || !blk->s_qkv || !blk->w_o || !blk->s_o || !blk->w_up || !blk->s_up)
    return block_fail(W8_ERR_INVALID_ARGUMENT, "missing int8 weights or scales");
  if (!blk->w_down16 && (!blk->w_down || !blk->s_down))
    return block_fail(W8_ERR_INVALID_ARGUMENT, "down projection: int8 weights and scales, or 16-bit weights");
  if (!al16(X) || !al16(Y) || (blk->w_down16 && !al16(blk->w_down16)) || (blk->b_down && !al16(blk->b_down)))
    return block_fail(W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  const BlockWs L = block_layout(M, D, F);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlignB - 1)) != 0 || workspace_bytes < L.total)
    return block_fail(W8_ERR_WORKSPACE, "workspace must be 256-byte aligned and at least %zu bytes", L.total);
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float t = blk->threshold;
  w8_status st;
  const w8_producer none{W8_PRODUCER_NONE, nullptr, nullptr, nullptr, 0.0f};
  const w8_producer gelu{W8_PRODUCER_GELU_TANH, nullptr, nullptr, nullptr, 0.0f};

  // qkv = Linear8(RMSNorm1(X))
  st = int8_mixed_linear_fused(X, W8_DT_F16, M, D, &blk->norm1, blk->w_qkv, blk->s_qkv, blk->b_qkv, 3 * D, t,
                               at(L.qkv), W8_DT_F16, at(L.ws8), L.n8, stream);
  if (st != W8_OK) return block_fail(st, "qkv: %s", w8_last_error());
  w8::launch_take_value(static_cast<const uint16_t*>(at(L.qkv)), M, static_cast<int>(D),
                        static_cast<uint16_t*>(at(L.a)), s);
  st = int8_mixed_linear_fused(at(L.a), W8_DT_F16, M, D, &none, blk->w_o, blk->s_o, blk->b_o, D, t, at(L.o),
                               W8_DT_F16, at(L.ws8), L.n8, stream);
  if (st != W8_OK) return block_fail(st, "o: %s", w8_last_error());
  w8::launch_residual(static_cast<const uint16_t*>(X), at(L.o), false, nullptr, M, static_cast<int>(D),
                      static_cast<uint16_t*>(at(L.h)), s);
  st = int8_mixed_linear_fused(at(L.h), W8_DT_F16, M, D, &blk->norm2, blk->w_up, blk->s_up, blk->b_up, F, t,
                               at(L.u), W8_DT_F16, at(L.ws8), L.n8, stream);
  if (st != W8_OK) return block_fail(st, "up: %s", w8_last_error());
  if (blk->w_down16) {
    // the massive-activation writer, unquantized: GELU(u) W16^T in 16 bit
    w8::launch_produce(at(L.u), false, M, static_cast<int>(F), w8::kProdGelu, w8::ProdArgs{}, at(L.g), s);
    w8::GemmPlan p16 = w8::plan_linear16(M, D, F, block_cus());
    if (p16.counters() > w8::kCntCap || p16.partial_bytes() > L.plan16.partial_bytes())
      p16 = w8::plan_linear16_tail(M, D, 1, block_cus());
    w8::launch_linear16(static_cast<const uint16_t*>(at(L.g)), blk->w_down16, false, M, D, F, at(L.d), 2, p16,
                        reinterpret_cast<float*>(ws + L.part16), reinterpret_cast<int*>(ws + L.ws8), s);
    w8::launch_residual(static_cast<const uint16_t*>(at(L.h)), at(L.d), true, blk->b_down, M, static_cast<int>(D),
                        static_cast<uint16_t*>(Y), s);
  } else {
    st = int8_mixed_linear_fused(at(L.u), W8_DT_F16, M, F, &gelu, blk->w_down, blk->s_down, blk->b_down, D, t,
                                 at(L.d), W8_DT_F16, at(L.ws8), L.n8, stream);
    if (st != W8_OK) return block_fail(st, "down: %s", w8_last_error());
    w8::launch_residual(static_cast<const uint16_t*>(at(L.h)), at(L.d), false, nullptr, M, static_cast<int>(D),
                        static_cast<uint16_t*>(Y), s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return block_fail(W8_ERR_HIP, "w8_dit_block_forward: %s", hipGetErrorString(e));
  return static_cast<w8_status>(w8::report_status(W8_OK, ""));
}

// The parity export's tiling: the driver's own plan (split 0), 256x256 blocks
// with the last partial wave's tiles in `split` K-slices, or 128x128 blocks
// all in `split` K-slices.
static w8::GemmPlan linear16_debug_plan(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (split == 0) return w8::plan_linear16(M, N, K, block_cus());
  if (tile == 256) return w8::plan_linear16_tail(M, N, split, block_cus());
  return w8::plan_w8a16_gemm_split(M, N, split, 128);
}

size_t w8dbg_linear16_workspace_size(int64_t M, int64_t N, int64_t K, int split, int tile) {
  if (M < 1 || N < 1 || K < 1 || split < 0) return 0;
  const w8::GemmPlan p = linear16_debug_plan(M, N, K, split, tile);
  return w8::kFront + upb(p.partial_bytes());
}

// The offsets of the block's intermediates in its workspace (parity export):
// qkv, a, o, h, u, g (GELU(u), written only with the 16-bit down-projection),
// d (fp16, or fp32 with the 16-bit down-projection).
w8_status w8dbg_dit_block_layout(int64_t M, int64_t D, int64_t F, size_t* offsets) {
  if (!offsets || M < 1 || D < 1 || F < 1) return block_fail(W8_ERR_INVALID_ARGUMENT, "bad arguments");
  const BlockWs L = block_layout(M, D, F);
  const size_t v[7] = {L.qkv, L.a, L.o, L.h, L.u, L.g, L.d};
  for (int i = 0; i < 7; ++i) offsets[i] = v[i];
  return static_cast<w8_status>(w8::report_status(W8_OK, ""));
}

w8_status w8dbg_linear16(const void* X, int x_dt, int64_t M, int64_t K, const void* W, int64_t N, int split, int tile,
                         void* Y, int y_dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !W || !Y) return block_fail(W8_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (x_dt != W8_DT_F16 && x_dt != W8_DT_BF16) return block_fail(W8_ERR_UNSUPPORTED, "X must be f16 or bf16");
  if (y_dt != W8_DT_BF16 && y_dt != W8_DT_F16 && y_dt != W8_DT_F32)
    return block_fail(W8_ERR_UNSUPPORTED, "Y must be bf16, f16 or f32");
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || K > 65536 || N >= (int64_t(1) << 31))
    return block_fail(K % 64 != 0 ? W8_ERR_UNSUPPORTED : W8_ERR_INVALID_ARGUMENT,
                      "need M, N >= 1 and K a multiple of 64 in [64, 65536]");
  if (M * K * 2 >= (int64_t(1) << 32) || N * K * 2 >= (int64_t(1) << 32))
    return block_fail(W8_ERR_UNSUPPORTED, "X and W must each be smaller than 4 GiB");
  if (split < 0 || split > K / 64) return block_fail(W8_ERR_UNSUPPORTED, "split must be in [0, K / 64]");
  if (split > 0 && tile != 128 && tile != 256) return block_fail(W8_ERR_INVALID_ARGUMENT, "tile must be 128 or 256");
  if (!al16(X) || !al16(W) || !al16(Y)) return block_fail(W8_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  const w8::GemmPlan p = linear16_debug_plan(M, N, K, split, tile);
  if (p.counters() > w8::kCntCap) return block_fail(W8_ERR_UNSUPPORTED, "too many split tiles");
  const size_t need = w8::kFront + upb(p.partial_bytes());
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & (kAlignB - 1)) != 0 || workspace_bytes < need)
    return block_fail(W8_ERR_WORKSPACE, "workspace must be 256-byte aligned and at least %zu bytes", need);
  const int ydt = y_dt == W8_DT_BF16 ? 0 : (y_dt == W8_DT_F16 ? 1 : 2);
  char* ws = static_cast<char*>(workspace);
  w8::launch_linear16(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), x_dt == W8_DT_BF16, M, N, K,
                      Y, ydt, p, reinterpret_cast<float*>(ws + w8::kFront), reinterpret_cast<int*>(ws),
                      static_cast<hipStream_t>(stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return block_fail(W8_ERR_HIP, "w8dbg_linear16: %s", hipGetErrorString(e));
  return static_cast<w8_status>(w8::report_status(W8_OK, ""));
}

}  // extern "C"
