// Measured peaks of the matrix cores (parity/measurement export of libw8mp):
// every wave issues `iters` rounds of back-to-back MFMAs on register
// operands, four independent accumulators in turn so that no instruction
// waits for the previous one's result, and stores a checksum so that nothing
// is optimised away. The rate this reaches with every SIMD busy is the
// chip's attainable dense MFMA peak at the clock it holds under that load;
// GEMM fractions can be read against it beside the published figure.
// The matrix cores' power, and so the clock the chip holds, depends on the
// operand bits: with RND the operands change every round (a linear
// congruential step per register, hidden under the MFMAs), as a GEMM's
// operands do, which gives the rate a GEMM on random data can approach.
#include <hip/hip_runtime.h>

#include "common.h"
#include "w8mp.h"

namespace w8 {

namespace {

typedef int v16i_ __attribute__((ext_vector_type(16)));
typedef float v16f_ __attribute__((ext_vector_type(16)));

// kind 0: v_mfma_i32_32x32x32_i8 (2*32*32*32 ops); 1: v_mfma_scale_f32_32x32x64_f8f6f4
// with E4M3 operands (2*32*32*64 flops); 2: v_mfma_f32_32x32x16_bf16 (2*32*32*16).
template <int KIND, bool RND>
__global__ __launch_bounds__(256) void k_mfma_peak(int iters, int seed, unsigned* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  unsigned sum = 0;
  if constexpr (KIND == 0) {
    v4i a = {seed + lane, 3, 5, 7}, b = {seed ^ lane, 11, 13, 17};
    v16i_ c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[j][r] = 0;
    if (RND) {
      a = v4i{a[0] * 2654435 + lane, a[1] * 40503 + 1, a[2] ^ (lane << 8), a[3] + lane * 977};
      b = v4i{b[0] * 69069 + 7, b[1] ^ (lane << 16), b[2] * 3 + lane, b[3] * 1103515245};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
      if (RND) {
        a = a * 1664525 + 1013904223;
        b = b * 22695477 + 1;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += static_cast<unsigned>(c[j][r]);
  } else if constexpr (KIND == 1) {
    v8i a = {0x38383838 + lane, 0x38383838, 0x30303030, 0x38383838, 0x38383838, 0x30303030, 0x38383838, 0x38383838};
    v8i b = a;
    v16f_ c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
    // changing E4M3 operands keep every byte's exponent field at most 0111
    // (no NaN, no overflow of the sums)
    constexpr int kF8Mask = 0x3F3F3F3F;
    if (RND) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = (a[e] * (2654435 + 2 * e) + lane * 977) & kF8Mask;
        b[e] = (b[e] * (40503 + 2 * e) + lane) & kF8Mask;
      }
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 127, 0, 127);
      if (RND) {
        a = (a * 1664525 + 1013904223) & kF8Mask;
        b = (b * 22695477 + 1) & kF8Mask;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += __float_as_uint(c[j][r]);
  } else {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = static_cast<__bf16>(static_cast<float>(e + lane) * 0.125f);
      b[e] = static_cast<__bf16>(static_cast<float>(e ^ seed) * 0.25f);
    }
    v16f_ c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += __float_as_uint(c[j][r]);
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// Operand streaming into LDS, the GEMMs' load path: every block owns a panel
// of 256 rows with row pitch K bytes (block b takes panel b % panels) and
// moves one K step of SEG bytes of all 256 rows per iteration into a 4-slot
// LDS ring with buffer loads (1 KB per wave instruction: 1024 / SEG rows of
// SEG bytes), keeping 12 KB per wave in flight, walking the panel's K
// steps round robin. With panels small enough to stay in L2 this is the L2 ->
// LDS rate; SEG 64 is the GEMMs' 64-byte K step (half a 128-byte line per
// row), SEG 128 whole lines.
template <int SEG>
__global__ __launch_bounds__(256, 1) void k_lds_stream(const int8_t* __restrict__ buf, int K, int panels, int iters,
                                                      unsigned* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[4 * 32768];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  constexpr int kLpr = SEG / 16;               // lanes per row
  constexpr int kRpi = 64 / kLpr;              // rows per instruction
  constexpr int kNi = 256 / kRpi / 4;          // instructions per wave per step
  const int panel = blockIdx.x % panels;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(buf) + static_cast<int64_t>(panel) * 256 * K, 0, 256u * static_cast<uint32_t>(K), 0x00020000);
  const int nk = K / SEG;
  for (int it = 0; it < iters; ++it) {
    int8_t* st = lds + (it & 3) * 32768;
    const int k0 = (it % nk) * SEG;
#pragma unroll
    for (int i = 0; i < kNi; ++i) {
      const int row = (wave * kNi + i) * kRpi + lane / kLpr;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, st + ((wave * kNi + i) * 1024) % 32768, 16,
                                               static_cast<uint32_t>(row * K + (lane % kLpr) * 16), k0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | 12);   // vmcnt(12)
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = static_cast<unsigned>(lds[4 * lane]);
}

// Every float32 bit pattern x, paired with y = x ^ 0x5A5A5A5A (so every
// pattern takes both places of a pair): the packed conversion against the two
// scalar ones. out[0]: mismatching pairs of non-NaN inputs; out[1]: pairs with
// a NaN input whose fp16 results differ; out[2]: the smallest x of a non-NaN
// mismatch (0xFFFFFFFF if none).
__global__ __launch_bounds__(256) void k_cvt_f16_pair_check(unsigned* __restrict__ out) {
  const uint32_t stride = gridDim.x * blockDim.x;
  unsigned bad = 0, bad_nan = 0, first = 0xFFFFFFFFu;
  for (uint64_t p = blockIdx.x * blockDim.x + threadIdx.x; p < (uint64_t{1} << 32); p += stride) {
    const uint32_t xb = static_cast<uint32_t>(p), yb = xb ^ 0x5A5A5A5Au;
    const float x = __uint_as_float(xb), y = __uint_as_float(yb);
    const uint32_t pk = f32x2_to_f16x2_bits(x, y);
    const uint32_t sc = f32_to_f16_bits(x) | (static_cast<uint32_t>(f32_to_f16_bits(y)) << 16);
    if (pk != sc) {
      if (__builtin_isnan(x) || __builtin_isnan(y)) {
        ++bad_nan;
      } else {
        ++bad;
        first = min(first, xb);
      }
    }
  }
  if (bad) atomicAdd(out, bad);
  if (bad_nan) atomicAdd(out + 1, bad_nan);
  if (first != 0xFFFFFFFFu) atomicMin(out + 2, first);
}

}  // namespace

}  // namespace w8

extern "C" {

// See include/w8mp.h.
w8_status w8dbg_cvt_f16_pair_check(unsigned* out, void* stream) {
  if (!out) return W8_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  w8::k_cvt_f16_pair_check<<<dim3(2048), dim3(256), 0, s>>>(out);
  return hipGetLastError() == hipSuccess ? W8_OK : W8_ERR_HIP;
}

// See include/w8mp.h.
w8_status w8dbg_mfma_peak(int kind, int blocks, int iters, unsigned* out, double* ops, void* stream) {
  if (!out || !ops || kind < 0 || kind > 4 || blocks < 1 || iters < 1)
    return W8_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(256);
  if (kind == 0) w8::k_mfma_peak<0, false><<<grid, block, 0, s>>>(iters, 1, out);
  else if (kind == 1) w8::k_mfma_peak<1, false><<<grid, block, 0, s>>>(iters, 1, out);
  else if (kind == 2) w8::k_mfma_peak<2, false><<<grid, block, 0, s>>>(iters, 1, out);
  else if (kind == 3) w8::k_mfma_peak<0, true><<<grid, block, 0, s>>>(iters, 1, out);
  else w8::k_mfma_peak<1, true><<<grid, block, 0, s>>>(iters, 1, out);
  kind = kind == 3 ? 0 : (kind == 4 ? 1 : kind);
  const double per_inst = kind == 0 ? 2.0 * 32 * 32 * 32 : (kind == 1 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16);
  *ops = per_inst * 4.0 * iters * (static_cast<double>(blocks) * 4.0);   // 4 waves per block, 4 per round
  return hipGetLastError() == hipSuccess ? W8_OK : W8_ERR_HIP;
}

// See include/w8mp.h.
w8_status w8dbg_lds_stream(const void* buf, size_t buf_bytes, int K, int seg, int blocks, int panels, int iters,
                           unsigned* out, double* bytes, void* stream) {
  if (!buf || !out || !bytes || (seg != 64 && seg != 128) || K < seg || K % seg != 0 || blocks < 1 || panels < 1 ||
      iters < 1 || static_cast<int64_t>(K) * 256 >= (int64_t{1} << 31) ||
      buf_bytes < static_cast<size_t>(panels) * 256 * static_cast<size_t>(K))
    return W8_ERR_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(256);
  if (seg == 64) w8::k_lds_stream<64><<<grid, block, 0, s>>>(static_cast<const int8_t*>(buf), K, panels, iters, out);
  else w8::k_lds_stream<128><<<grid, block, 0, s>>>(static_cast<const int8_t*>(buf), K, panels, iters, out);
  *bytes = 256.0 * seg * iters * static_cast<double>(blocks);
  return hipGetLastError() == hipSuccess ? W8_OK : W8_ERR_HIP;
}

}  // extern "C"
