// FP8-E4M3 W8A8 GEMM with per-token x per-channel scale epilogue (gfx950).
//
//   acc[m,n] = sum_k e4m3(xq[m,k]) * e4m3(wq[n,k])   (fp32 accumulation)
//   Y[m,n]   = acc * sx[m] * sw[n]
//
// E4M3 weights with one scale per output channel and per-token activation
// scales ("Qwen-Image-2.1 Text Encoder: FP8" card, section "Format"); a static
// per-tensor input scale arrives as the same sx vector ("Darkstar ... ModelOpt
// FP8" card, section "Precision map").
//
// The contraction uses v_mfma_scale_f32_16x16x128_f8f6f4 with both block
// scales at 2^0 (E8M0 code 127) and format E4M3 on both sides: 16x16 output,
// K = 128 per instruction, 32 bytes of each operand per lane.
// Tiling: 256 threads = 4 waves as 2x2, block tile 128x128, K step 128 bytes,
// each wave 64x64 = 4x4 MFMA tiles. LDS: 2 stages x (16 + 16) KB, 16-byte XOR
// swizzle over the 8 chunks of a 128-byte row.
#include "common.h"

namespace w8 {

constexpr int kFBM = 128, kFBN = 128, kFBK = 128;

__device__ __forceinline__ int swz128(int row, int ch) { return row * kFBK + ((ch ^ ((row >> 1) & 7)) << 4); }

// YDT: 0 bf16, 1 fp16, 2 fp32
template <int YDT>
__global__ __launch_bounds__(256, 2) void k_fp8_gemm(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                     int M, int N, int K, const float* __restrict__ sx,
                                                     const float* __restrict__ sw, void* __restrict__ Y,
                                                     int tiles_m) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kFBM * kFBK];
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * kFBM, n0 = tn * kFBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // staging: 128 rows x 8 chunks per operand = 1024 chunks; 4 per thread:
  // chunk (tid & 7) of rows tid/8 + 32*i
  const int ld_ch = tid & 7;
  const uint8_t* a_src[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    a_src[i] = A + static_cast<int64_t>(min(m0 + r, M - 1)) * K + ld_ch * 16;
    b_src[i] = B + static_cast<int64_t>(min(n0 + r, N - 1)) * K + ld_ch * 16;
  }
  uint4 ra[4], rb[4];
  const int nk = (K + kFBK - 1) / kFBK;
  auto gload = [&](int kt) {
    const int k0 = kt * kFBK;
    const bool ok = k0 + ld_ch * 16 < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ok ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = ok ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<uint4*>(&lds[st][0][swz128(r, ld_ch)]) = ra[i];
      *reinterpret_cast<uint4*>(&lds[st][1][swz128(r, ld_ch)]) = rb[i];
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 15, fc = lane >> 4;  // 32-byte K slice fc = chunks 2fc, 2fc+1
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    v8i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + fr;
      const v4i lo = *reinterpret_cast<const v4i*>(&lds[st][0][swz128(r, 2 * fc)]);
      const v4i hi = *reinterpret_cast<const v4i*>(&lds[st][0][swz128(r, 2 * fc + 1)]);
      a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + fr;
      const v4i lo = *reinterpret_cast<const v4i*>(&lds[st][1][swz128(r, 2 * fc)]);
      const v4i hi = *reinterpret_cast<const v4i*>(&lds[st][1][swz128(r, 2 * fc + 1)]);
      b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  const int mb = m0 + wm * 64 + 4 * (lane >> 4);
  const int nb = n0 + wn * 64 + (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nb + j * 16;
    const float cs = sw[min(n, N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mb + i * 16 + e;
        if (m < M && n < N) {
          const float y = acc[i][j][e] * sx[m] * cs;
          const int64_t o = static_cast<int64_t>(m) * N + n;
          if constexpr (YDT == 0) static_cast<uint16_t*>(Y)[o] = static_cast<uint16_t>(bf16_rne_bits(y));
          else if constexpr (YDT == 1) static_cast<uint16_t*>(Y)[o] = f32_to_f16_bits(y);
          else static_cast<float*>(Y)[o] = y;
        }
      }
  }
}

// ydt: 0 bf16, 1 fp16, 2 fp32
void launch_fp8_gemm(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                     const float* sw, void* Y, int ydt, hipStream_t s) {
  const int tiles_m = static_cast<int>((M + kFBM - 1) / kFBM);
  const int tiles_n = static_cast<int>((N + kFBN - 1) / kFBN);
  const dim3 grid(tiles_m * tiles_n), block(256);
  if (ydt == 0) k_fp8_gemm<0><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
  else if (ydt == 1) k_fp8_gemm<1><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
  else k_fp8_gemm<2><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
}

}  // namespace w8
