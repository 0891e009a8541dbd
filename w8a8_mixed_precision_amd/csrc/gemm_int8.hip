// int8 x int8 -> int32 MFMA GEMM with the LLM.int8 epilogue (gfx950).
//
//   acc[m,n] = sum_k q[m,k] * Wq[n,k]                 (v_mfma_i32_16x16x64_i8, exact)
//   f        = float(acc) * (sx[m] / 127)
//   f       += sum_j XO[m,j] * WO[n,j]                (v_mfma_f32_16x16x32_{bf16,f16})
//   Y[m,n]   = f * (sw[n] / 127)
//
// The side product runs over the gathered outlier columns of X (XO) and the
// same columns of Wq cast to 16 bits (WO), both zero-padded to a multiple of
// 32; the 16x16 f32 and i32 MFMA results share one register layout, so it
// accumulates straight into the converted int32 tile. This is the LLM.int8
// decomposition ("Image21-INT8" card, section "Quantization": outliers are
// handled in floating point) with LLM.int8()'s vector-wise dequantisation.
//
// Tiling: 256 threads = 4 waves as 2x2, block tile 256x256, K step 64 bytes.
// Each wave owns a 128x128 sub-tile = 8x8 MFMA 16x16 tiles (256 accumulator
// registers). Operands are staged through LDS (2 stages x 32 KB) with a 16-byte
// XOR swizzle; both operands are K-contiguous ([M,K] and [N,K]).
#include <type_traits>

#include "common.h"

namespace w8 {

constexpr int kBM = 256, kBN = 256, kBK = 64;

// LDS byte offset of 16-byte chunk `ch` (0..3) of tile row `row` (64 B per row).
__device__ __forceinline__ int swz64(int row, int ch) { return row * kBK + ((ch ^ ((row >> 2) & 3)) << 4); }

// XCD-aware block order: the hardware deals consecutive workgroups round-robin
// over the 8 XCDs; renumber so each XCD gets a contiguous range, then walk
// tiles in groups of kGroupM tile-rows so blocks that run together on one XCD
// share A rows and B columns in that XCD's L2.
constexpr int kXcds = 8, kGroupM = 4;

__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per = (nblocks + kXcds - 1) / kXcds;
  const int tall = nblocks - (per - 1) * kXcds;  // XCDs that get `per` blocks
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int id = (xcd < tall) ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
  const int in_group = kGroupM * tiles_n;
  const int g = id / in_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = id % in_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// MODE 0: raw int32 accumulators to Y (int32 [M,N]); 1: fp16 Y; 2: fp32 Y.
template <int MODE, bool XBF16>
__global__ __launch_bounds__(256, 1) void k_int8_gemm(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                      int M, int N, int K, const float* __restrict__ sx,
                                                      const float* __restrict__ sw, const int* __restrict__ nO_ptr,
                                                      const uint16_t* __restrict__ XO,
                                                      const uint16_t* __restrict__ WO, void* __restrict__ Y,
                                                      int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t lds[2][2][kBM * kBK];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: this thread moves chunk (tid&3) of rows tid/4 + 64*i
  const int ld_ch = tid & 3;
  const int8_t* a_src[4];
  const int8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 2) + 64 * i;
    a_src[i] = A + static_cast<int64_t>(min(m0 + r, M - 1)) * K + ld_ch * 16;
    b_src[i] = B + static_cast<int64_t>(min(n0 + r, N - 1)) * K + ld_ch * 16;
  }
  uint4 ra[4], rb[4];
  const int nk = (K + kBK - 1) / kBK;

  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
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
      const int r = (tid >> 2) + 64 * i;
      *reinterpret_cast<uint4*>(&lds[st][0][swz64(r, ld_ch)]) = ra[i];
      *reinterpret_cast<uint4*>(&lds[st][1][swz64(r, ld_ch)]) = rb[i];
    }
  };

  v4i acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  gload(0);
  lstore(0);
  __syncthreads();

  const int fr = lane & 15, fc = lane >> 4;  // fragment row within 16, 16-byte K chunk
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    v4i a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const v4i*>(&lds[st][0][swz64(wm * 128 + i * 16 + fr, fc)]);
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = *reinterpret_cast<const v4i*>(&lds[st][1][swz64(wn * 128 + j * 16 + fr, fc)]);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // Output coordinates of accumulator element e of tile (i, j):
  //   m = m0 + wm*128 + i*16 + 4*(lane>>4) + e,  n = n0 + wn*128 + j*16 + (lane&15)
  const int mb = m0 + wm * 128 + 4 * (lane >> 4);
  const int nb = n0 + wn * 128 + (lane & 15);

  if constexpr (MODE == 0) {
    int32_t* y = static_cast<int32_t*>(Y);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mb + i * 16 + e, n = nb + j * 16;
          if (m < M && n < N) y[static_cast<int64_t>(m) * N + n] = acc[i][j][e];
        }
  } else {
    // One 16-row block of the wave tile at a time keeps 32 floats live.
    const int nO = *nO_ptr;
    const int P = (nO + 31) & ~31;
    using V8 = typename std::conditional<XBF16, v8bf, v8h>::type;
    float cs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) cs[j] = sw[min(nb + j * 16, N - 1)] / 127.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float rs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rs[e] = sx[min(mb + i * 16 + e, M - 1)] / 127.0f;
      v4f f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[j][e] = static_cast<float>(acc[i][j][e]) * rs[e];
      const int64_t xrow = static_cast<int64_t>(min(m0 + wm * 128 + i * 16 + fr, M - 1)) * P;
      for (int c = 0; c < P; c += 32) {
        // A fragment: XO row of this lane, outlier slots c + 8*fc .. +8
        const V8 xa = *reinterpret_cast<const V8*>(XO + xrow + c + 8 * fc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const V8 wb = *reinterpret_cast<const V8*>(
              WO + static_cast<int64_t>(min(n0 + wn * 128 + j * 16 + fr, N - 1)) * P + c + 8 * fc);
          if constexpr (XBF16)
            f[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wb, f[j], 0, 0, 0);
          else
            f[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, wb, f[j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = nb + j * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mb + i * 16 + e;
          if (m < M && n < N) {
            const float y = f[j][e] * cs[j];
            if constexpr (MODE == 1)
              static_cast<uint16_t*>(Y)[static_cast<int64_t>(m) * N + n] = f32_to_f16_bits(y);
            else
              static_cast<float*>(Y)[static_cast<int64_t>(m) * N + n] = y;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// mode: 0 int32 acc, 1 fp16 out, 2 fp32 out
void launch_int8_gemm(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                      const float* sw, const int* nO, const uint16_t* XO, const uint16_t* WO, bool xbf16,
                      void* Y, int mode, hipStream_t s) {
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const dim3 grid(tiles_m * tiles_n), block(256);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (mode == 0)
    k_int8_gemm<0, true><<<grid, block, 0, s>>>(A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n);
  else if (mode == 1) {
    if (xbf16) k_int8_gemm<1, true><<<grid, block, 0, s>>>(A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n);
    else k_int8_gemm<1, false><<<grid, block, 0, s>>>(A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n);
  } else {
    if (xbf16) k_int8_gemm<2, true><<<grid, block, 0, s>>>(A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n);
    else k_int8_gemm<2, false><<<grid, block, 0, s>>>(A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n);
  }
}

}  // namespace w8
