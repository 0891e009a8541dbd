// int8 x int8 -> int32 MFMA GEMM with the LLM.int8 epilogue (gfx950).
//
//   acc[m,n] = sum_k q[m,k] * Wq[n,k]                 (v_mfma_i32_32x32x32_i8, exact)
//   side     = sum_j XO[m,j] * WO[n,j]                (v_mfma_f32_32x32x16_{bf16,f16})
//   Y[m,n]   = (float(acc) * (sx[m] / 127) + side) * (sw[n] / 127)
//
// The side product runs over the gathered outlier columns of X (XO) and the
// same columns of Wq cast to 16 bits (WO), both zero-padded to a multiple of
// 32. The 32x32 f32 and i32 MFMA results share one register layout, so the
// side product lines up element for element with the int32 tile. This is the
// LLM.int8 decomposition ("Image21-INT8" card, section "Quantization":
// outliers are handled in floating point) with LLM.int8()'s vector-wise
// dequantisation.
//
// Tiling: 256 threads = 4 waves as 2x2, block tile 256x256, K step 64 bytes.
// Each wave owns a 128x128 sub-tile = 4x4 MFMA 32x32 tiles (256 accumulator
// registers). On gfx950 the 32x32x32 int8 MFMA runs at the full int8 rate
// (the 16x16x64 form issues at half of it). Both operands are K-contiguous
// ([M,K] and [N,K]) and staged through LDS with a 16-byte XOR swizzle.
#include <type_traits>

#include "common.h"

namespace w8 {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64;

// LDS byte offset of logical 16-byte chunk `ch` (0..3) of tile row `row`
// (64 bytes per row). The XOR term makes the fragment reads (32 rows at one
// chunk per half-wave) hit distinct banks in every 8- and 16-lane group.
__device__ __forceinline__ int swz_term(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int swz64(int row, int ch) { return row * kBK + ((ch ^ swz_term(row)) << 4); }

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

// One K step (64 bytes) of the wave's 128x128 tile from LDS: two 32-byte
// sub-steps; lane l supplies row (l & 31), chunk 2*s + (l >> 5).
__device__ __forceinline__ void mma_step(const int8_t* sa, const int8_t* sb, v16i (&acc)[4][4], int wm, int wn,
                                         int lane) {
  const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    v4i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const v4i*>(sa + swz64(wm * 128 + i * 32 + fr, 2 * s + fh));
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const v4i*>(sb + swz64(wn * 128 + j * 32 + fr, 2 * s + fh));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[i][j], 0, 0, 0);
  }
}

// Epilogue shared by both GEMM kernels. The MFMAs compute each 32x32 tile
// transposed (Wq fragment as the first operand), so element r of tile (i, j)
// of a lane is
//   m = m0 + wm*128 + 32*i + (lane&31),
//   n = n0 + wn*128 + 32*j + 8*(r>>2) + 4*(lane>>5) + (r&3):
// one output row per lane and four consecutive columns per group of four
// registers, stored as one 8-byte (fp16) or 16-byte (fp32 / int32) write.
//
// rsx[i]: sx[m]/127 for the lane's row of block i (prefetched by the caller);
// scol: LDS copy of sw[n0 .. n0+256) / 127.
template <int MODE, bool XBF16>
__device__ __forceinline__ void epilogue(v16i (&acc)[4][4], int M, int N, int m0, int n0, int wm, int wn, int lane,
                                         const float (&rsx)[4], const float* scol, int nO,
                                         const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
                                         void* __restrict__ Y) {
  const int fr = lane & 31, fh = lane >> 5;
  const bool vec = (N & 3) == 0;            // 4 consecutive columns are aligned and in one row
  auto col_of = [&](int j, int g) { return n0 + wn * 128 + 32 * j + 8 * g + 4 * fh; };

  if constexpr (MODE == 0) {
    int32_t* y = static_cast<int32_t*>(Y);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + 32 * i + fr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = col_of(j, g);
          int32_t* dst = y + static_cast<int64_t>(m) * N + n;
          if (vec && n + 3 < N) {
            *reinterpret_cast<v4i*>(dst) =
                v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) dst[e] = acc[i][j][4 * g + e];
          }
        }
    }
  } else {
    // side product for one 32-row block at a time: o[j] = WO(block j) . XO(rows of block i)^T
    const int P = (nO + 31) & ~31;
    using V8 = typename std::conditional<XBF16, v8bf, v8h>::type;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + 32 * i + fr;
      v16f o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[j][r] = 0.0f;
      const int64_t xrow = static_cast<int64_t>(min(m, M - 1)) * P;
      for (int c = 0; c < P; c += 16) {
        const V8 xb = *reinterpret_cast<const V8*>(XO + xrow + c + 8 * fh);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const V8 wa = *reinterpret_cast<const V8*>(
              WO + static_cast<int64_t>(min(n0 + wn * 128 + 32 * j + fr, N - 1)) * P + c + 8 * fh);
          if constexpr (XBF16)
            o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xb, o[j], 0, 0, 0);
          else
            o[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa, xb, o[j], 0, 0, 0);
        }
      }
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = col_of(j, g);
          const v4f cs = *reinterpret_cast<const v4f*>(scol + (n - n0));
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            y[e] = (static_cast<float>(acc[i][j][4 * g + e]) * rsx[i] + o[j][4 * g + e]) * cs[e];
          if constexpr (MODE == 1) {
            uint16_t* dst = static_cast<uint16_t*>(Y) + static_cast<int64_t>(m) * N + n;
            if (vec && n + 3 < N) {
              const uint32_t lo = f32_to_f16_bits(y[0]) | (static_cast<uint32_t>(f32_to_f16_bits(y[1])) << 16);
              const uint32_t hi = f32_to_f16_bits(y[2]) | (static_cast<uint32_t>(f32_to_f16_bits(y[3])) << 16);
              *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = f32_to_f16_bits(y[e]);
            }
          } else {
            float* dst = static_cast<float*>(Y) + static_cast<int64_t>(m) * N + n;
            if (vec && n + 3 < N) {
              *reinterpret_cast<v4f*>(dst) = v4f{y[0], y[1], y[2], y[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) dst[e] = y[e];
            }
          }
        }
    }
  }
}

// Per-tile epilogue inputs, loaded at tile start so their latency hides under
// the K loop: this lane's four row scales, one column scale per thread (later
// staged through LDS), and the outlier count.
struct EpiIn {
  float rsx[4];
  float my_sw;
  int nO;
};

template <int MODE>
__device__ __forceinline__ void epi_prefetch(EpiIn& e, int M, int N, int m0, int n0, int wm, int lane,
                                             const float* __restrict__ sx, const float* __restrict__ sw,
                                             const int* __restrict__ nO_ptr) {
  if constexpr (MODE != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = sx[min(m0 + wm * 128 + 32 * i + (lane & 31), M - 1)];
    e.my_sw = sw[min(n0 + static_cast<int>(threadIdx.x), N - 1)];
    e.nO = *nO_ptr;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = 0.0f;
    e.my_sw = 0.0f;
    e.nO = 0;
  }
}

// Finishes the prefetch (divides by 127, publishes the column scales in
// `scol`, 256 floats of LDS no longer used by the K loop) and runs the
// epilogue. Every wave of the block must call it.
template <int MODE, bool XBF16>
__device__ __forceinline__ void finish_tile(v16i (&acc)[4][4], EpiIn& e, float* scol, int M, int N, int m0, int n0,
                                            int wm, int wn, int lane, const uint16_t* __restrict__ XO,
                                            const uint16_t* __restrict__ WO, void* __restrict__ Y) {
  if constexpr (MODE != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = e.rsx[i] / 127.0f;
    scol[threadIdx.x] = e.my_sw / 127.0f;
    __syncthreads();
  }
  epilogue<MODE, XBF16>(acc, M, N, m0, n0, wm, wn, lane, e.rsx, scol, e.nO, XO, WO, Y);
}

__device__ __forceinline__ void zero_acc(v16i (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
}

// ---------------------------------------------------------------------------
// General kernel (any K % 16 == 0): register-staged loads with zero fill past
// K, two LDS stages. MODE 0: raw int32 accumulators to Y (int32 [M,N]);
// 1: fp16 Y; 2: fp32 Y.
template <int MODE, bool XBF16>
__global__ __launch_bounds__(256, 1) void k_int8_gemm(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                      int M, int N, int K, const float* __restrict__ sx,
                                                      const float* __restrict__ sw, const int* __restrict__ nO_ptr,
                                                      const uint16_t* __restrict__ XO,
                                                      const uint16_t* __restrict__ WO, void* __restrict__ Y,
                                                      int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t lds[2][2][kBM * kBK];
  __shared__ float scol[kBN];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  EpiIn ein;
  epi_prefetch<MODE>(ein, M, N, m0, n0, wm, lane, sx, sw, nO_ptr);

  // this thread moves logical chunk (tid & 3) of rows tid/4 + 64*i
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

  v16i acc[4][4];
  zero_acc(acc);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    mma_step(lds[st][0], lds[st][1], acc, wm, wn, lane);
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }
  finish_tile<MODE, XBF16>(acc, ein, scol, M, N, m0, n0, wm, wn, lane, XO, WO, Y);
}

// ---------------------------------------------------------------------------
// Pipelined kernel for K % 64 == 0.
//  * Operands go straight from global memory into LDS with
//    global_load_lds_dwordx4 (no staging registers) through a ring of S
//    stages; each wave-level load writes 1 KB of contiguous LDS (lane l at
//    +16*l), so the swizzle is obtained by choosing, per lane, which global
//    chunk lands in that slot. Completion is tracked with explicit vmcnt waits
//    (the compiler does not see the LDS side of these loads).
//  * MFMA operands are software-pipelined: while the 16 MFMAs of one 32-byte
//    sub-step run, the fragments of the next sub-step are read from LDS, the
//    reads interleaved between the MFMAs. One barrier per K-step, placed
//    between the two sub-steps, publishes the next stage and retires the
//    current one (whose slot the next DMA refills).

// s_waitcnt with only a vmcnt limit (expcnt/lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt with only an lgkmcnt limit.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

__device__ __forceinline__ void block_barrier() {
  // a scheduling/memory fence for the compiler, and the hardware barrier
  __asm__ volatile("s_barrier" ::: "memory");
}

// A and B fragments of one 32-byte sub-step: f[0..3] rows of A, f[4..7] of B.
__device__ __forceinline__ void load_frags(const int8_t* sa, int sub, int wm, int wn, int lane, v4i (&f)[8]) {
  const int fr = lane & 31, fh = lane >> 5;
  const int8_t* sb = sa + kBM * kBK;
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = *reinterpret_cast<const v4i*>(sa + swz64(wm * 128 + i * 32 + fr, 2 * sub + fh));
#pragma unroll
  for (int j = 0; j < 4; ++j) f[4 + j] = *reinterpret_cast<const v4i*>(sb + swz64(wn * 128 + j * 32 + fr, 2 * sub + fh));
}

__device__ __forceinline__ void mfma_sub(const v4i (&f)[8], v16i (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[4 + j], f[i], acc[i][j], 0, 0, 0);
}

// One 32-byte sub-step as 8 fixed groups of {2 MFMAs on the current
// fragments, 1 LDS read of the next fragments, [1 DMA of a future K-step]}.
// sched_barrier keeps the order: the loads are spread over the MFMA
// shadow instead of stalling the wave's in-order issue in a burst.
template <bool DMA>
__device__ __forceinline__ void mma_phase(const v4i (&fm)[8], v16i (&acc)[4][4], const int8_t* sfr, int sub,
                                          int wm, int wn, int lane, v4i (&fl)[8],
                                          const int8_t* const (&a_src)[4], const int8_t* const (&b_src)[4],
                                          int k0, int8_t* st, int wave) {
  const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p0 = 2 * t, p1 = 2 * t + 1;
    acc[p0 >> 2][p0 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p0 & 3)], fm[p0 >> 2], acc[p0 >> 2][p0 & 3], 0, 0, 0);
    acc[p1 >> 2][p1 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p1 & 3)], fm[p1 >> 2], acc[p1 >> 2][p1 & 3], 0, 0, 0);
    if (t < 4)
      fl[t] = *reinterpret_cast<const v4i*>(sfr + swz64(wm * 128 + t * 32 + fr, 2 * sub + fh));
    else
      fl[t] = *reinterpret_cast<const v4i*>(sfr + kBM * kBK + swz64(wn * 128 + (t - 4) * 32 + fr, 2 * sub + fh));
    if (DMA) {
      if (t < 4)
        __builtin_amdgcn_global_load_lds(a_src[t] + k0, st + (wave * 4 + t) * 1024, 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(b_src[t - 4] + k0, st + kBM * kBK + (wave * 4 + t - 4) * 1024, 16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int MODE, bool XBF16, int S>
__global__ __launch_bounds__(256, 1) void k_int8_gemm_dma(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                          int M, int N, int K, const float* __restrict__ sx,
                                                          const float* __restrict__ sw, const int* __restrict__ nO_ptr,
                                                          const uint16_t* __restrict__ XO,
                                                          const uint16_t* __restrict__ WO, void* __restrict__ Y,
                                                          int tiles_m, int tiles_n) {
  constexpr int kStage = 2 * kBM * kBK;       // A then B, 32 KB
  constexpr int kLoads = 8;                   // DMA instructions per wave per step
  __shared__ __attribute__((aligned(1024))) int8_t lds[S * kStage];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  EpiIn ein;
  epi_prefetch<MODE>(ein, M, N, m0, n0, wm, lane, sx, sw, nO_ptr);

  // DMA source of this lane for load instruction i (0..3) of each operand:
  // tile row r = wave*64 + 16*i + lane/4 lands in LDS slot (lane & 3) of that
  // row, which holds logical 16-byte chunk (lane & 3) ^ swz_term(r).
  const int8_t* a_src[4];
  const int8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 64 + 16 * i + (lane >> 2);
    const int ch = (lane & 3) ^ swz_term(r);
    a_src[i] = A + static_cast<int64_t>(min(m0 + r, M - 1)) * K + ch * 16;
    b_src[i] = B + static_cast<int64_t>(min(n0 + r, N - 1)) * K + ch * 16;
  }
  const int nk = K / kBK;
  // DMA of K-step kt into its ring slot. Past the last step the load repeats
  // the last step's data into the slot just retired, which no later step
  // reads: every iteration then issues the same number of loads, so the wait
  // below is one constant.
  auto issue = [&](int kt) {
    int8_t* st = lds + (kt % S) * kStage;
    const int k0 = min(kt, nk - 1) * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds(a_src[i] + k0, st + (wave * 4 + i) * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(b_src[i] + k0, st + kBM * kBK + (wave * 4 + i) * 1024, 16, 0, 0);
    }
  };

  v16i acc[4][4];
  zero_acc(acc);

  for (int s = 0; s < S; ++s) issue(s);
  wait_vmcnt<(S - 1) * kLoads>();                 // step 0 landed (this wave)
  block_barrier();                                // ... for every wave
  v4i f0[8], f1[8];
  load_frags(lds, 0, wm, wn, lane, f0);
  for (int kt = 0; kt < nk - 1; ++kt) {
    int8_t* sa = lds + (kt % S) * kStage;
    // sub-step 0 multiplies while sub-step 1's fragments are read
    mma_phase<false>(f0, acc, sa, 1, wm, wn, lane, f1, a_src, b_src, 0, nullptr, wave);
    wait_lgkmcnt<0>();                            // this slot is fully read
    wait_vmcnt<(S - 2) * kLoads>();               // step kt+1 landed (this wave)
    block_barrier();                              // ... for every wave; slot kt retired
    // sub-step 1 multiplies while step kt+1's first fragments are read and
    // step kt+S is fetched into the retired slot
    mma_phase<true>(f1, acc, lds + ((kt + 1) % S) * kStage, 0, wm, wn, lane, f0, a_src, b_src,
                    min(kt + S, nk - 1) * kBK, sa, wave);
  }
  load_frags(lds + ((nk - 1) % S) * kStage, 1, wm, wn, lane, f1);
  mfma_sub(f0, acc);
  mfma_sub(f1, acc);
  wait_vmcnt<0>();                                // retire the trailing repeat loads
  block_barrier();                                // every wave is done with the ring
  finish_tile<MODE, XBF16>(acc, ein, reinterpret_cast<float*>(lds), M, N, m0, n0, wm, wn, lane, XO, WO, Y);
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
#define W8_GEMM_ARGS A, B, m, n, k, sx, sw, nO, XO, WO, Y, tiles_m, tiles_n
  if (K % kBK == 0) {
    constexpr int S = 4;
    if (mode == 0) k_int8_gemm_dma<0, true, S><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1 && xbf16) k_int8_gemm_dma<1, true, S><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1) k_int8_gemm_dma<1, false, S><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (xbf16) k_int8_gemm_dma<2, true, S><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else k_int8_gemm_dma<2, false, S><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
  } else {
    if (mode == 0) k_int8_gemm<0, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1 && xbf16) k_int8_gemm<1, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1) k_int8_gemm<1, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (xbf16) k_int8_gemm<2, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else k_int8_gemm<2, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
  }
#undef W8_GEMM_ARGS
}

}  // namespace w8
