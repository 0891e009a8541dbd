// W4A8 linear for gfx950: int4 weights with one fp32 scale per group of 128
// K values, int8 activations with one scale per token, on the int8 MFMA.
//
//   acc_g[m,n] = sum_{k in group g} qx[m,k] * qw[n,k]           (exact, int32)
//   Y[m,n]     = (sx[m] / 127) * sum_g acc_g[m,n] * sw[g,n] / 7  (fp32)
//
// "Qwen-Image-fni8" card, section "Format": int4 per-group weights, int8
// activations, fp32 scales; its dp4a kernels and resident layout are prior
// art. Here the contraction runs on v_mfma_i32_32x32x32_i8: the packed int4
// codes go to LDS as they are (half the bytes of int8 weights) and every wave
// widens its fragments in registers. Storage: two codes per byte, 8 per 32-bit
// word; byte b of word c of a row holds k = 8c + b (low nibble) and
// k = 8c + b + 4 (high nibble). Then `w & 0xF0F0F0F0` and
// `(w << 4) & 0xF0F0F0F0` are the int8 bytes 16*q of k = 8c+4..8c+7 and
// k = 8c..8c+3: no sign extension is needed, and the factor 16 (exact) goes
// into the group scale. Scales are group-major, sw[g, n].
//
// Activations are coded per token by the int8 path's row pass with no outlier
// columns (threshold +inf).
#include <algorithm>

#include "launch.h"
#include "tile.h"

namespace w8 {

// ---------------------------------------------------------------------------
// Weight quantisation: one group (128 values of one row) per 16 lanes; a lane
// encodes 8 consecutive values into one packed word.
//   s = max |w| over the group (fp32), r = fl32(7 / s),
//   q = clamp(rne(fl32(w * r)), -7, 7), 0 when s == 0 or w == 0.
__device__ __forceinline__ int int4_code(float x, float r) {
  if (x == 0.0f) return 0;
  float p = __builtin_rintf(x * r);
  p = fminf(fmaxf(p, -7.0f), 7.0f);
  return static_cast<int>(p);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_int4_groups(const uint16_t* __restrict__ W, int64_t N, int K,
                                                     uint32_t* __restrict__ packed, float* __restrict__ sw) {
#pragma clang fp contract(off)
  const int groups = K / kW4Group;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  const bool live = gid < N * groups;
  const int64_t n = live ? gid / groups : 0;
  const int g = live ? static_cast<int>(gid % groups) : 0;
  float f[8];
  if (live) {
    const uint4 v = reinterpret_cast<const uint4*>(W + n * K + g * kW4Group)[l16];
    unpack8<BF16>(v, f);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(f[e]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 16));
  const float r = 7.0f / a;                     // IEEE division; +inf for a == 0 (codes are 0 then)
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t lo = static_cast<uint32_t>(a == 0.0f ? 0 : int4_code(f[b], r)) & 0xFu;
    const uint32_t hi = static_cast<uint32_t>(a == 0.0f ? 0 : int4_code(f[b + 4], r)) & 0xFu;
    w |= (lo | (hi << 4)) << (8 * b);
  }
  if (live) {
    packed[n * (K / 8) + g * (kW4Group / 8) + l16] = w;
    if (l16 == 0) sw[static_cast<int64_t>(g) * N + n] = a;
  }
}

void launch_int4_weights(const void* W, bool bf16, int64_t N, int K, uint8_t* packed, float* sw, hipStream_t s) {
  const int64_t groups = N * (K / kW4Group);
  const dim3 grid(static_cast<unsigned>((groups + 15) / 16)), block(256);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  if (bf16) k_int4_groups<true><<<grid, block, 0, s>>>(w, N, K, p, sw);
  else k_int4_groups<false><<<grid, block, 0, s>>>(w, N, K, p, sw);
}

// ---------------------------------------------------------------------------
// GEMM. Block 128x128, 4 waves as 2x2, each 64x64 = 2x2 tiles of 32x32; K step
// 64 values: A (int8 codes) 128 rows x 64 bytes, B (packed int4) 128 rows x
// 32 bytes, a ring of kW4Stages such stages; two blocks per CU. The MFMAs take
// the activation fragment first, so element r of tile (i, j) of a lane is
//   m = m0 + wm*64 + 32*i + 8*(r>>2) + 4*(lane>>5) + (r&3),
//   n = n0 + wn*64 + 32*j + (lane&31):
// a lane owns one output column per tile column j, and so needs one group
// scale per j. Each group (two K steps) accumulates in int32 from zero and is
// folded into fp32 sums with its scale sw[g,n] / 7 / 16.
constexpr int kW4BM = 128;
constexpr int kW4AStage = kW4BM * 64;          // 8 KB
constexpr int kW4Stage = kW4AStage + kW4BM * 32;   // + 4 KB
constexpr int kW4Stages = 6;
constexpr int kW4ALoads = 2;                   // DMA instructions per wave per step (A)
constexpr int kW4Loads = 3;                    // + 1 (B)
constexpr int kW4PartBytes = kW4BM * kW4BM * 4;
constexpr int kW4Chunks = 16;                  // 16-byte accumulator chunks per lane

// B rows: two 16-byte chunks, swapped on every other group of 8 rows (chunk
// ^ ((row >> 3) & 1)); a lane reads the 8-byte half fh of chunk s.
__device__ __forceinline__ int swz_b32(int row, int ch) { return row * 32 + ((ch ^ ((row >> 3) & 1)) << 4); }

__device__ __forceinline__ void w4_dma(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ v16i mfma_w4(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Fragments of one 32-value sub-step: a[i] (A rows of tile row i), b[j]
// (B rows of tile column j, widened) and the packed B halves before widening.
struct W4Frags {
  v4i a[2];
  v4i b[2];
  v2u raw[2];
};

__device__ __forceinline__ void w4_read(W4Frags& F, const uint8_t* sl, int h, int wm, int wn, int fr, int fh) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = wn * 64 + 32 * j + fr;
    F.raw[j] = *reinterpret_cast<const v2u*>(sl + kW4AStage + swz_b32(row, h) + 8 * fh);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + 32 * i + fr;
    F.a[i] = *reinterpret_cast<const v4i*>(sl + swz64(row, 2 * h + fh));
  }
}

__device__ __forceinline__ void w4_widen(W4Frags& F) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t w0 = F.raw[j][0], w1 = F.raw[j][1];
    F.b[j] = v4i{static_cast<int>((w0 << 4) & 0xF0F0F0F0u), static_cast<int>(w0 & 0xF0F0F0F0u),
                 static_cast<int>((w1 << 4) & 0xF0F0F0F0u), static_cast<int>(w1 & 0xF0F0F0F0u)};
  }
}

// DMA of K step kt into its ring slot (repeats the last step past the end).
__device__ __forceinline__ void w4_issue(uint8_t* lds, int kt, int nk, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, const uint32_t* a_off, uint32_t b_off,
                                         int wave) {
  uint8_t* st = lds + (kt % kW4Stages) * kW4Stage;
  const uint32_t k0 = static_cast<uint32_t>(min(kt, nk - 1));
#pragma unroll
  for (int d = 0; d < kW4ALoads; ++d) w4_dma(ra, st + (wave * kW4ALoads + d) * 1024, a_off[d], k0 * 64u);
  w4_dma(rb, st + kW4AStage + wave * 1024, b_off, k0 * 32u);
}

// YDT: 0 bf16, 1 fp16, 2 fp32. Grid and split-K protocol as in the FP8 W8A8
// kernel (slices of whole groups; fp32 partials summed in slice order).
template <int YDT>
__global__ __launch_bounds__(256, 2) void k_w4a8_gemm(const int8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                      int M, int N, int K, const float* __restrict__ sx,
                                                      const float* __restrict__ sw, void* __restrict__ Y,
                                                      int tiles_m, int tiles_n, int dp_tiles, int split,
                                                      float* __restrict__ part, int* __restrict__ cnt) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kW4Stages * kW4Stage];
  static_assert(sizeof(lds) >= kEpiLds + 4, "epilogue LDS and arrival flag");
  int* const s_last = reinterpret_cast<int*>(lds + kEpiLds);

  const int ng_all = K / kW4Group;
  int tm, tn, gb = 0, ge = ng_all;
  int slot = -1, sk_tile = 0, R = 0;
  if (static_cast<int>(blockIdx.x) < dp_tiles) {
    tile_coords(blockIdx.x, dp_tiles, tiles_m, tiles_n, tm, tn);
  } else {
    const int nu = gridDim.x - dp_tiles;
    const int v = xcd_remap(blockIdx.x - dp_tiles, nu);
    R = nu / split;
    const int piece = v / R;
    sk_tile = v % R;
    slot = v;
    group_tile(dp_tiles + sk_tile, tiles_m, tiles_n, tm, tn);
    gb = piece * ng_all / split;
    ge = (piece + 1) * ng_all / split;
  }
  const int m0 = tm * kW4BM, n0 = tn * kW4BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  const int kb = gb * (kW4Group / 64);          // first K step of the slice
  const int nk = (ge - gb) * (kW4Group / 64);

  // DMA sources as byte offsets. A: load d of wave w covers rows
  // (2w + d)*16 + lane/4, chunk (lane & 3) ^ swz_term(row). B: rows
  // w*32 + lane/2, chunk (lane & 1) ^ ((row >> 3) & 1).
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(A), 0, static_cast<int>(static_cast<uint32_t>(M) * static_cast<uint32_t>(K)), kRawBuffer);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B), 0, static_cast<int>(static_cast<uint32_t>(N) * static_cast<uint32_t>(K / 2)),
      kRawBuffer);
  uint32_t a_off[kW4ALoads];
#pragma unroll
  for (int d = 0; d < kW4ALoads; ++d) {
    const int r = (wave * kW4ALoads + d) * 16 + (lane >> 2);
    const int ch = (lane & 3) ^ swz_term(r);
    a_off[d] = static_cast<uint32_t>(min(m0 + r, M - 1)) * static_cast<uint32_t>(K) + kb * 64 + ch * 16;
  }
  uint32_t b_off;
  {
    const int r = wave * 32 + (lane >> 1);
    const int ch = (lane & 1) ^ ((r >> 3) & 1);
    b_off = static_cast<uint32_t>(min(n0 + r, N - 1)) * static_cast<uint32_t>(K / 2) + kb * 32 + ch * 16;
  }

  // the lane's two output columns, and their group scales read one group ahead
  int ncol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ncol[j] = min(n0 + wn * 64 + 32 * j + fr, N - 1);

  v16f facc[2][2];
  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) facc[i][j][r] = 0.0f;
  const v16i zero16 = {};

  // group scales of the lane's columns, read two groups ahead: a load's wait
  // then falls behind the ring's own (loads complete in order), where a wait
  // for a scale read one group ahead would drain the ring at every group
  const int ng = ge - gb;
  float gs[2], gs1[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    gs[j] = sw[static_cast<int64_t>(gb) * N + ncol[j]];
    gs1[j] = ng > 1 ? sw[static_cast<int64_t>(gb + 1) * N + ncol[j]] : 0.0f;
  }
  for (int s = 0; s < kW4Stages; ++s) w4_issue(lds, s, nk, ra, rb, a_off, b_off, wave);
  W4Frags fa, fb;
  // One group = two K steps = four sub-steps. Step kt: wait until it has
  // landed (this wave's loads, then every wave's: the barrier), which also
  // retires step kt-1's slot, refilled at once with step kt-1+S (past the end
  // the last step is loaded again, so every step issues the same loads and the
  // wait is one constant after the first). Then its two sub-steps multiply.
  for (int g = 0; g < ng; ++g) {
    float gs2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) gs2[j] = g + 2 < ng ? sw[static_cast<int64_t>(gb + g + 2) * N + ncol[j]] : 0.0f;
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2) {
      const int kt = 2 * g + st2;
      if (kt == 0) wait_vmcnt<(kW4Stages - 1) * kW4Loads>();
      else wait_vmcnt<(kW4Stages - 2) * kW4Loads>();
      block_barrier();
      if (kt >= 1) w4_issue(lds, kt - 1 + kW4Stages, nk, ra, rb, a_off, b_off, wave);
      const uint8_t* sl = lds + (kt % kW4Stages) * kW4Stage;
      w4_read(fa, sl, 0, wm, wn, fr, fh);
      w4_read(fb, sl, 1, wm, wn, fr, fh);
      w4_widen(fa);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_w4(fa.a[i], fa.b[j], st2 == 0 ? zero16 : acc[i][j]);
      w4_widen(fb);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_w4(fb.a[i], fb.b[j], acc[i][j]);
    }
    // fold the group: facc += acc * sw[g,n] / 7 / 16
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float f = (gs[j] / 7.0f) * 0.0625f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          facc[i][j][r] = __builtin_fmaf(static_cast<float>(acc[i][j][r]), f, facc[i][j][r]);
      gs[j] = gs1[j];
      gs1[j] = gs2[j];
    }
  }
  wait_vmcnt<0>();                              // retire the trailing loads
  block_barrier();

  if (slot >= 0) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lane_off = (wv * kW4Chunks * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t mine = partial_rsrc(part, slot, kW4PartBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (i * 2 + j) * 4 + q;
          const v4f v{facc[i][j][4 * q], facc[i][j][4 * q + 1], facc[i][j][4 * q + 2], facc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), mine, lane_off + c * 1024, 0, kSc1);
        }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      *s_last = __hip_atomic_fetch_add(cnt + sk_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == split - 1;
    __syncthreads();
    if (!*s_last) return;
    if (tid == 0) cnt[sk_tile] = 0;
    for (int p = 0; p < split; ++p) {
      const __amdgpu_buffer_rsrc_t src = partial_rsrc(part, p * R + sk_tile, kW4PartBytes);
      v4f w[kW4Chunks];
#pragma unroll
      for (int t = 0; t < kW4Chunks; ++t)
        w[t] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(src, lane_off + t * 1024, 0, kSc1));
#pragma unroll
      for (int t = 0; t < kW4Chunks; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = t >> 3, j = (t >> 2) & 1, r = 4 * (t & 3) + e;
          facc[i][j][r] = p == 0 ? w[t][e] : facc[i][j][r] + w[t][e];
        }
    }
  }

  // Epilogue: y = facc * sx[m] / 127, staged through LDS a 32-row block at a
  // time (64 columns of the wave tile per staged row) and stored as row segments.
  constexpr int EB = YDT == 2 ? 4 : 2;
  constexpr int RB = 64 * EB;                   // 128 or 256 bytes
  const bool vec = (static_cast<int64_t>(N) * EB) % 16 == 0;
  char* const stg = reinterpret_cast<char*>(lds) + kEpiCols + wave * kStgWave;
  char* const y = static_cast<char*>(Y);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rbase = m0 + wm * 64 + 32 * i;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = 8 * (r >> 2) + 4 * fh + (r & 3);
      const float rs = sx[min(rbase + ml, M - 1)] / 127.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float v = facc[i][j][r] * rs;
        char* dst = stg + ml * kStgPitch + (32 * j + fr) * EB;
        if constexpr (YDT == 0) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(bf16_rne_bits(v));
        else if constexpr (YDT == 1) *reinterpret_cast<uint16_t*>(dst) = f32_to_f16_bits(v);
        else *reinterpret_cast<float*>(dst) = v;
      }
    }
    wave_lds_fence();
    flush_staged<EB, RB>(stg, y, M, N, rbase, n0 + wn * 64, lane, vec);
    wave_lds_fence();
  }
}

// ---------------------------------------------------------------------------
// Launch plan: K-slicing (whole groups per slice) for 128x128 blocks, by the
// weight-only planner's kind of model: a lone block step (12 KB) takes
// kW4Lat; two blocks on a CU stream at most kW4CuRate bytes/us; the chip
// kW4L2Rate; partials kW4PartRate after kW4SplitLat; kW4Fixed per launch.
constexpr double kW4Lat = 0.45;
constexpr double kW4CuRate = 46e3;
constexpr double kW4L2Rate = 10e6;
constexpr double kW4PartRate = 5e6;
constexpr double kW4SplitLat = 2.0;
constexpr double kW4Fixed = 3.0;
constexpr int kW4MaxSplit = 16;

static double w4_plan_time(int64_t M, int64_t N, int64_t ng, int s, int cus) {
  const int64_t T = ((M + kW4BM - 1) / kW4BM) * ((N + kW4BM - 1) / kW4BM);
  const int64_t units = T * s;
  const int64_t per_cu = (units + cus - 1) / cus;
  const double steps = static_cast<double>((ng + s - 1) / s) * (kW4Group / 64);
  const double step_bytes = kW4Stage;
  double t = static_cast<double>(units) * steps * step_bytes / kW4L2Rate;
  const double rounds = static_cast<double>((per_cu + 1) / 2);
  const double conc = static_cast<double>(std::min<int64_t>(per_cu, 2));
  t = std::max(t, rounds * steps * std::max(kW4Lat, conc * step_bytes / kW4CuRate));
  if (s > 1) t += (static_cast<double>(units) + static_cast<double>(T) * s) * kW4PartBytes / kW4PartRate + kW4SplitLat;
  return t + kW4Fixed;
}

GemmPlan plan_w4a8_gemm_split(int64_t M, int64_t N, int split) {
  GemmPlan p{};
  p.bm = kW4BM;
  p.tiles_m = static_cast<int>((M + kW4BM - 1) / kW4BM);
  p.tiles_n = static_cast<int>((N + kW4BM - 1) / kW4BM);
  const int T = p.tiles_m * p.tiles_n;
  p.split = split;
  p.dp_tiles = split > 1 ? 0 : T;
  p.sk_tiles = split > 1 ? T : 0;
  return p;
}

GemmPlan plan_w4a8_gemm(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t ng = K / kW4Group;
  double best_t = 0.0;
  int best_s = 1;
  for (int s = 1; s <= std::min<int64_t>(ng, kW4MaxSplit); ++s) {
    const double t = w4_plan_time(M, N, ng, s, std::max(cus, 1));
    if (s == 1 || t < best_t) best_t = t, best_s = s;
  }
  return plan_w4a8_gemm_split(M, N, best_s);
}

// K % 128 == 0 (checked by the caller); plan.split <= K / 128. ydt: 0 bf16,
// 1 fp16, 2 fp32. `part` / `cnt` as for the other split-K GEMMs.
void launch_w4a8_gemm(const int8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                      const float* sw, void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s) {
  const dim3 block(256);
  const dim3 grid(plan.dp_tiles + plan.sk_tiles * plan.split);
#define W8_W4_ARGS A, B, (int)M, (int)N, (int)K, sx, sw, Y, plan.tiles_m, plan.tiles_n, plan.dp_tiles, plan.split, part, cnt
  if (ydt == 0) k_w4a8_gemm<0><<<grid, block, 0, s>>>(W8_W4_ARGS);
  else if (ydt == 1) k_w4a8_gemm<1><<<grid, block, 0, s>>>(W8_W4_ARGS);
  else k_w4a8_gemm<2><<<grid, block, 0, s>>>(W8_W4_ARGS);
#undef W8_W4_ARGS
}

}  // namespace w8
