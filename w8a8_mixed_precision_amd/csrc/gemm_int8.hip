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
#include <algorithm>
#include <type_traits>

#include "launch.h"
#include "produce.h"
#include "tile.h"

namespace w8 {

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

// The 16-bit side-product MFMA behind a plain function (a target builtin with
// template-dependent arguments can make the host compilation pass drop the
// kernel templates that use it).
template <bool XBF16, typename V8>
__device__ __forceinline__ v16f mfma_side(V8 a, V8 b, v16f c) {
  if constexpr (XBF16) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The 16-bit outlier operands of a 256x256 tile, copied into LDS at tile
// start when the padded outlier count P is 32 (at most 32 outlier columns, the
// usual case): XO rows m0 .. m0+255, then WO rows n0 .. n0+255, 64 bytes (32
// values) per row. The four 16-byte chunks of row r are XOR-permuted by
// (r >> 2) & 3, so eight consecutive rows read at one chunk hit distinct banks.
constexpr int kSideRows = 256;
constexpr int kSideLds = 2 * kSideRows * 64;    // 32 KB
__device__ __forceinline__ int side_off(int row, int ch) { return row * 64 + ((ch ^ ((row >> 2) & 3)) << 4); }

// Epilogue staging, one 32-column block of the wave tile at a time: all its
// 32*WT rows x 32 columns go to the wave's staging area (row pitch
// kStgPitchJ), then out as 128-byte row segments, whole cache lines: one
// block of 32-bit outputs, or two neighbouring blocks of fp16 outputs staged
// side by side (a line written in two halves at different times can be
// evicted in between and then costs two line writes). Every element of a
// column block shares the lane's 16 column scales and biases, so these are
// read from LDS once per block.
constexpr int kStgPitchJ = 128 + 16;            // a staged row: 32 x 4 bytes + pad
constexpr int kStgWaveJ = 128 * kStgPitchJ;     // one wave's staged rows (WT <= 4)
constexpr int kEpiLds8 = kEpiCols + 4 * kStgWaveJ;

// Column block j of the wave tile, registers -> staging area:
// y = fl(acc) * rsx[i] (+ o[i]) then * cs + bias, per element; SIDE: o holds
// the block's 16-bit outlier product per 32-row block i. MODE 0 stages the raw
// int32 accumulators. ncol: first column of the block within the block tile.
template <int MODE, bool SIDE, int WT>
__device__ __forceinline__ void stage_cols(const v16i (&acc)[WT][WT], const v16f* o, int j, const float (&rsx)[4],
                                           const float* __restrict__ scol, const float* __restrict__ sbias,
                                           int ncol, int lane, char* __restrict__ stg) {
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int EB = MODE == 1 ? 2 : 4;         // bytes per output element
  v4f cs[4], bs[4];
  if constexpr (MODE != 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      cs[g] = *reinterpret_cast<const v4f*>(scol + ncol + 8 * g + 4 * fh);
      bs[g] = *reinterpret_cast<const v4f*>(sbias + ncol + 8 * g + 4 * fh);
    }
  }
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      char* dst = stg + (32 * i + fr) * kStgPitchJ + (8 * g + 4 * fh) * EB;
      if constexpr (MODE == 0) {
        *reinterpret_cast<v4i*>(dst) =
            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      } else {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = static_cast<float>(acc[i][j][4 * g + e]);
          const float t = SIDE ? __builtin_fmaf(a, rsx[i], o[i][4 * g + e]) : a * rsx[i];
          v[e] = __builtin_fmaf(t, cs[g][e], bs[g][e]);
        }
        if constexpr (MODE == 1) {
          const uint32_t lo = f32x2_to_f16x2_bits(v[0], v[1]);
          const uint32_t hi = f32x2_to_f16x2_bits(v[2], v[3]);
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
        }
      }
    }
}

// Writes the R staged rows (128 bytes each: 128 / EB elements) to Y rows
// m_base.. and columns n_base.. (clipped to [M, N)): every lane stores
// 16-byte chunks, 8 rows per instruction, reading at most 8 chunks from LDS
// ahead of their stores. vec: rows of Y are 16-byte aligned.
template <int EB, int R>
__device__ __forceinline__ void flush_cols(const char* stg, char* __restrict__ y, int M, int N, int m_base,
                                           int n_base, int lane, bool vec) {
  constexpr int EPC = 16 / EB;                  // elements per 16-byte chunk
  constexpr int CPR = 8;                        // chunks per staged row
  constexpr int RPI = 64 / CPR;                 // rows per instruction
  constexpr int T = R / RPI;                    // store instructions
  constexpr int TB = T > 8 ? 8 : T;             // chunks read ahead
  const int ch = lane % CPR;
  // wave-uniform block origin (the callers' row index is a per-lane copy)
  const int mb = __builtin_amdgcn_readfirstlane(m_base), nb = __builtin_amdgcn_readfirstlane(n_base);
  if (vec && mb + R <= M && nb + CPR * EPC <= N && static_cast<int64_t>(R) * N * EB < (int64_t{1} << 31)) {
    // Interior block: every staged row and column lies in [M, N). One buffer
    // store per chunk from the block origin: the lane's row and column in the
    // per-lane offset, the 8-row step of each store in the scalar offset, so
    // no address arithmetic or bounds test per store. The stores (here and
    // in the edge path below) are marked non-temporal: the output is not read
    // again by the GEMM, and the hint keeps it from displacing the operand
    // panels the other blocks of the XCD stream through the same L2 (DiT
    // 1024^2 int8 step 857 -> 841 us and 830 -> 816 us, A/B on two boxes; the
    // same hint in the FP8 and weight-only epilogues measured no change).
    const uint32_t rowb = static_cast<uint32_t>(N) * EB;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        y + (static_cast<int64_t>(mb) * N + nb) * EB, 0, static_cast<int>(R * rowb), kRawBuffer);
    const uint32_t voff = static_cast<uint32_t>(lane / CPR) * rowb + ch * 16;
#pragma unroll
    for (int t0 = 0; t0 < T; t0 += TB) {
      uint4 v[TB];
#pragma unroll
      for (int t = 0; t < TB; ++t)
        v[t] = *reinterpret_cast<const uint4*>(stg + (RPI * (t0 + t) + lane / CPR) * kStgPitchJ + ch * 16);
#pragma unroll
      for (int t = 0; t < TB; ++t)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v[t]), rs, voff,
                                               static_cast<int>(static_cast<uint32_t>(RPI * (t0 + t)) * rowb), kNt);
    }
    return;
  }
  const int n = n_base + ch * EPC;
#pragma unroll
  for (int t0 = 0; t0 < T; t0 += TB) {
    uint4 v[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t)
      v[t] = *reinterpret_cast<const uint4*>(stg + (RPI * (t0 + t) + lane / CPR) * kStgPitchJ + ch * 16);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int m = m_base + RPI * (t0 + t) + lane / CPR;
      if (m < M) {
        char* dst = y + (static_cast<int64_t>(m) * N + n) * EB;
        if (vec && n + EPC <= N) {
          __builtin_nontemporal_store(__builtin_bit_cast(v4u, v[t]), reinterpret_cast<v4u*>(dst));
        } else {
          const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if (n + e >= N) break;
            if constexpr (EB == 2)
              *reinterpret_cast<uint16_t*>(dst + 2 * e) = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
            else
              *reinterpret_cast<uint32_t*>(dst + 4 * e) = w[e];
          }
        }
      }
    }
  }
}

// More outlier columns than the XO/WO staging holds (kOutCap): the whole
// block gathers 32 of them at a time into an LDS area laid out like the
// tile-start staging (side_off), from X (made from H by the producer) and from
// Wq, through the ascending outlier list: rows m0 .. m0+R-1 of X, then rows
// n0 .. n0+R-1 of Wq (R = 64 WT, clamped into [M, N); slots past nO are 0).
template <bool XBF16, int WT>
__device__ __forceinline__ void gather_side_chunk(char* buf, const SideSrc& src, int M, int N, int m0, int n0,
                                                  int c0, int nO) {
  constexpr int R = 64 * WT;
  using E = typename std::conditional<XBF16, __bf16, _Float16>::type;
#pragma unroll 1
  for (int idx = threadIdx.x; idx < 2 * R * 32; idx += 256) {
    const int row = idx >> 5, jj = idx & 31, j = c0 + jj;
    const bool xrow = row < R;
    const int r = xrow ? row : row - R;
    uint32_t v = 0;
    if (j < nO) {
      const int k = src.O[j];
      if (xrow) {
        const int m = min(m0 + r, M - 1);
        const float rstd = src.prod == kProdRms ? src.pa.rstd[m] : 0.0f;
        v = produce1_any<XBF16>(src.prod, src.H[static_cast<int64_t>(m) * src.K + k], k, rstd, src.pa);
      } else {
        const int n = min(n0 + r, N - 1);
        v = __builtin_bit_cast(uint16_t, static_cast<E>(static_cast<float>(src.Wq[static_cast<int64_t>(n) * src.K + k])));
      }
    }
    char* base = buf + (xrow ? 0 : kSideRows * 64);
    *reinterpret_cast<uint16_t*>(base + side_off(r, jj >> 3) + (jj & 7) * 2) = static_cast<uint16_t>(v);
  }
}

// o[i] += the outlier product of one 32-column block over 32 outlier columns
// staged in LDS (side_off layout: X rows, then W rows from kSideRows).
template <bool XBF16, int WT>
__device__ __forceinline__ void side_from_lds(v16f* o, const char* side, int ncol, int wm, int fr, int fh) {
  using V8 = typename std::conditional<XBF16, v8bf, v8h>::type;
  const char* sx_rows = side;
  const char* sw_rows = side + kSideRows * 64;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const V8 wa = *reinterpret_cast<const V8*>(sw_rows + side_off(ncol + fr, 2 * c + fh));
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      const V8 xb = *reinterpret_cast<const V8*>(sx_rows + side_off(wm * 32 * WT + 32 * i + fr, 2 * c + fh));
      o[i] = mfma_side<XBF16>(wa, xb, o[i]);
    }
  }
}

// Epilogue shared by the GEMM kernels, for a wave tile of WT x WT 32x32 MFMA
// tiles (WT = 4: 256x256 blocks, 2: 128x128 blocks). The MFMAs compute each
// tile transposed (Wq fragment as the first operand), so element r of tile
// (i, j) of a lane is
//   m = m0 + wm*32*WT + 32*i + (lane&31),
//   n = n0 + wn*32*WT + 32*j + 8*(r>>2) + 4*(lane>>5) + (r&3).
// Staged one column block j at a time (stage_cols) and written in whole
// 128-byte row segments (flush_cols).
//
// rsx[i]: sx[m]/127 for the lane's row of block i (prefetched by the caller);
// scol, sbias: LDS copies of sw[n0 .. n0+64*WT) / 127 and of the bias there
// (zeros without one); side: the tile's outlier operands in LDS (side_off
// layout; null: none were staged); stg: this wave's staging area (kStgWaveJ).
template <int MODE, bool XBF16, int WT = 4>
__device__ __forceinline__ void epilogue(v16i (&acc)[WT][WT], int M, int N, int m0, int n0, int wm, int wn, int lane,
                                         const float (&rsx)[4], const float* scol, const float* sbias, int nO,
                                         const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
                                         const SideSrc& src, const char* side, char* side_buf, void* __restrict__ Y,
                                         char* stg) {
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int EB = MODE == 1 ? 2 : 4;         // bytes per output element
  constexpr int WR = 32 * WT;                   // rows (= columns) of the wave tile
  constexpr bool PAIR = EB == 2;                // two column blocks per staged row
  static_assert(WT % 2 == 0, "column blocks pair up");
  const int P = (nO + 31) & ~31;
  const bool vec = (static_cast<int64_t>(N) * EB) % 16 == 0;
  using V8 = typename std::conditional<XBF16, v8bf, v8h>::type;
  char* const y = static_cast<char*>(Y);
  // an opaque copy: the row indices below are then recomputed here rather than
  // kept live across the K loop from the prologue's identical expressions
  int row0 = m0 + wm * WR;
  __asm__ volatile("" : "+v"(row0));
#pragma unroll
  for (int j = 0; j < WT; ++j) {
    const int ncol = wn * WR + 32 * j;
    const int soff = PAIR ? (j & 1) * 64 : 0;   // byte offset of the block in a staged row
    if (MODE == 0 || P == 0) {
      stage_cols<MODE, false, WT>(acc, nullptr, j, rsx, scol, sbias, ncol, lane, stg + soff);
    } else {
      // side product for this column block: o[i] = WO(block j) . XO(rows of block i)^T
      v16f o[WT];
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
      if (side && P == 32) {
        side_from_lds<XBF16, WT>(o, side, ncol, wm, fr, fh);
      } else if (P <= kOutCap) {
        const int64_t wrow = static_cast<int64_t>(min(n0 + ncol + fr, N - 1)) * P;
        for (int c = 0; c < P; c += 16) {
          const V8 wa = *reinterpret_cast<const V8*>(WO + wrow + c + 8 * fh);
#pragma unroll
          for (int i = 0; i < WT; ++i) {
            const V8 xb = *reinterpret_cast<const V8*>(
                XO + static_cast<int64_t>(min(row0 + 32 * i + fr, M - 1)) * P + c + 8 * fh);
            o[i] = mfma_side<XBF16>(wa, xb, o[i]);
          }
        }
      } else {
        // every wave runs this branch (P is the block's), so the barriers match
        for (int c0 = 0; c0 < P; c0 += 32) {
          __syncthreads();                      // the previous chunk is fully read
          gather_side_chunk<XBF16, WT>(side_buf, src, M, N, m0, n0, c0, nO);
          __syncthreads();
          side_from_lds<XBF16, WT>(o, side_buf, ncol, wm, fr, fh);
        }
      }
      stage_cols<MODE, true, WT>(acc, o, j, rsx, scol, sbias, ncol, lane, stg + soff);
    }
    if (PAIR && (j & 1) == 0) continue;         // the pair's second block completes the lines
    wave_lds_fence();
    flush_cols<EB, WR>(stg, y, M, N, row0, n0 + ncol - (PAIR ? 32 : 0), lane, vec);
    wave_lds_fence();                           // staging reads done before the next block writes
  }
}

// Per-tile epilogue inputs, loaded at tile start so their latency hides under
// the K loop: this lane's four row scales, one column scale per thread (later
// staged through LDS), and the outlier count.
struct EpiIn {
  float rsx[4];
  float my_sw;
  float my_bias;
  int nO;
};

template <int MODE, int WT = 4>
__device__ __forceinline__ void epi_prefetch(EpiIn& e, int M, int N, int m0, int n0, int wm, int lane,
                                             const float* __restrict__ sx, const float* __restrict__ sw,
                                             const float* __restrict__ bias, const int* __restrict__ nO_ptr) {
  if constexpr (MODE != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = sx[min(m0 + wm * 32 * WT + 32 * i + (lane & 31), M - 1)];
    e.my_sw = sw[min(n0 + static_cast<int>(threadIdx.x), N - 1)];
    e.my_bias = bias ? bias[min(n0 + static_cast<int>(threadIdx.x), N - 1)] : 0.0f;
    e.nO = *nO_ptr;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = 0.0f;
    e.my_sw = 0.0f;
    e.my_bias = 0.0f;
    e.nO = 0;
  }
}

// Finishes the prefetch (divides by 127, publishes the column scales in LDS)
// and runs the epilogue. `lds` is at least kEpiLds8 bytes of LDS that the K loop
// no longer uses. Every wave of the block must call it.
template <int MODE, bool XBF16, int WT = 4>
__device__ __forceinline__ void finish_tile(v16i (&acc)[WT][WT], EpiIn& e, char* lds, int M, int N, int m0, int n0,
                                            int wm, int wn, int lane, const uint16_t* __restrict__ XO,
                                            const uint16_t* __restrict__ WO, const SideSrc& src, const char* side,
                                            char* side_buf, void* __restrict__ Y) {
  float* scol = reinterpret_cast<float*>(lds);
  float* sbias = scol + 256;
  if constexpr (MODE != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e.rsx[i] = e.rsx[i] / 127.0f;
    scol[threadIdx.x] = e.my_sw / 127.0f;
    sbias[threadIdx.x] = e.my_bias;             // 0 without a bias
    __syncthreads();
  }
  epilogue<MODE, XBF16, WT>(acc, M, N, m0, n0, wm, wn, lane, e.rsx, scol, sbias, e.nO, XO, WO, src, side, side_buf,
                            Y, lds + kEpiCols + (threadIdx.x >> 6) * kStgWaveJ);
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
                                                      const uint16_t* __restrict__ WO,
                                                      const float* __restrict__ bias, void* __restrict__ Y,
                                                      int tiles_m, int tiles_n, SideSrc src) {
  // two stages of A and B, and the epilogue's LDS after the K loop
  constexpr int kLdsBytes = 4 * kBM * kBK > kEpiLds8 ? 4 * kBM * kBK : kEpiLds8;
  // the K loop's two stages (later the epilogue's staging), then the area of
  // the outlier columns gathered in the epilogue when there are more than
  // kOutCap of them
  __shared__ __attribute__((aligned(16))) int8_t lds_raw[kLdsBytes + kSideLds];
  int8_t (*lds)[2][kBM * kBK] = reinterpret_cast<int8_t (*)[2][kBM * kBK]>(lds_raw);

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  EpiIn ein;
  epi_prefetch<MODE>(ein, M, N, m0, n0, wm, lane, sx, sw, bias, nO_ptr);

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
  finish_tile<MODE, XBF16>(acc, ein, reinterpret_cast<char*>(&lds[0][0][0]), M, N, m0, n0, wm, wn, lane, XO, WO,
                           src, nullptr, reinterpret_cast<char*>(lds_raw) + kLdsBytes, Y);
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
// fragments, LDS reads of the next fragments, [a DMA of a future K-step]}.
// sched_barrier keeps the order: the loads are spread over the MFMA shadow
// instead of stalling the wave's in-order issue in a burst. The next
// fragments are read in the order the next sub-step consumes them (A0, then
// B0..B3, then A1..A3), two per group in the first four groups, so they have
// landed when the next sub-step starts: the compiler puts a wait for every
// outstanding LDS read there, as it counts the LDS DMAs in flight among them.
// LOAD 1 issues a future step's 4 A loads, LOAD 2 its 4 B loads, one every
// other group: a step's loads are spread over two sub-steps.
template <int LOAD>
__device__ __forceinline__ void mma_phase(const v4i (&fm)[8], v16i (&acc)[4][4], const int8_t* sfr, int sub,
                                          int wm, int wn, int lane, v4i (&fl)[8], const DmaSrc& src, int k0,
                                          int8_t* st, int wave) {
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int kOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};   // fragment index: 0..3 rows of A, 4..7 rows of B
  auto read = [&](int f) {
    if (f < 4)
      fl[f] = *reinterpret_cast<const v4i*>(sfr + swz64(wm * 128 + f * 32 + fr, 2 * sub + fh));
    else
      fl[f] = *reinterpret_cast<const v4i*>(sfr + kBM * kBK + swz64(wn * 128 + (f - 4) * 32 + fr, 2 * sub + fh));
  };
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p0 = 2 * t, p1 = 2 * t + 1;
    acc[p0 >> 2][p0 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p0 & 3)], fm[p0 >> 2], acc[p0 >> 2][p0 & 3], 0, 0, 0);
    acc[p1 >> 2][p1 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p1 & 3)], fm[p1 >> 2], acc[p1 >> 2][p1 & 3], 0, 0, 0);
    if (t < 4) {
      read(kOrder[2 * t]);
      read(kOrder[2 * t + 1]);
    }
    if (LOAD == 1 && (t & 1) == 0) dma_a(src, st + (wave * 4 + t / 2) * 1024, t / 2, k0);
    if (LOAD == 2 && (t & 1) == 0) dma_b(src, st + kBM * kBK + (wave * 4 + t / 2) * 1024, t / 2, k0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// 128x128 blocks for the leftover tiles of a last, partial wave. A 256x256
// tile takes the same time on its CU however few tiles share the wave, so a
// wave of R < cus tiles costs as much as a full one; each leftover tile is
// instead covered by four 128x128 blocks (2x2 waves of 64x64 outputs, 2x2
// MFMA tiles each), optionally cut into `split` K-slices. The smaller block
// streams twice the operand bytes per MFMA, but it runs alone on its CU while
// the chip is otherwise idle. Ring: 2*S stages of 16 KB in the same LDS.
constexpr int kSmall = 128;
constexpr int kSmallStage = 2 * kSmall * kBK;   // one K step of A then B, 16 KB
constexpr int kSmallLoads = 4;                  // DMA instructions per wave per step
constexpr int kSmallPartBytes = kSmall * kSmall * 4;

// The MFMA builtin of the small-block loop behind a plain function (with
// template-dependent arguments the host compilation pass can drop the kernel
// templates that use it).
__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i lo4(v8i v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ v4i hi4(v8i v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

// LDS row of small-block fragment f (0, 1: A row blocks; 2, 3: B row blocks).
__device__ __forceinline__ const int8_t* small_frag(const int8_t* slot, int f, int wm, int wn, int fr, int ch) {
  return f < 2 ? slot + swz64(wm * 64 + f * 32 + fr, ch) : slot + kSmall * kBK + swz64(wn * 64 + (f - 2) * 32 + fr, ch);
}

template <int SS>
__device__ __forceinline__ void small_issue(int8_t* lds, int kt, int nk, const DmaSrc& src, int wave) {
  int8_t* st = lds + (kt % SS) * kSmallStage;
  const int k0 = min(kt, nk - 1) * kBK;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    dma_a(src, st + (wave * 2 + i) * 1024, i, k0);
    dma_b(src, st + kSmall * kBK + (wave * 2 + i) * 1024, i, k0);
  }
}

// K step kt of the small-block loop: wait for step kt+1 (all waves) and for
// every wave to be done with step kt's slot; then 8 MFMAs (both 32-byte halves
// of the 2x2 tiles, half-major so back-to-back MFMAs are independent) on fc,
// one 16-byte read of step kt+1's fragments per MFMA (order A0, B0, B1, A1)
// and one DMA of step kt+SS into the retired slot per two MFMAs. The last step
// runs the same code: its reads stay in the ring and its DMA repeats the last
// step into its own, retired slot.
template <int SS>
__device__ __forceinline__ void small_body(const v8i* fc, v8i* fn, v16i (*acc)[2], int8_t* lds, int kt, int nk,
                                           int wm, int wn, int lane, const DmaSrc& src, int wave) {
  wait_lgkmcnt<0>();
  wait_vmcnt<(SS - 2) * kSmallLoads>();
  block_barrier();
  const int fr = lane & 31, fh = lane >> 5;
  const int8_t* sn = lds + ((kt + 1) % SS) * kSmallStage;
  int8_t* st = lds + (kt % SS) * kSmallStage;
  const int k0 = min(kt + SS, nk - 1) * kBK;
  constexpr int kOrd[4] = {0, 2, 3, 1};
  v4i lo;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int half = t >> 2, i = (t >> 1) & 1, j = t & 1;
    const v4i a = half ? hi4(fc[i]) : lo4(fc[i]);
    const v4i b = half ? hi4(fc[2 + j]) : lo4(fc[2 + j]);
    acc[i][j] = mfma_i8(b, a, acc[i][j]);
    const int f = kOrd[t >> 1];
    if ((t & 1) == 0) {
      lo = *reinterpret_cast<const v4i*>(small_frag(sn, f, wm, wn, fr, fh));
      const int d = t >> 1;
      if (d < 2) dma_a(src, st + (wave * 2 + d) * 1024, d, k0);
      else dma_b(src, st + kSmall * kBK + (wave * 2 + d - 2) * 1024, d - 2, k0);
    } else {
      const v4i hi = *reinterpret_cast<const v4i*>(small_frag(sn, f, wm, wn, fr, 2 + fh));
      fn[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 128-byte K steps (K % 128 == 0; the 256x256 tiles and the quarter blocks
// below). LDS rows are 128 bytes; chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7), so 16 consecutive rows read at one chunk hit 16
// distinct 16-byte bank groups.
constexpr int kBK2 = 128;
constexpr int kStage2 = 2 * kBM * kBK2;         // 64 KB: A rows, then B rows

__device__ __forceinline__ int swz128(int row, int ch) { return row * kBK2 + ((ch ^ ((row >> 1) & 7)) << 4); }

// Sources of a block's 128-byte-step loads: its rows of A and of B, and the
// lane's row and chunk offset for even / odd loads i (the XOR term of the
// chunk differs by 4 between them).
struct Dma128 {
  __amdgpu_buffer_rsrc_t a, b;   // the block's rows of A and of B (zeros past M / N)
  uint32_t voff[2];              // this lane's row and chunk offset for even / odd i
  int rows8;                     // bytes between a wave's consecutive loads: 8 K
};

// The quarter blocks of the 128-byte-step kernel (K % 128 == 0, at most
// K / 128 slices): whole 128-byte row segments, as in the 256x256 tiles, which
// the load path moves faster than the 64-byte half lines of the 64-byte steps
// (a quarter block streams twice a whole tile's bytes per MFMA). Ring of 4
// stages of 32 KB (A rows, then B rows; chunk c of row r at chunk
// c ^ ((r >> 1) & 7)) in the same LDS; a step is two 64-byte phases of 8 MFMAs
// per wave, one barrier per step, and its 8 loads per wave are split between
// the phase after the barrier (A rows) and the next step's first phase (B
// rows), like the whole tiles'.
constexpr int kSmallStage2 = 2 * kSmall * kBK2;  // 32 KB
constexpr int kSmallS2 = 4;

// Load i (0..3) of a wave covers block rows wave*32 + 8i + lane/8, 8 lanes of
// 16 bytes per row; the XOR term of its chunk alternates with the parity of i.
__device__ __forceinline__ Dma128 small128_src(const int8_t* A, const int8_t* B, int m0, int n0, int M, int N, int K,
                                               int k_off, int wave, int lane) {
  Dma128 d;
  d.a = operand_rsrc(A, m0, M, K, k_off, kSmall);
  d.b = operand_rsrc(B, n0, N, K, k_off, kSmall);
  const int r = wave * 32 + (lane >> 3);
  const int ch = (lane & 7) ^ ((r >> 1) & 7);
  d.voff[0] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + (ch << 4);
  d.voff[1] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + ((ch ^ 4) << 4);
  d.rows8 = 8 * K;
  return d;
}

// Load q (0..7) of a step into stage st: q < 4 are A's loads 0..3, the others B's.
__device__ __forceinline__ void small128_dma(const Dma128& d, int8_t* st, int q, int k0, int wave) {
  const int i = q & 3;
  if (q < 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, st + (wave * 4 + i) * 1024, 16, d.voff[i & 1] + i * d.rows8, k0, 0,
                                             0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, st + kSmall * kBK2 + (wave * 4 + i) * 1024, 16,
                                             d.voff[i & 1] + i * d.rows8, k0, 0, 0);
}

// 16-byte chunk ch of the lane's row of fragment f (0, 1: A row blocks; 2, 3: B).
__device__ __forceinline__ const int8_t* small128_frag(const int8_t* slot, int f, int wm, int wn, int fr, int ch) {
  return f < 2 ? slot + swz128(wm * 64 + f * 32 + fr, ch)
               : slot + kSmall * kBK2 + swz128(wn * 64 + (f - 2) * 32 + fr, ch);
}

// One 64-byte phase: 8 MFMAs on fc (both 32-byte sub-steps of the 2x2 tiles,
// sub-step-major so back-to-back MFMAs are independent) while the fragments
// of half `half` of stage sn are read into fn (two 16-byte reads per MFMA in
// the first four, in the order the next phase consumes them: A0, B0, B1, A1)
// and, one per MFMA pair, the 4 loads of a future step's A rows (LOAD 1) or
// B rows (LOAD 2) go to stage st.
template <int LOAD>
__device__ __forceinline__ void small128_phase(const v8i* fc, v8i* fn, v16i (*acc)[2], const int8_t* sn, int half,
                                               int wm, int wn, int lane, const Dma128& d, int k0, int8_t* st,
                                               int wave) {
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int kOrd[4] = {0, 2, 3, 1};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int h = t >> 2, i = (t >> 1) & 1, j = t & 1;
    const v4i a = h ? hi4(fc[i]) : lo4(fc[i]);
    const v4i b = h ? hi4(fc[2 + j]) : lo4(fc[2 + j]);
    acc[i][j] = mfma_i8(b, a, acc[i][j]);
    if (t < 4) {
      const int f = kOrd[t];
      const v4i lo = *reinterpret_cast<const v4i*>(small128_frag(sn, f, wm, wn, fr, 4 * half + fh));
      const v4i hi = *reinterpret_cast<const v4i*>(small128_frag(sn, f, wm, wn, fr, 4 * half + 2 + fh));
      fn[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if (LOAD != 0 && (t & 1) == 0) small128_dma(d, st, 4 * (LOAD - 1) + t / 2, k0, wave);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 128x128 block of the leftover tiles: block tb of the nu tail blocks,
// which are `split` K-slices of 4*R quarter tiles (R leftover 256x256 tiles,
// numbered slice-major per XCD like the big split). A quarter outside [M, N)
// returns at once (its other slices do too). With split > 1 the slices
// exchange int32 partials and counters as the big split-K does (exact sums,
// any order).
template <int MODE, bool XBF16, int S, bool K128>
__device__ __forceinline__ void small_block(int8_t* lds, const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                            int M, int N, int K, const float* __restrict__ sx,
                                            const float* __restrict__ sw, const int* __restrict__ nO_ptr,
                                            const uint16_t* __restrict__ XO, const uint16_t* __restrict__ WO,
                                            const float* __restrict__ bias, void* __restrict__ Y, int tiles_m,
                                            int tiles_n, int dp_tiles, int tb, int nu, int split,
                                            int* __restrict__ part, int* __restrict__ cnt, const SideSrc& src) {
  constexpr int SS = 2 * S;                     // the same LDS as S big stages
  int* const s_last = reinterpret_cast<int*>(lds + kEpiLds8);
  const int v = xcd_remap(tb, nu);
  const int Q = nu / split;                     // quarter tiles
  const int piece = v / Q, sub = v % Q;
  int tm, tn;
  group_tile(dp_tiles + sub / 4, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM + (sub & 2) * 64, n0 = tn * kBN + (sub & 1) * 128;
  if (m0 >= M || n0 >= N) return;
  const int kstep = K128 ? kBK2 : kBK;          // K bytes per step
  const int nk_all = K / kstep;
  const int kb = piece * nk_all / split, ke = (piece + 1) * nk_all / split, nk = ke - kb;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  EpiIn ein;
  epi_prefetch<MODE, 2>(ein, M, N, m0, n0, wm, lane, sx, sw, bias, nO_ptr);

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  if constexpr (K128) {
    constexpr int SS2 = kSmallS2;
    static_assert(SS2 * kSmallStage2 <= S * 2 * kBM * kBK, "the 128-byte ring fits the big one");
    const Dma128 d = small128_src(A, B, m0, n0, M, N, K, kb * kBK2, wave, lane);
    for (int st = 0; st < SS2; ++st)
#pragma unroll
      for (int q = 0; q < 8; ++q) small128_dma(d, lds + st * kSmallStage2, q, min(st, nk - 1) * kBK2, wave);
    wait_vmcnt<(SS2 - 1) * 8>();                // step 0 landed (this wave)
    block_barrier();                            // ... for every wave
    v8i fa[4], fb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v4i lo = *reinterpret_cast<const v4i*>(small128_frag(lds, f, wm, wn, fr, fh));
      const v4i hi = *reinterpret_cast<const v4i*>(small128_frag(lds, f, wm, wn, fr, 2 + fh));
      fa[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // Step kt: its first half multiplies while its second half's fragments
    // are read and the B rows of step kt-1+S2 go into the slot retired in the
    // previous step (the first S2 steps came whole with the fill); then (step
    // kt+1 landed everywhere, slot kt read by every wave) the second half
    // multiplies while step kt+1's first fragments are read and the A rows of
    // step kt+S2 are fetched into slot kt. The last step runs the same code:
    // its stray reads stay in the ring, its loads repeat the last step into
    // retired slots.
    for (int kt = 0; kt < nk; ++kt) {
      int8_t* sc = lds + (kt % SS2) * kSmallStage2;
      if (kt > 0)
        small128_phase<2>(fa, fb, acc, sc, 1, wm, wn, lane, d, min(kt - 1 + SS2, nk - 1) * kBK2,
                          lds + ((kt - 1) % SS2) * kSmallStage2, wave);
      else
        small128_phase<0>(fa, fb, acc, sc, 1, wm, wn, lane, d, 0, nullptr, wave);
      wait_lgkmcnt<0>();
      wait_vmcnt<(SS2 - 2) * 8>();
      block_barrier();
      small128_phase<1>(fb, fa, acc, lds + ((kt + 1) % SS2) * kSmallStage2, 0, wm, wn, lane, d,
                        min(kt + SS2, nk - 1) * kBK2, sc, wave);
    }
  } else {
  // load i (0, 1) of each operand: block row r = wave*32 + 16*i + lane/4
  // lands in LDS slot (lane & 3) of that row
  const DmaSrc src_k = dma_src(A, B, m0, n0, M, N, K, kb * kBK, kSmall, wave, lane);
  for (int st = 0; st < SS; ++st) small_issue<SS>(lds, st, nk, src_k, wave);
  wait_vmcnt<(SS - 1) * kSmallLoads>();
  block_barrier();
  v8i fa[4], fb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const v4i lo = *reinterpret_cast<const v4i*>(small_frag(lds, f, wm, wn, fr, fh));
    const v4i hi = *reinterpret_cast<const v4i*>(small_frag(lds, f, wm, wn, fr, 2 + fh));
    fa[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    small_body<SS>(fa, fb, acc, lds, kt, nk, wm, wn, lane, src_k, wave);
    small_body<SS>(fb, fa, acc, lds, kt + 1, nk, wm, wn, lane, src_k, wave);
  }
  if (kt < nk) small_body<SS>(fa, fb, acc, lds, kt, nk, wm, wn, lane, src_k, wave);
  }
  wait_lgkmcnt<0>();
  wait_vmcnt<0>();                              // retire the trailing repeat loads
  block_barrier();                              // every wave is done with the ring

  if (split > 1) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lane_off = (wv * 16 * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t mine = partial_rsrc(part, v, kSmallPartBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4i val{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, val), mine,
                                                 lane_off + ((i * 2 + j) * 4 + q) * 1024, 0, kSc1);
        }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      *s_last = __hip_atomic_fetch_add(cnt + sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == split - 1;
    __syncthreads();
    if (!*s_last) return;
    if (tid == 0) cnt[sub] = 0;
    for (int p = 0; p < split; ++p) {
      if (p == piece) continue;
      const __amdgpu_buffer_rsrc_t other = partial_rsrc(part, p * Q + sub, kSmallPartBytes);
      v4i w[16];
#pragma unroll
      for (int t = 0; t < 16; ++t)
        w[t] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(other, lane_off + t * 1024, 0, kSc1));
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t >> 3][(t >> 2) & 1][4 * (t & 3) + e] += w[t][e];
    }
  }
  finish_tile<MODE, XBF16, 2>(acc, ein, reinterpret_cast<char*>(lds), M, N, m0, n0, wm, wn, lane, XO, WO, src, nullptr,
                              reinterpret_cast<char*>(lds) + S * 2 * kBM * kBK, Y);
}

// ---------------------------------------------------------------------------
// Whole 256x256 tiles on 128-byte K steps (K % 128 == 0). Each row segment a
// step moves is a whole 128-byte line, which the L2 -> LDS path streams about
// 25% faster than the 64-byte half lines of the 64-byte step (measured with
// w8dbg_lds_stream), and a step is 64 MFMAs per wave between barriers. The
// ring holds two 64 KB steps; the loads of step kt + 2 go out after the
// barrier that retires step kt's slot: its A rows in the phase that
// multiplies step kt's last 32-byte sub-step, its B rows in the first phase of
// step kt + 1, one load per MFMA pair. The B rows then have two sub-steps to
// land. All 16 loads of a wave in one phase (64 per CU, 1 KB each, about
// twice what the CU's load path moves in that phase) held up the MFMA issue
// behind the queued loads: 2790 against 2405 shader cycles per step on the
// DiT QKV shape.

// Fragments of 32-byte sub-step `sub` (0..3) of the step in slot `sa`.
__device__ __forceinline__ void load_frags128(const int8_t* sa, int sub, int wm, int wn, int lane, v4i (&f)[8]) {
  const int fr = lane & 31, fh = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = *reinterpret_cast<const v4i*>(sa + swz128(wm * 128 + i * 32 + fr, 2 * sub + fh));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f[4 + j] = *reinterpret_cast<const v4i*>(sa + kBM * kBK2 + swz128(wn * 128 + j * 32 + fr, 2 * sub + fh));
}

// The 128-byte step's loads: load i (0..7) of a wave covers tile rows
// wave*64 + 8i + lane/8, 8 lanes (16 bytes each) per row; lane l's 16 bytes
// land in physical chunk l & 7 of its row, which holds logical chunk
// (l & 7) ^ ((row >> 1) & 7). For odd i that XOR term is 4 more than for
// even i, so two per-lane offsets serve all 8 loads.
__device__ __forceinline__ Dma128 dma128_src(const int8_t* A, const int8_t* B, int m0, int n0, int M, int N, int K,
                                             int wave, int lane) {
  Dma128 d;
  d.a = operand_rsrc(A, m0, M, K, 0, kBM);
  d.b = operand_rsrc(B, n0, N, K, 0, kBN);
  const int r = wave * 64 + (lane >> 3);
  const int ch = (lane & 7) ^ ((r >> 1) & 7);
  d.voff[0] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + (ch << 4);
  d.voff[1] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + ((ch ^ 4) << 4);
  d.rows8 = 8 * K;
  return d;
}

// Load q (0..15) of a step: q < 8 are A's loads 0..7, q >= 8 B's.
__device__ __forceinline__ void dma128(const Dma128& d, int8_t* st, int q, int k0, int wave) {
  const int i = q & 7;
  if (q < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, st + (wave * 8 + i) * 1024, 16, d.voff[i & 1] + i * d.rows8, k0, 0,
                                             0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, st + kBM * kBK2 + (wave * 8 + i) * 1024, 16,
                                             d.voff[i & 1] + i * d.rows8, k0, 0, 0);
}

// One 32-byte sub-step: 16 MFMAs on fm, interleaved with the 8 fragment reads
// of the next sub-step (READ, two per MFMA pair in the first half, so they
// have landed when the next sub-step starts: the compiler waits for every LDS
// read there, because it counts the LDS DMAs in flight as LDS operations too)
// and, one per MFMA pair, the 8 loads of a future step's A rows (LOAD 1) or
// B rows (LOAD 2); order pinned with sched_barrier.
template <bool READ, int LOAD>
__device__ __forceinline__ void phase128(const v4i (&fm)[8], v16i (&acc)[4][4], const int8_t* sn, int sub, int wm,
                                         int wn, int lane, v4i (&fl)[8], const Dma128& d, int k0, int8_t* st,
                                         int wave) {
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int kOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};   // next fragments in the order they are consumed
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int p0 = 2 * t, p1 = 2 * t + 1;
    acc[p0 >> 2][p0 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p0 & 3)], fm[p0 >> 2], acc[p0 >> 2][p0 & 3], 0, 0, 0);
    if (LOAD != 0) dma128(d, st, 8 * (LOAD - 1) + t, k0, wave);
    acc[p1 >> 2][p1 & 3] =
        __builtin_amdgcn_mfma_i32_32x32x32_i8(fm[4 + (p1 & 3)], fm[p1 >> 2], acc[p1 >> 2][p1 & 3], 0, 0, 0);
    if (READ && t < 4) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int f = kOrder[2 * t + u];
        if (f < 4)
          fl[f] = *reinterpret_cast<const v4i*>(sn + swz128(wm * 128 + f * 32 + fr, 2 * sub + fh));
        else
          fl[f] = *reinterpret_cast<const v4i*>(sn + kBM * kBK2 + swz128(wn * 128 + (f - 4) * 32 + fr, 2 * sub + fh));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// A whole-tile block of the 128-byte-step kernel: ring fill, K loop, epilogue.
template <int MODE, bool XBF16>
__device__ __forceinline__ void tile128(int8_t* lds, const int8_t* __restrict__ A, const int8_t* __restrict__ B, int M,
                                        int N, int K, const float* __restrict__ sx, const float* __restrict__ sw,
                                        const int* __restrict__ nO_ptr, const uint16_t* __restrict__ XO,
                                        const uint16_t* __restrict__ WO, const float* __restrict__ bias,
                                        void* __restrict__ Y, int tiles_m, int tiles_n, int dp_tiles, int lb,
                                        const SideSrc& src, long long* __restrict__ tl) {
  auto stamp = [&](int p, long long v) {
    if (tl != nullptr && threadIdx.x == 0) tl[static_cast<int64_t>(lb) * 8 + p] = v;
  };
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(lb, dp_tiles, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  EpiIn ein;
  epi_prefetch<MODE>(ein, M, N, m0, n0, wm, lane, sx, sw, bias, nO_ptr);
  const Dma128 d = dma128_src(A, B, m0, n0, M, N, K, wave, lane);
  const int nk = K / kBK2;
  stamp(0, wall_clock64());

  v16i acc[4][4];
  zero_acc(acc);
  // steps 0 and 1 (step 0 again when there is only one)
#pragma unroll
  for (int q = 0; q < 16; ++q) dma128(d, lds, q, 0, wave);
#pragma unroll
  for (int q = 0; q < 16; ++q) dma128(d, lds + kStage2, q, min(1, nk - 1) * kBK2, wave);
  const bool side = MODE != 0 && XO != nullptr && WO != nullptr;
  if (side) {
    int8_t* sl = lds + 2 * kStage2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = (wave * 4 + t) * 16 + (lane >> 2);
      const int ch = (lane & 3) ^ ((r >> 2) & 3);
      __builtin_amdgcn_global_load_lds(XO + static_cast<int64_t>(min(m0 + r, M - 1)) * 32 + ch * 8,
                                       sl + (wave * 4 + t) * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(WO + static_cast<int64_t>(min(n0 + r, N - 1)) * 32 + ch * 8,
                                       sl + kSideRows * 64 + (wave * 4 + t) * 1024, 16, 0, 0);
    }
  }
  // step 0 landed (this wave); step 1's loads and the side loads are behind it
  if (side) wait_vmcnt<16 + 8>();
  else wait_vmcnt<16>();
  block_barrier();                                // ... for every wave
  stamp(1, wall_clock64());
  stamp(4, clock64());
  v4i f0[8], f1[8];
  load_frags128(lds, 0, wm, wn, lane, f0);
  for (int kt = 0; kt < nk - 1; ++kt) {
    int8_t* sa = lds + (kt & 1) * kStage2;
    // step kt+1's B rows go out with the first sub-step (its A rows went out
    // in the previous step's last phase; step 1 came whole with the fill)
    if (kt > 0)
      phase128<true, 2>(f0, acc, sa, 1, wm, wn, lane, f1, d, (kt + 1) * kBK2, lds + ((kt + 1) & 1) * kStage2, wave);
    else
      phase128<true, 0>(f0, acc, sa, 1, wm, wn, lane, f1, d, 0, nullptr, wave);
    phase128<true, 0>(f1, acc, sa, 2, wm, wn, lane, f0, d, 0, nullptr, wave);
    phase128<true, 0>(f0, acc, sa, 3, wm, wn, lane, f1, d, 0, nullptr, wave);
    wait_lgkmcnt<0>();                            // this slot is fully read
    wait_vmcnt<0>();                              // step kt+1 landed (this wave)
    block_barrier();                              // ... for every wave; slot kt retired
    // the last sub-step multiplies while step kt+1's first fragments are read
    // and the A rows of step kt+2 (or of a repeat of the last step) are
    // fetched into the retired slot
    phase128<true, 1>(f1, acc, lds + ((kt + 1) & 1) * kStage2, 0, wm, wn, lane, f0, d,
                      min(kt + 2, nk - 1) * kBK2, sa, wave);
  }
  {
    const int8_t* sa = lds + ((nk - 1) & 1) * kStage2;
    load_frags128(sa, 1, wm, wn, lane, f1);
    mfma_sub(f0, acc);
    load_frags128(sa, 2, wm, wn, lane, f0);
    mfma_sub(f1, acc);
    load_frags128(sa, 3, wm, wn, lane, f1);
    mfma_sub(f0, acc);
    mfma_sub(f1, acc);
  }
  wait_vmcnt<0>();                                // retire the trailing repeat loads
  block_barrier();                                // every wave is done with the ring
  stamp(2, wall_clock64());
  stamp(5, clock64());
  finish_tile<MODE, XBF16>(acc, ein, reinterpret_cast<char*>(lds), M, N, m0, n0, wm, wn, lane, XO, WO, src,
                           side ? reinterpret_cast<const char*>(lds) + 2 * kStage2 : nullptr,
                           reinterpret_cast<char*>(lds) + 2 * kStage2, Y);
  stamp(3, wall_clock64());
}

// Work split for the last, partial wave of tiles (split-K). The first
// dp_tiles blocks each own a whole 256x256 tile. The remaining blocks are
// `split` K-slices of each of the R = (gridDim.x - dp_tiles) / split leftover
// tiles: every slice writes its int32 partial sums to its own slot of `part`,
// bumps the tile's arrival counter in `cnt` (zero on entry, left zero on
// exit), and the last slice to arrive adds the other slices' partials to its
// own and runs the epilogue. Integer sums are exact in any order, so the result does not
// depend on which slice arrives last. No block ever waits for another.

template <int MODE, bool XBF16, int S, bool K128>
__global__ __launch_bounds__(256, 1) void k_int8_gemm_dma(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                          int M, int N, int K, const float* __restrict__ sx,
                                                          const float* __restrict__ sw, const int* __restrict__ nO_ptr,
                                                          const uint16_t* __restrict__ XO,
                                                          const uint16_t* __restrict__ WO,
                                                          const float* __restrict__ bias, void* __restrict__ Y,
                                                          int tiles_m, int tiles_n, int dp_tiles, int split,
                                                          int small, int tfirst, int* __restrict__ part,
                                                          int* __restrict__ cnt, SideSrc src,
                                                          long long* __restrict__ tl) {
  constexpr int kStage = 2 * kBM * kBK;       // A then B, 32 KB
  constexpr int kLoads = 8;                   // DMA instructions per wave per step
  // the ring, then the tile's outlier operands (kSideLds)
  __shared__ __attribute__((aligned(1024))) int8_t lds[S * kStage + kSideLds];
  static_assert(S * kStage >= kEpiLds8, "epilogue LDS");
  // A second __shared__ object would make the compiler guard every LDS read in
  // the K loop with a full vmcnt wait (it cannot tell the DMA destinations
  // apart from it); the split-K arrival flag lives in the ring instead, which
  // the K loop no longer uses by then (past the epilogue's LDS, so the
  // epilogue cannot overwrite it while a wave still reads it).
  int* const s_last = reinterpret_cast<int*>(lds + kEpiLds8);
  static_assert(S * kStage >= kEpiLds8 + 4, "epilogue LDS and arrival flag");

  // Logical block index: whole tiles 0 .. dp_tiles-1, then the blocks past
  // them. With tfirst > 0 (128x128 quarters only) the grid launches those
  // tfirst blocks first, so the partial last wave starts with the first one
  // instead of after the last (tfirst % 8 == 0 keeps every block's XCD).
  const int bid = static_cast<int>(blockIdx.x);
  const int lb = tfirst > 0 ? (bid < tfirst ? dp_tiles + bid : bid - tfirst) : bid;
  // Optional per-block timeline (debug export only; tl is null otherwise):
  // wave 0's first lane writes 8 words per logical block: [0] start, [1] K
  // loop start, [2] K loop end, [3] end (100 MHz constant clock,
  // wall_clock64), [4], [5] the shader-clock counter (clock64) at [1] and [2].
  // A block with several tile pieces leaves [1]..[5] of its last piece that
  // writes them; a piece that hands its partial to another block writes no end.
  auto stamp = [&](int p, long long v) {
    if (tl != nullptr && threadIdx.x == 0) {
      tl[static_cast<int64_t>(lb) * 8 + p] = v;
    }
  };
  if (small == 1 && lb >= dp_tiles) {
    stamp(0, wall_clock64());
    small_block<MODE, XBF16, S, K128>(lds, A, B, M, N, K, sx, sw, nO_ptr, XO, WO, bias, Y, tiles_m, tiles_n, dp_tiles,
                                lb - dp_tiles, static_cast<int>(gridDim.x) - dp_tiles, split, part, cnt, src);
    stamp(3, wall_clock64());
    return;
  }
  if constexpr (K128) {
    // every other block owns a whole tile (the launcher's condition)
    static_assert(S * kStage == 2 * kStage2, "the 128-byte steps use the same ring");
    tile128<MODE, XBF16>(lds, A, B, M, N, K, sx, sw, nO_ptr, XO, WO, bias, Y, tiles_m, tiles_n, dp_tiles, lb, src,
                         tl);
    return;
  }
  const int nk_all = K / kBK;
  const int tid = threadIdx.x, lane0 = tid & 63, wave0 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool side = MODE != 0 && XO != nullptr && WO != nullptr;

  // The block's work as a range [g0, g1) of K steps over a sequence of tiles
  // (tile-major, nk_all steps per tile), cut at tile boundaries into pieces.
  //  * whole-tile blocks (blockIdx < dp_tiles): one tile, all its K steps;
  //  * split-K slices (small == 0): K-slice `piece` of leftover tile sk_tile;
  //  * stream-K blocks (small == 2): the leftover tiles' K steps dealt out
  //    evenly, block v taking [v*per, (v+1)*per) of W = tiles * nk_all steps
  //    (per = ceil(W / nb); the last blocks may get fewer or none).
  // A piece with every K step of its tile runs the epilogue; otherwise it
  // writes its int32 partial to its slot, bumps the tile's arrival counter,
  // and the last piece to arrive adds the others' partials to its own and
  // runs the epilogue. Integer sums are exact in any order.
  const int mode = lb < dp_tiles ? 0 : (small == 2 ? 2 : 1);
  const int nb = gridDim.x - dp_tiles;          // blocks past the whole tiles
  int v = 0, R = 0, piece = 0, dp_id = 0, per = 1, t = 0;
  int g0 = 0, g1 = nk_all;                        // (W < 2^31: at most 2 cus leftover tiles)
  if (mode == 0) {
    dp_id = lb;
  } else {
    // slices and stream-K blocks are numbered per XCD (xcd_remap), so the
    // blocks of one XCD share the A rows of neighbouring tiles
    v = xcd_remap(lb - dp_tiles, nb);
    if (mode == 1) {
      R = nb / split;
      piece = v / R;
      t = v % R;
      g0 = t * nk_all + piece * nk_all / split;
      g1 = t * nk_all + (piece + 1) * nk_all / split;
    } else {
      const int W = (tiles_m * tiles_n - dp_tiles) * nk_all;
      per = (W + nb - 1) / nb;
      g0 = min(v * per, W);
      g1 = min(g0 + per, W);
      t = g0 / nk_all;
    }
  }

  bool first = true;
  for (int g = g0; g < g1; ++t) {
    // Per-piece opaque copies of the lane and wave indices: values derived
    // from them (epilogue and staging addresses) are then computed in the
    // piece instead of hoisted out of the loop and kept live across the K loop.
    int lane = lane0, wave = wave0;
    __asm__ volatile("" : "+v"(lane), "+s"(wave));
    const int wm = wave >> 1, wn = wave & 1;
    // tile t (counted from the first leftover tile unless mode 0) and its K steps [kb, ke)
    const int ts = t * nk_all;
    const int ge = min(g1, ts + nk_all);
    const int kb = g - ts, ke = ge - ts;
    const bool whole = kb == 0 && ke == nk_all;
    // this piece's partial slot, and the tile's pieces (slots of the others)
    int own_slot = -1, npieces = 1, self = 0, b_lo = 0;
    if (!whole) {
      if (mode == 1) {
        own_slot = v;
        npieces = split;
        self = piece;
      } else {
        own_slot = 2 * v + (first ? 0 : 1);
        // the stream-K blocks that cover the tile's first and last step
        b_lo = ts / per;
        npieces = (ts + nk_all - 1) / per - b_lo + 1;
        self = v - b_lo;
      }
    }
    // slot of piece p of this tile: split-K slices by slice index; a stream-K
    // block's first piece in slot 2b, its last in 2b + 1 (a tile shared by
    // several blocks is the first piece of those that start inside it)
    auto slot_of = [&](int p) -> int {
      if (mode == 1) return p * R + t;
      const int b = b_lo + p;
      return 2 * b + (b * per >= ts ? 0 : 1);
    };
    const bool first_piece = first;
    first = false;
    g = ge;

    int tm, tn;
    if (mode == 0) tile_coords(dp_id, dp_tiles, tiles_m, tiles_n, tm, tn);
    else group_tile(dp_tiles + t, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    EpiIn ein;
    epi_prefetch<MODE>(ein, M, N, m0, n0, wm, lane, sx, sw, bias, nO_ptr);

    // load instruction i (0..3) of each operand: tile row r = wave*64 + 16*i +
    // lane/4 lands in LDS slot (lane & 3) of that row, which holds logical
    // 16-byte chunk (lane & 3) ^ swz_term(r)
    const DmaSrc src_k = dma_src(A, B, m0, n0, M, N, K, kb * kBK, kBM, wave, lane);
    const int nk = ke - kb;
    block_barrier();                              // the previous piece's epilogue is done with the LDS
    if (first_piece) stamp(0, wall_clock64());    // (after the set-up: a store before it costs uniformity)
    // DMA of K-step kt into its ring slot (the fill; in the loop a step's A
    // rows go out after the barrier that retires its slot and its B rows in
    // the next sub-step). Past the last step the load repeats the last step's
    // data into the slot just retired, which no later step reads: every step
    // then issues the same number of loads, so the wait below is one constant.
    auto issue = [&](int kt) {
      int8_t* st = lds + (kt % S) * kStage;
      const int k0 = min(kt, nk - 1) * kBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma_a(src_k, st + (wave * 4 + i) * 1024, i, k0);
        dma_b(src_k, st + kBM * kBK + (wave * 4 + i) * 1024, i, k0);
      }
    };

    v16i acc[4][4];
    zero_acc(acc);

    for (int s = 0; s < S; ++s) issue(s);
    // The outlier operands of the tile for a padded outlier count of 32 (the
    // count is not known yet; the epilogue uses them only for that count), after
    // the ring's first stages so that step 0 does not wait for them. XO and WO
    // hold at least 32 values per row, so the clamped rows are in bounds.
    if (side) {
      int8_t* sl = lds + S * kStage;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = (wave * 4 + q) * 16 + (lane >> 2);
        const int ch = (lane & 3) ^ ((r >> 2) & 3);
        __builtin_amdgcn_global_load_lds(XO + static_cast<int64_t>(min(m0 + r, M - 1)) * 32 + ch * 8,
                                         sl + (wave * 4 + q) * 1024, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(WO + static_cast<int64_t>(min(n0 + r, N - 1)) * 32 + ch * 8,
                                         sl + kSideRows * 64 + (wave * 4 + q) * 1024, 16, 0, 0);
      }
    }
    // step 0 landed (this wave); the waits of the first K steps also cover
    // the 8 side loads, in flight behind the ring's
    if (side) wait_vmcnt<(S - 1) * kLoads + 8>();
    else wait_vmcnt<(S - 1) * kLoads>();
    block_barrier();                              // ... for every wave
    stamp(1, wall_clock64());
    stamp(4, clock64());
    v4i f0[8], f1[8];
    load_frags(lds, 0, wm, wn, lane, f0);
    for (int kt = 0; kt < nk - 1; ++kt) {
      int8_t* sa = lds + (kt % S) * kStage;
      // sub-step 0 multiplies while sub-step 1's fragments are read and the
      // B rows of step kt-1+S go into the slot retired in the previous step
      // (its A rows went out there; the first S steps came whole with the fill)
      if (kt > 0)
        mma_phase<2>(f0, acc, sa, 1, wm, wn, lane, f1, src_k, min(kt - 1 + S, nk - 1) * kBK,
                     lds + ((kt - 1) % S) * kStage, wave);
      else
        mma_phase<0>(f0, acc, sa, 1, wm, wn, lane, f1, src_k, 0, nullptr, wave);
      wait_lgkmcnt<0>();                          // this slot is fully read
      wait_vmcnt<(S - 2) * kLoads>();             // step kt+1 landed (this wave)
      block_barrier();                            // ... for every wave; slot kt retired
      // sub-step 1 multiplies while step kt+1's first fragments are read and
      // the A rows of step kt+S are fetched into the retired slot
      mma_phase<1>(f1, acc, lds + ((kt + 1) % S) * kStage, 0, wm, wn, lane, f0, src_k,
                   min(kt + S, nk - 1) * kBK, sa, wave);
    }
    load_frags(lds + ((nk - 1) % S) * kStage, 1, wm, wn, lane, f1);
    mfma_sub(f0, acc);
    mfma_sub(f1, acc);
    wait_vmcnt<0>();                              // retire the trailing repeat loads
    block_barrier();                              // every wave is done with the ring
    stamp(2, wall_clock64());
    stamp(5, clock64());

    if (own_slot >= 0) {
      // Partials go through sc1 buffer accesses (partial_rsrc). Once a wave's
      // stores have completed (vmcnt 0) they are visible to any later sc1
      // load; the arrival counter is bumped only after every wave's stores
      // have completed.
      const int lane_off = (wave * 64 * 64 + lane) * 16;
      const __amdgpu_buffer_rsrc_t mine = partial_rsrc(part, own_slot);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = (i * 4 + j) * 4 + q;
            const v4i x{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, x), mine, lane_off + c * 1024, 0, kSc1);
          }
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial is visible
      __syncthreads();                                        // ... and every wave's
      if (tid == 0)
        *s_last = __hip_atomic_fetch_add(cnt + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == npieces - 1;
      __syncthreads();
      // one value for the whole block: a uniform branch (a branch on the LDS
      // value itself would count as divergent and cost registers)
      if (!__builtin_amdgcn_readfirstlane(*s_last)) continue;   // another piece of the tile finishes it
      if (tid == 0) cnt[t] = 0;                   // every piece has arrived: leave the counter zero
      // one 32-row block at a time, so only its 64 accumulators leave the AGPRs
      // and 16 loads of 1 KB per wave are in flight
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        for (int p = 0; p < npieces; ++p) {
          if (p == self) continue;
          const __amdgpu_buffer_rsrc_t other = partial_rsrc(part, slot_of(p));
          v4i w[16];
#pragma unroll
          for (int q = 0; q < 16; ++q)
            w[q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(other, lane_off + (i * 16 + q) * 1024,
                                                                                 0, kSc1));
#pragma unroll
          for (int q = 0; q < 16; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][q >> 2][4 * (q & 3) + e] += w[q][e];
        }
      }
    }
    finish_tile<MODE, XBF16>(acc, ein, reinterpret_cast<char*>(lds), M, N, m0, n0, wm, wn, lane, XO, WO, src,
                             side ? reinterpret_cast<const char*>(lds) + S * kStage : nullptr,
                             reinterpret_cast<char*>(lds) + S * kStage, Y);
    stamp(3, wall_clock64());
  }
}

// ---------------------------------------------------------------------------
// Launch plan. Whole tiles fill as many complete waves of `cus` blocks as they
// can; the leftover R = T mod cus tiles of the last, partial wave run either
// whole, cut into `split` K-slices, or as four 128x128 blocks each (optionally
// sliced), whichever a cost model in units of one 256x256 K step says is
// cheapest, fitted to MI355X timings:
//  * a sparse wave of whole tiles runs at ~3/4 of a full tile's time (the few
//    busy CUs clock higher and share the memory system with no one);
//  * a 256x256 slice costs its K steps, kSliceFixed of start-up and epilogue
//    and kSliceCost per extra slice (the last slice re-reads the others' 256 KB
//    partials from another CU);
//  * a 128x128 block step costs kSmallStep of a 256x256 step, plus
//    kSmallFixed, plus kSmallSlice per extra slice (64 KB partials); with more
//    than one block per CU the CU's blocks run back to back.
constexpr int kSliceCost = 10;
constexpr int kSliceFixed = 10;
constexpr int kMinSliceSteps = 4;
constexpr int kMaxSplit = 16;
constexpr double kSmallStep = 0.30;
constexpr double kSmallFixed = 6.0;
constexpr double kSmallSlice = 3.0;

GemmPlan plan_int8_gemm(int64_t M, int64_t N, int64_t K, int cus) {
  GemmPlan p{};
  p.tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  p.tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int T = p.tiles_m * p.tiles_n;
  p.dp_tiles = T;
  p.split = 1;
  p.sk_tiles = 0;
  if (K % kBK != 0 || cus <= 0) return p;
  const int R = T % cus;
  if (R == 0) return p;
  // (Stream-K over the last full wave and the leftover tiles, which evens
  // out the blocks' K steps, measured 12-30% slower on the DiT 1024^2 linears:
  // its blocks work at different K offsets, so the blocks of an XCD no longer
  // share A and B panels in its L2. It stays available to the debug export.)
  const int nk = static_cast<int>(K / kBK);
  double best_cost = 0.75 * nk;
  int best_split = 1;
  bool best_small = false;
  const int smax = std::min(nk / kMinSliceSteps, kMaxSplit);
  for (int s = 2; s <= std::min(cus / R, smax); ++s) {
    const double cost = (nk + s - 1) / s + kSliceCost * (s - 1) + kSliceFixed;
    if (cost < best_cost) best_cost = cost, best_split = s, best_small = false;
  }
  for (int s = 1; s <= smax; ++s) {
    const int per_cu = (4 * R * s + cus - 1) / cus;
    const double cost = per_cu * (kSmallStep * ((nk + s - 1) / s) + kSmallFixed) + kSmallSlice * (s - 1);
    if (cost < best_cost) best_cost = cost, best_split = s, best_small = true;
  }
  if (best_split == 1 && !best_small) return p;
  p.dp_tiles = T - R;
  p.split = best_split;
  p.sk_tiles = R;
  p.small = best_small;
  p.tail_first = best_small && (p.grid() - p.dp_tiles) % kXcds == 0;
  return p;
}

// The same grid with a given treatment of the leftover tiles: small = false
// and split = 1 runs every tile whole; otherwise the R = T mod cus leftover
// tiles (all tiles when T < cus) run as `split` slices of 256x256 tiles or, with
// small, of 128x128 quarters. split must be in [1, K / 64] and K % 64 == 0.
GemmPlan plan_int8_gemm_forced(int64_t M, int64_t N, int cus, bool small, int split) {
  GemmPlan p{};
  p.tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  p.tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int T = p.tiles_m * p.tiles_n;
  const int R = cus > 0 ? T % cus : T;
  p.dp_tiles = T;
  p.split = 1;
  p.sk_tiles = 0;
  if ((split <= 1 && !small) || R == 0) return p;
  p.dp_tiles = T - R;
  p.split = split;
  p.sk_tiles = R;
  p.small = small;
  return p;
}

GemmPlan plan_int8_gemm_streamk(int64_t M, int64_t N, int cus) {
  GemmPlan p{};
  p.tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  p.tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int T = p.tiles_m * p.tiles_n;
  p.split = 1;
  p.dp_tiles = T;
  p.sk_tiles = 0;
  if (cus <= 0) return p;
  p.dp_tiles = T >= 2 * cus ? (T / cus - 1) * cus : 0;
  p.sk_tiles = T - p.dp_tiles;
  p.streamk = true;
  p.sk_blocks = cus;
  return p;
}

// ---------------------------------------------------------------------------
// mode: 0 int32 acc, 1 fp16 out, 2 fp32 out. `part` / `cnt` are needed when
// plan.split > 1 (plan.partial_bytes() of partials, plan.counters() counters
// that must be zero; they are left zero). XO [M, P] and WO [N, P] (P = the
// outlier count nO padded to 32) may be null when mode is 0; otherwise their
// buffers hold kOutCap values per row. `src`: where the epilogue gathers the
// outlier columns when P > kOutCap (unused in mode 0).
void launch_int8_gemm(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                      const float* sw, const int* nO, const uint16_t* XO, const uint16_t* WO, bool xbf16,
                      const float* bias, void* Y, int mode, const GemmPlan& plan, int* part, int* cnt,
                      const SideSrc& src, hipStream_t s, long long* timeline) {
  const int tiles_m = plan.tiles_m, tiles_n = plan.tiles_n;
  const int m = (int)M, n = (int)N, k = (int)K;
  const dim3 block(256);
  if (K % kBK == 0) {
    constexpr int S = 4;
    const dim3 grid(plan.grid());
    // 128-byte K steps when K allows and every block past the small tail owns a
    // whole tile (the tail's quarter blocks then step 128 bytes too, so at
    // most K / 128 slices of them)
    const bool k128 = K % kBK2 == 0 && !plan.streamk && (plan.small ? plan.split <= K / kBK2 : plan.split == 1);
#define W8_GEMM_ARGS A, B, m, n, k, sx, sw, nO, XO, WO, bias, Y, tiles_m, tiles_n, plan.dp_tiles, plan.split, \
    plan.streamk ? 2 : (plan.small ? 1 : 0), plan.tail_first ? plan.grid() - plan.dp_tiles : 0, part, cnt, src, \
    timeline
    if (k128) {
      if (mode == 0) k_int8_gemm_dma<0, true, S, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (mode == 1 && xbf16) k_int8_gemm_dma<1, true, S, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (mode == 1) k_int8_gemm_dma<1, false, S, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (xbf16) k_int8_gemm_dma<2, true, S, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else k_int8_gemm_dma<2, false, S, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    } else {
      if (mode == 0) k_int8_gemm_dma<0, true, S, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (mode == 1 && xbf16) k_int8_gemm_dma<1, true, S, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (mode == 1) k_int8_gemm_dma<1, false, S, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else if (xbf16) k_int8_gemm_dma<2, true, S, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
      else k_int8_gemm_dma<2, false, S, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    }
#undef W8_GEMM_ARGS
  } else {
    const dim3 grid(tiles_m * tiles_n);
#define W8_GEMM_ARGS A, B, m, n, k, sx, sw, nO, XO, WO, bias, Y, tiles_m, tiles_n, src
    if (mode == 0) k_int8_gemm<0, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1 && xbf16) k_int8_gemm<1, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (mode == 1) k_int8_gemm<1, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else if (xbf16) k_int8_gemm<2, true><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
    else k_int8_gemm<2, false><<<grid, block, 0, s>>>(W8_GEMM_ARGS);
#undef W8_GEMM_ARGS
  }
}

}  // namespace w8
