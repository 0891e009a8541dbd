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
// Main kernel (K % 64 == 0): the int8 GEMM's LDS-DMA ring and swizzle
// (tile.h) with 256x256 or 128x128 blocks, and v_mfma_scale_f32_32x32x64_f8f6f4 (both block scales 2^0,
// E8M0 code 127; format E4M3 on both sides), which issues at the full fp8 rate
// on gfx950 (the 16x16x128 form does not). One MFMA covers a whole 64-byte K
// step: lane l supplies row (l & 31) and the 32 bytes made of 16-byte chunks
// (l >> 5) and 2 + (l >> 5) of the step, the same chunks for both operands, so
// every k of the step is multiplied exactly once.
//
// Text-encoder shapes have few tokens (M = 512), so their grids use the
// smaller blocks and may be split along K to occupy the chip; the slices' fp32
// partials are summed in slice order 0, 1, ..., whichever slice adds them up,
// so results do not depend on arrival order.
#include <algorithm>

#include "launch.h"
#include "tile.h"

namespace w8 {

constexpr int kFBM = 128, kFBN = 128, kFBK = 128;

__device__ __forceinline__ int swz128(int row, int ch) { return row * kFBK + ((ch ^ ((row >> 1) & 7)) << 4); }

// General kernel (any K % 16 == 0): register-staged loads with zero fill past
// K, two LDS stages, 128x128 tiles of v_mfma_scale_f32_16x16x128_f8f6f4.
// YDT: 0 bf16, 1 fp16, 2 fp32.
template <int YDT>
__global__ __launch_bounds__(256, 2) void k_fp8_gemm_any(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
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


// ---------------------------------------------------------------------------
// Pipelined kernel (K % 64 == 0). Block = 2x2 waves; each wave owns WT x WT
// MFMA tiles of 32x32 outputs: WT = 4 gives 256x256 blocks (one per CU: 256
// accumulator registers per wave), WT = 2 gives 128x128 blocks (two per CU),
// which suit grids with few 256x256 tiles (the 512-token text encoder).
template <int WT>
struct Fp8Tile {
  static constexpr int BM = 64 * WT;                  // block rows = block columns
  static constexpr int kStage = 2 * BM * kBK;         // one K step of A then B in LDS
  static constexpr int kLoads = 2 * WT;               // DMA instructions per wave per step
  static constexpr int kFrags = 2 * WT;               // 32-byte fragments per wave per step
  static constexpr int kMfma = WT * WT;               // MFMAs per wave per step
  static constexpr int kChunks = 4 * WT * WT;         // 16-byte accumulator chunks per lane
  static constexpr int kPartBytes = BM * BM * 4;      // one fp32 partial
};

// The MFMA builtin of the K loop behind a plain (non-template) wrapper: called
// with template-dependent arguments directly, the host compilation pass drops
// the kernel templates that use it.
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// One fragment: both 16-byte halves of a 32x64-byte operand block for this
// lane (chunks fh and 2 + fh of its row).
__device__ __forceinline__ v8i frag_pair(const uint8_t* base, int row, int fh) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + swz64(row, fh));
  const v4i hi = *reinterpret_cast<const v4i*>(base + swz64(row, 2 + fh));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS row of fragment f of wave (wm, wn): f < WT are A row blocks, the rest B.
template <int WT>
__device__ __forceinline__ const uint8_t* frag_base(const uint8_t* slot, int f) {
  return f < WT ? slot : slot + Fp8Tile<WT>::BM * kBK;
}
template <int WT>
__device__ __forceinline__ int frag_row(int f, int wm, int wn, int fr) {
  return f < WT ? wm * 32 * WT + f * 32 + fr : wn * 32 * WT + (f - WT) * 32 + fr;
}

// One K step: the wave's WT*WT MFMAs on fragments fc, while the next step's
// fragments are read into fn (in the order the next step consumes them: A0,
// B0.., A1..) and the step's DMAs of a future K step go out, both spread evenly
// over the MFMAs; sched_barrier keeps that interleaving.
template <int WT>
__device__ __forceinline__ void fp8_step(const v8i* fc, v8i* fn, v16f (*acc)[WT], const uint8_t* sn, int wm, int wn,
                                         int lane, const DmaSrc& src, int k0, uint8_t* st, int wave) {
  using T = Fp8Tile<WT>;
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int kReads = 2 * T::kFrags;
  v4i lo;
#pragma unroll
  for (int t = 0; t < T::kMfma; ++t) {
    const int i = t / WT, j = t % WT;
    acc[i][j] = mfma_fp8(fc[WT + j], fc[i], acc[i][j]);
#pragma unroll
    for (int q = t * kReads / T::kMfma; q < (t + 1) * kReads / T::kMfma; ++q) {
      const int o = q >> 1;                              // o-th fragment in consumption order
      const int f = o == 0 ? 0 : (o <= WT ? WT + o - 1 : o - WT);
      const uint8_t* base = frag_base<WT>(sn, f);
      const int row = frag_row<WT>(f, wm, wn, fr);
      if ((q & 1) == 0) {
        lo = *reinterpret_cast<const v4i*>(base + swz64(row, fh));
      } else {
        const v4i hi = *reinterpret_cast<const v4i*>(base + swz64(row, 2 + fh));
        fn[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
#pragma unroll
    for (int d = t * T::kLoads / T::kMfma; d < (t + 1) * T::kLoads / T::kMfma; ++d) {
      int8_t* const s8 = reinterpret_cast<int8_t*>(st);
      if (d < WT)
        dma_a(src, s8 + (wave * WT + d) * 1024, d, k0);
      else
        dma_b(src, s8 + T::BM * kBK + (wave * WT + d - WT) * 1024, d - WT, k0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// DMA of K-step kt into its ring slot; past the last step the load repeats the
// last step into the slot just retired (read by no later step), so every step
// issues the same number of loads and one constant wait fits all.
template <int WT, int S>
__device__ __forceinline__ void fp8_issue(uint8_t* lds, int kt, int nk, const DmaSrc& src, int wave) {
  using T = Fp8Tile<WT>;
  int8_t* st = reinterpret_cast<int8_t*>(lds) + (kt % S) * T::kStage;
  const int k0 = min(kt, nk - 1) * kBK;
#pragma unroll
  for (int i = 0; i < WT; ++i) {
    dma_a(src, st + (wave * WT + i) * 1024, i, k0);
    dma_b(src, st + T::BM * kBK + (wave * WT + i) * 1024, i, k0);
  }
}

// K step kt of the loop: wait until step kt+1 has landed everywhere and every
// wave has read step kt's fragments (so its slot can be refilled with step
// kt+S), then multiply step kt while reading step kt+1's fragments. The last
// step runs the same code: its reads of the following slot (in the ring, never
// used) and its repeat DMA of the last step into its own, retired slot are
// harmless, and one loop body keeps register use at the loop's.
template <int WT, int S>
__device__ __forceinline__ void fp8_body(const v8i* fc, v8i* fn, v16f (*acc)[WT], uint8_t* lds, int kt, int nk,
                                         int wm, int wn, int lane, const DmaSrc& src, int wave) {
  using T = Fp8Tile<WT>;
  wait_lgkmcnt<0>();
  wait_vmcnt<(S - 2) * T::kLoads>();
  block_barrier();
  fp8_step<WT>(fc, fn, acc, lds + ((kt + 1) % S) * T::kStage, wm, wn, lane, src, min(kt + S, nk - 1) * kBK,
               lds + (kt % S) * T::kStage, wave);
}

// YDT: 0 bf16, 1 fp16, 2 fp32. Grid and split-K protocol as in the int8
// kernel: blocks below dp_tiles own whole tiles; the rest are `split` K-slices
// of each of R = (gridDim.x - dp_tiles) / split tiles. Each slice writes its
// fp32 partial to its own slot of `part`, bumps the tile's counter in `cnt`
// (zero on entry, left zero), and the last to arrive sums all slices' partials
// in slice order and runs the epilogue.
template <int YDT, int S, int WT>
__global__ __launch_bounds__(256, 4 / WT) void k_fp8_gemm_dma(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ B, int M, int N, int K,
                                                              const float* __restrict__ sx,
                                                              const float* __restrict__ sw, void* __restrict__ Y,
                                                              int tiles_m, int tiles_n, int dp_tiles, int split,
                                                              float* __restrict__ part, int* __restrict__ cnt,
                                                              int quarters) {
  using T = Fp8Tile<WT>;
  constexpr int BM = T::BM;
  // One LDS object only (a second one would make the compiler put a full vmcnt
  // wait before every LDS read of the K loop); the arrival flag lives in the
  // ring past the epilogue's area.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * T::kStage];
  static_assert(sizeof(lds) >= kEpiLds + 4, "epilogue LDS and arrival flag");
  int* const s_last = reinterpret_cast<int*>(lds + kEpiLds);

  const int nk_all = K / kBK;
  int tm, tn, kb = 0, ke = nk_all;
  int slot = -1, sk_tile = 0, piece = 0, R = 0;
  int m0, n0;
  if (quarters) {
    // (128x128 blocks only) the quarters of the leftover 256x256 tiles of a
    // 256x256 launch: tiles_m, tiles_n count 256x256 tiles, and the leftover
    // tiles are those from dp_tiles on in the grouped order
    const int v = xcd_remap(blockIdx.x, gridDim.x);
    group_tile(dp_tiles + v / 4, tiles_m, tiles_n, tm, tn);
    m0 = tm * 256 + ((v >> 1) & 1) * 128;
    n0 = tn * 256 + (v & 1) * 128;
    if (m0 >= M || n0 >= N) return;
  } else if (static_cast<int>(blockIdx.x) < dp_tiles) {
    tile_coords(blockIdx.x, dp_tiles, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM, n0 = tn * BM;
  } else {
    // slice-major per XCD: the blocks of one XCD share a K range
    const int nu = gridDim.x - dp_tiles;
    const int v = xcd_remap(blockIdx.x - dp_tiles, nu);
    R = nu / split;
    piece = v / R;
    sk_tile = v % R;
    slot = v;
    group_tile(dp_tiles + sk_tile, tiles_m, tiles_n, tm, tn);
    kb = piece * nk_all / split;
    ke = (piece + 1) * nk_all / split;
    m0 = tm * BM, n0 = tn * BM;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  // epilogue inputs, fetched now so their latency hides under the K loop
  float rsx[WT];
#pragma unroll
  for (int i = 0; i < WT; ++i) rsx[i] = sx[min(m0 + wm * 32 * WT + 32 * i + fr, M - 1)];
  const float my_sw = sw[min(n0 + (tid & (BM - 1)), N - 1)];

  // load instruction i of each operand: tile row r = wave*16*WT + 16*i +
  // lane/4 lands in LDS slot (lane & 3) of that row, which holds logical
  // 16-byte chunk (lane & 3) ^ swz_term(r)
  const DmaSrc src_k = dma_src(reinterpret_cast<const int8_t*>(A), reinterpret_cast<const int8_t*>(B), m0, n0, M, N,
                               K, kb * kBK, BM, wave, lane);
  const int nk = ke - kb;

  v16f acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int s = 0; s < S; ++s) fp8_issue<WT, S>(lds, s, nk, src_k, wave);
  wait_vmcnt<(S - 1) * T::kLoads>();            // step 0 landed (this wave)
  block_barrier();                              // ... for every wave
  v8i fa[2 * WT], fb[2 * WT];
#pragma unroll
  for (int f = 0; f < 2 * WT; ++f) fa[f] = frag_pair(frag_base<WT>(lds, f), frag_row<WT>(f, wm, wn, fr), fh);

  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    fp8_body<WT, S>(fa, fb, acc, lds, kt, nk, wm, wn, lane, src_k, wave);
    fp8_body<WT, S>(fb, fa, acc, lds, kt + 1, nk, wm, wn, lane, src_k, wave);
  }
  if (kt < nk) fp8_body<WT, S>(fa, fb, acc, lds, kt, nk, wm, wn, lane, src_k, wave);
  wait_lgkmcnt<0>();
  wait_vmcnt<0>();                              // retire the trailing repeat loads
  block_barrier();                              // every wave is done with the ring

  if (slot >= 0) {
    // partial layout: 16-byte chunk c of wave w's accumulators at byte
    // ((w * kChunks + c) * 64 + lane) * 16: every access is 1 KB contiguous
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lane_off = (wv * T::kChunks * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t mine = partial_rsrc(part, slot, T::kPartBytes);
#pragma unroll
    for (int i = 0; i < WT; ++i)
#pragma unroll
      for (int j = 0; j < WT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (i * WT + j) * 4 + q;
          const v4f v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), mine, lane_off + c * 1024, 0, kSc1);
        }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial is visible
    __syncthreads();                                        // ... and every wave's
    if (tid == 0)
      *s_last = __hip_atomic_fetch_add(cnt + sk_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == split - 1;
    __syncthreads();
    if (!*s_last) return;
    if (tid == 0) cnt[sk_tile] = 0;             // every slice has arrived: leave the counter zero
    // Sum all slices' partials in slice order (this slice's own included, read
    // back from its slot: summing from registers instead makes the compiler
    // spill), one 32-row block at a time, 4*WT loads of 1 KB per wave in flight.
#pragma unroll
    for (int i = 0; i < WT; ++i) {
      for (int p = 0; p < split; ++p) {
        const __amdgpu_buffer_rsrc_t src = partial_rsrc(part, p * R + sk_tile, T::kPartBytes);
        v4f w[4 * WT];
#pragma unroll
        for (int t = 0; t < 4 * WT; ++t)
          w[t] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                             src, lane_off + (i * 4 * WT + t) * 1024, 0, kSc1));
#pragma unroll
        for (int t = 0; t < 4 * WT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][t >> 2][4 * (t & 3) + e] = p == 0 ? w[t][e] : acc[i][t >> 2][4 * (t & 3) + e] + w[t][e];
      }
    }
  }

  // Epilogue: Y = acc * sx[m] * sw[n], rounded to the output type, staged
  // through LDS a 32-row block at a time (element r of tile (i, j) of a lane is
  // row m0 + wm*32*WT + 32i + (lane&31), column n0 + wn*32*WT + 32j + 8(r>>2)
  // + 4(lane>>5) + (r&3): the Wq fragment is the MFMA's first operand).
  float* scol = reinterpret_cast<float*>(lds);
  if (tid < BM) scol[tid] = my_sw;
  __syncthreads();
  constexpr int EB = YDT == 2 ? 4 : 2;          // bytes per output element
  constexpr int ROWB = 32 * WT * EB;            // bytes of one output row of the wave's tile
  constexpr int H = ROWB > 256 ? ROWB / 256 : 1;   // staging passes per 32-row block
  constexpr int PJ = WT / H;                    // 32-column tiles per pass
  constexpr int RB = 32 * PJ * EB;              // staged row bytes: 256 or 128
  const bool vec = (static_cast<int64_t>(N) * EB) % 16 == 0;
  char* const stg = reinterpret_cast<char*>(lds) + 1024 + wave * kStgWave;
  char* const y = static_cast<char*>(Y);
#pragma unroll
  for (int i = 0; i < WT; ++i) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
#pragma unroll
      for (int jj = 0; jj < PJ; ++jj) {
        const int j = h * PJ + jj;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          char* dst = stg + fr * kStgPitch + (32 * jj + 8 * g + 4 * fh) * EB;
          const v4f cs = *reinterpret_cast<const v4f*>(scol + wn * 32 * WT + 32 * j + 8 * g + 4 * fh);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * rsx[i] * cs[e];
          if constexpr (YDT == 0) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16),
                                                        bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16));
          } else if constexpr (YDT == 1) {
            const uint32_t lo = f32x2_to_f16x2_bits(v[0], v[1]);
            const uint32_t hi = f32x2_to_f16x2_bits(v[2], v[3]);
            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
          }
        }
      }
      wave_lds_fence();
      flush_staged<EB, RB>(stg, y, M, N, m0 + wm * 32 * WT + 32 * i, n0 + wn * 32 * WT + h * PJ * 32, lane, vec);
      wave_lds_fence();                         // staging reads done before the next pass writes
    }
  }
}

// ---------------------------------------------------------------------------
// Rectangular blocks on 128-byte K steps (K % 128 == 0), for grids with few
// tokens. A block is 128 rows x 64*TN columns (TN = 2: 128x128, TN = 3:
// 128x192) of 2x2 waves, each wave 2 x TN MFMA tiles of 32x32. At 512 tokens a
// 128x192 grid of the text encoder's gate and up projections is one block per
// CU (4 x 64 blocks), where 128x128 blocks left half the CUs with two blocks
// and streamed 20% more operand bytes; a GEMM step at this size is bound by
// the rate at which a CU streams operand rows into LDS, and whole 128-byte
// row segments stream faster than 64-byte halves. Ring: 4 stages of one K
// step (A rows, then B rows, 128 bytes each, chunk c of row r at chunk
// c ^ ((r >> 1) & 7)). Each step is two 64-byte sub-steps of one
// v_mfma_scale_f32_32x32x64_f8f6f4 per MFMA tile, with the operand bytes of
// the square kernel's 64-byte step (lane l: row l & 31, chunks l >> 5 and
// 2 + (l >> 5) of the sub-step), so the products and their order are the
// same. Split-K and the epilogue arithmetic are those of the square kernel.
template <int TN>
struct Fp8Rect {
  static constexpr int BM = 128, BN = 64 * TN;
  static constexpr int kStep = 128;                    // K bytes per step
  static constexpr int kStage = (BM + BN) * kStep;     // 32 or 40 KB
  static constexpr int kLoadsA = 4, kLoadsB = 2 * TN;  // DMA instructions per wave per step (rect_dma)
  static constexpr int kLoads = kLoadsA + kLoadsB;
  static constexpr int kMfma = 2 * TN;                 // MFMAs per wave per sub-step
  static constexpr int kReads = 2 * (2 + TN);          // 16-byte fragment reads per wave per sub-step
  static constexpr int kChunks = 8 * TN;               // 16-byte accumulator chunks per lane
  static constexpr int kPartBytes = BM * BN * 4;       // one fp32 partial
  static constexpr int kS = 4;                         // ring stages
};

__device__ __forceinline__ int rswz(int row, int ch) { return row * 128 + ((ch ^ ((row >> 1) & 7)) << 4); }

// The block's operand rows for the DMA: A rows m0 .. m0+127 and B rows
// n0 .. n0+64*TN-1 from byte k_off of each row (rows past M / N read as zeros,
// the buffer range check). Load i of a wave covers 8 rows, 8 lanes (16 bytes
// each) per row; lane l lands in physical chunk l & 7 of its row, which holds
// logical chunk (l & 7) ^ ((row >> 1) & 7); the wave's rows start at a
// multiple of 16, so that term depends on l and the parity of i only.
struct RectSrc {
  __amdgpu_buffer_rsrc_t a, b;
  uint32_t va[2], vb[2];                         // per-lane offsets for even / odd i
  int rows8;                                     // bytes between a wave's consecutive loads: 8 K
};

template <int TN>
__device__ __forceinline__ RectSrc rect_src(const uint8_t* A, const uint8_t* B, int m0, int n0, int M, int N, int K,
                                            int k_off, int wave, int lane) {
  RectSrc d;
  d.a = operand_rsrc(reinterpret_cast<const int8_t*>(A), m0, M, K, k_off, Fp8Rect<TN>::BM);
  d.b = operand_rsrc(reinterpret_cast<const int8_t*>(B), n0, N, K, k_off, Fp8Rect<TN>::BN);
  const uint32_t ra = static_cast<uint32_t>(wave * 32 + (lane >> 3));
  const uint32_t rb = static_cast<uint32_t>(wave * 16 * TN + (lane >> 3));
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const uint32_t ch = static_cast<uint32_t>((lane & 7) ^ ((par * 4 + (lane >> 4)) & 7)) << 4;
    d.va[par] = ra * static_cast<uint32_t>(K) + ch;
    d.vb[par] = rb * static_cast<uint32_t>(K) + ch;
  }
  d.rows8 = 8 * K;
  return d;
}

// Load q of K step k0 into stage st: q < 4 are A's loads, the others B's (lb
// per wave). Not a template: a target builtin with template-dependent
// arguments can make the host compilation pass drop the kernel templates.
__device__ __forceinline__ void rect_dma(const RectSrc& d, uint8_t* st, int q, int k0, int wave, int lb) {
  if (q < 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, st + (wave * 4 + q) * 1024, 16, d.va[q & 1] + q * d.rows8, k0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, st + 128 * 128 + (wave * lb + q - 4) * 1024, 16,
                                             d.vb[(q - 4) & 1] + (q - 4) * d.rows8, k0, 0, 0);
}

template <int TN>
__device__ __forceinline__ void rect_issue(uint8_t* lds, int kt, int nk, const RectSrc& d, int wave) {
  using T = Fp8Rect<TN>;
  uint8_t* st = lds + (kt % T::kS) * T::kStage;
  const int k0 = min(kt, nk - 1) * T::kStep;
#pragma unroll
  for (int q = 0; q < T::kLoads; ++q) rect_dma(d, st, q, k0, wave, T::kLoadsB);
}

// Row in the stage of fragment f (0, 1: A row blocks; 2..: B row blocks).
template <int TN>
__device__ __forceinline__ int rect_row(int f, int wm, int wn, int fr) {
  return f < 2 ? wm * 64 + f * 32 + fr : Fp8Rect<TN>::BM + wn * 32 * TN + (f - 2) * 32 + fr;
}

// One 64-byte sub-step: the wave's 2 x TN MFMAs on fragments fc while the
// fragments of sub-step `sub` of the stage sn are read into fn (in the order
// the MFMAs consume them: A0, B0 .., A1) and the loads of a future K step's
// A rows (LOAD 1) or B rows (LOAD 2) go to stage st; both spread evenly over
// the MFMAs, the interleaving pinned by sched_barrier. A step's loads are
// split over two sub-steps: all of them in one (40 KB per CU for TN = 3 in
// 384 MFMA cycles) is more than the CU's load path moves meanwhile, and the
// queued loads hold up the wave's in-order issue.
template <int TN, int LOAD>
__device__ __forceinline__ void rect_phase(const v8i* fc, v8i* fn, v16f (*acc)[TN], const uint8_t* sn, int sub,
                                           int wm, int wn, int lane, const RectSrc& d, int k0, uint8_t* st,
                                           int wave) {
  using T = Fp8Rect<TN>;
  const int fr = lane & 31, fh = lane >> 5;
  constexpr int kQ0 = LOAD == 2 ? T::kLoadsA : 0;                          // first load of the phase
  constexpr int kDma = LOAD == 1 ? T::kLoadsA : (LOAD == 2 ? T::kLoadsB : 0);
  v4i lo;
#pragma unroll
  for (int t = 0; t < T::kMfma; ++t) {
    const int i = t / TN, j = t % TN;
    acc[i][j] = mfma_fp8(fc[2 + j], fc[i], acc[i][j]);
#pragma unroll
    for (int q = t * T::kReads / T::kMfma; q < (t + 1) * T::kReads / T::kMfma; ++q) {
      const int o = q >> 1;                              // o-th fragment in consumption order
      const int f = o == 0 ? 0 : (o <= TN ? 2 + o - 1 : 1);
      const int row = rect_row<TN>(f, wm, wn, fr);
      if ((q & 1) == 0) {
        lo = *reinterpret_cast<const v4i*>(sn + rswz(row, 4 * sub + fh));
      } else {
        const v4i hi = *reinterpret_cast<const v4i*>(sn + rswz(row, 4 * sub + 2 + fh));
        fn[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
#pragma unroll
    for (int q = t * kDma / T::kMfma; q < (t + 1) * kDma / T::kMfma; ++q)
      rect_dma(d, st, kQ0 + q, k0, wave, T::kLoadsB);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// YDT: 0 bf16, 1 fp16, 2 fp32. Grid as in the square kernel: blocks below
// dp_tiles own whole tiles, the rest are `split` K-slices of the
// (gridDim.x - dp_tiles) / split remaining tiles, numbered slice-major per XCD.
template <int YDT, int TN>
__global__ __launch_bounds__(256, 1) void k_fp8_gemm_rect(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ B, int M, int N, int K,
                                                          const float* __restrict__ sx, const float* __restrict__ sw,
                                                          void* __restrict__ Y, int tiles_m, int tiles_n,
                                                          int dp_tiles, int split, float* __restrict__ part,
                                                          int* __restrict__ cnt) {
  using T = Fp8Rect<TN>;
  constexpr int BM = T::BM, BN = T::BN, S = T::kS;
  constexpr int EB = YDT == 2 ? 4 : 2;                 // bytes per output element
  constexpr int RB = 32 * TN * EB;                     // bytes of one output row of the wave's tile
  constexpr int kPitch = RB + 16;                      // staged row
  constexpr int kEpi = 1024 + 4 * 32 * kPitch;         // column scales, then 4 staging areas
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * T::kStage];
  static_assert(S * T::kStage >= kEpi + 4, "epilogue LDS and arrival flag");
  int* const s_last = reinterpret_cast<int*>(lds + kEpi);

  const int nk_all = K / T::kStep;
  int tm, tn, kb = 0, ke = nk_all, slot = -1, sk_tile = 0, R = 0;
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
    kb = piece * nk_all / split;
    ke = (piece + 1) * nk_all / split;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;
  // epilogue inputs, fetched now so their latency hides under the K loop
  float rsx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) rsx[i] = sx[min(m0 + wm * 64 + 32 * i + fr, M - 1)];
  const float my_sw = sw[min(n0 + min(tid, BN - 1), N - 1)];

  const RectSrc d = rect_src<TN>(A, B, m0, n0, M, N, K, kb * T::kStep, wave, lane);
  const int nk = ke - kb;

  v16f acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int s = 0; s < S; ++s) rect_issue<TN>(lds, s, nk, d, wave);
  wait_vmcnt<(S - 1) * T::kLoads>();              // step 0 landed (this wave)
  block_barrier();                                // ... for every wave
  v8i fa[2 + TN], fb[2 + TN];
#pragma unroll
  for (int f = 0; f < 2 + TN; ++f) {
    const int row = rect_row<TN>(f, wm, wn, fr);
    const v4i lo = *reinterpret_cast<const v4i*>(lds + rswz(row, fh));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + rswz(row, 2 + fh));
    fa[f] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  // K step kt: its first sub-step multiplies while its second's fragments are
  // read and the B rows of step kt-1+S go into the slot retired in the
  // previous step; then (step kt+1 landed everywhere, slot kt read by every
  // wave) the second multiplies while step kt+1's first fragments are read
  // and the A rows of step kt+S are fetched into slot kt. The first S steps
  // came whole with the fill. The last step runs the same code: its stray
  // reads stay in the ring, its loads repeat the last step into retired slots.
  for (int kt = 0; kt < nk; ++kt) {
    uint8_t* sc = lds + (kt % S) * T::kStage;
    if (kt > 0)
      rect_phase<TN, 2>(fa, fb, acc, sc, 1, wm, wn, lane, d, min(kt - 1 + S, nk - 1) * T::kStep,
                        lds + ((kt - 1) % S) * T::kStage, wave);
    else
      rect_phase<TN, 0>(fa, fb, acc, sc, 1, wm, wn, lane, d, 0, nullptr, wave);
    wait_lgkmcnt<0>();
    wait_vmcnt<(S - 2) * T::kLoads>();
    block_barrier();
    rect_phase<TN, 1>(fb, fa, acc, lds + ((kt + 1) % S) * T::kStage, 0, wm, wn, lane, d,
                      min(kt + S, nk - 1) * T::kStep, sc, wave);
  }
  wait_lgkmcnt<0>();
  wait_vmcnt<0>();                                // retire the trailing repeat loads
  block_barrier();                                // every wave is done with the ring

  if (slot >= 0) {
    // the square kernel's partial protocol: 16-byte chunk c of wave w's
    // accumulators at byte ((w * kChunks + c) * 64 + lane) * 16
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lane_off = (wv * T::kChunks * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t mine = partial_rsrc(part, slot, T::kPartBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (i * TN + j) * 4 + q;
          const v4f v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), mine, lane_off + c * 1024, 0, kSc1);
        }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial is visible
    __syncthreads();                                        // ... and every wave's
    if (tid == 0)
      *s_last = __hip_atomic_fetch_add(cnt + sk_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == split - 1;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(*s_last)) return;
    if (tid == 0) cnt[sk_tile] = 0;               // every slice has arrived: leave the counter zero
    // all slices' partials in slice order, this one's own included
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      for (int p = 0; p < split; ++p) {
        const __amdgpu_buffer_rsrc_t src = partial_rsrc(part, p * R + sk_tile, T::kPartBytes);
        v4f w[4 * TN];
#pragma unroll
        for (int t = 0; t < 4 * TN; ++t)
          w[t] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                             src, lane_off + (i * 4 * TN + t) * 1024, 0, kSc1));
#pragma unroll
        for (int t = 0; t < 4 * TN; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][t >> 2][4 * (t & 3) + e] = p == 0 ? w[t][e] : acc[i][t >> 2][4 * (t & 3) + e] + w[t][e];
      }
    }
  }

  // Epilogue: Y = acc * sx[m] * sw[n] rounded to the output type, staged one
  // 32-row block at a time (element r of tile (i, j) of a lane is row
  // m0 + wm*64 + 32i + (lane&31), column n0 + wn*32*TN + 32j + 8(r>>2) +
  // 4(lane>>5) + (r&3)) and stored as 16-byte pieces of whole rows.
  float* scol = reinterpret_cast<float*>(lds);
  if (tid < BN) scol[tid] = my_sw;
  __syncthreads();
  constexpr int CPR = RB / 16;                    // 16-byte chunks per staged row
  constexpr int EPC = 16 / EB;                    // elements per chunk
  const bool vec = (static_cast<int64_t>(N) * EB) % 16 == 0;
  char* const stg = reinterpret_cast<char*>(lds) + 1024 + wave * 32 * kPitch;
  char* const y = static_cast<char*>(Y);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        char* dst = stg + fr * kPitch + (32 * j + 8 * g + 4 * fh) * EB;
        const v4f cs = *reinterpret_cast<const v4f*>(scol + wn * 32 * TN + 32 * j + 8 * g + 4 * fh);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * rsx[i] * cs[e];
        if constexpr (YDT == 0) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16),
                                                      bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16));
        } else if constexpr (YDT == 1) {
          const uint32_t lo = f32x2_to_f16x2_bits(v[0], v[1]);
          const uint32_t hi = f32x2_to_f16x2_bits(v[2], v[3]);
          *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
        }
      }
    wave_lds_fence();
    const int mb = m0 + wm * 64 + 32 * i;
    const int nb = n0 + wn * 32 * TN;
#pragma unroll
    for (int t = 0; t < 32 * CPR / 64; ++t) {
      const int q = t * 64 + lane, row = q / CPR, c = q % CPR;
      const uint4 val = *reinterpret_cast<const uint4*>(stg + row * kPitch + c * 16);
      const int m = mb + row, n = nb + c * EPC;
      if (m < M) {
        char* dp = y + (static_cast<int64_t>(m) * N + n) * EB;
        if (vec && n + EPC <= N) {
          *reinterpret_cast<uint4*>(dp) = val;
        } else {
          const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            if (n + e >= N) break;
            if constexpr (EB == 2)
              *reinterpret_cast<uint16_t*>(dp + 2 * e) = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
            else
              *reinterpret_cast<uint32_t*>(dp + 4 * e) = w[e];
          }
        }
      }
    }
    wave_lds_fence();                             // staging reads done before the next block writes
  }
}

// ---------------------------------------------------------------------------
// Launch plan: block size (256 or 128) and K-slicing, all tiles alike, chosen
// by a bandwidth model of MI355X fitted to measured timings (microseconds):
//  * a 256x256 block step (32 KB of operands, 1024 MFMA cycles) takes
//    kStep256 on one CU;
//  * a 128x128 block step moves 16 KB, and one CU streams at most kCuRate
//    bytes/us into LDS (two blocks share a CU); its MFMAs take kMfma128;
//  * all CUs together stream at most kL2Rate bytes/us from L2;
//  * K-slicing writes every slice's fp32 partial and re-reads them all for the
//    last slice (through memory, kPartRate bytes/us) after a latency kSplitLat;
//  * kFixed per launch (start-up, epilogue);
//  * with K % 128 == 0, 128 x 128 and 128 x 192 blocks on 128-byte K steps
//    (one per CU): whole 128-byte row segments stream at kCuRateRect per CU,
//    under the same aggregate L2 rate; 128 x 128 blocks may be cut into at
//    most kFp8RectMaxSplit K-slices, the last slice of a tile writing its
//    partial and reading all of them at that per-CU rate after kSplitLat
//    (measured at 512 tokens: two slices of 128 x 128 blocks pay off for
//    K = 12288, N = 4096, where the whole tiles fill only half the CUs; more
//    slices, sliced 128 x 192 blocks, or slicing a grid that fills the chip
//    lose).
constexpr double kStep256 = 0.65;
constexpr double kCuRateRect = 75e3;
constexpr double kCuRate = 62e3;
constexpr double kMfma128 = 0.13;
constexpr double kL2Rate = 12e6;
constexpr double kPartRate = 5e6;
constexpr double kSplitLat = 2.0;
constexpr double kFixed = 3.0;
constexpr int kFp8MinSliceSteps = 4;
constexpr int kFp8MaxSplit = 16;
constexpr int kFp8RectMaxSplit = 2;

double fp8_plan_time(int64_t M, int64_t N, int64_t nk, int bm, int s, int cus) {
  const int64_t T = ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
  const int64_t units = T * s;
  const double per_cu = static_cast<double>((units + cus - 1) / cus);      // blocks on the busiest CU
  const double steps = static_cast<double>((nk + s - 1) / s);
  const double step_bytes = 2.0 * bm * kBK;
  const double total = static_cast<double>(units) * steps * step_bytes;
  double t = total / kL2Rate;
  if (bm == 256) t = std::max(t, per_cu * steps * kStep256);
  else t = std::max(t, per_cu * steps * std::max(step_bytes / kCuRate, kMfma128));
  if (s > 1) {
    const double part = 4.0 * bm * bm;
    t += (static_cast<double>(units) + static_cast<double>(T) * s) * part / kPartRate + kSplitLat;
  }
  return t + kFixed;
}

GemmPlan plan_fp8_gemm_split(int64_t M, int64_t N, int split, int bm) {
  GemmPlan p{};
  p.bm = bm;
  p.tiles_m = static_cast<int>((M + bm - 1) / bm);
  p.tiles_n = static_cast<int>((N + bm - 1) / bm);
  const int T = p.tiles_m * p.tiles_n;
  p.split = split;
  p.dp_tiles = split > 1 ? 0 : T;
  p.sk_tiles = split > 1 ? T : 0;
  return p;
}

GemmPlan plan_fp8_gemm_rect(int64_t M, int64_t N, int split, int bn) {
  GemmPlan p{};
  p.bm = 128;
  p.bn = bn;
  p.rect = true;
  p.tiles_m = static_cast<int>((M + 127) / 128);
  p.tiles_n = static_cast<int>((N + bn - 1) / bn);
  const int T = p.tiles_m * p.tiles_n;
  p.split = split;
  p.dp_tiles = split > 1 ? 0 : T;
  p.sk_tiles = split > 1 ? T : 0;
  return p;
}

GemmPlan plan_fp8_gemm(int64_t M, int64_t N, int64_t K, int cus) {
  if (K % kBK != 0 || cus <= 0) return plan_fp8_gemm_split(M, N, 1, 256);
  const int64_t nk = K / kBK;
  double best_t = 0.0;
  int best_bm = 256, best_s = 1;
  bool have = false;
  for (int bm : {256, 128}) {
    for (int s = 1; s == 1 || (s <= kFp8MaxSplit && s * kFp8MinSliceSteps <= nk); ++s) {
      const double t = fp8_plan_time(M, N, nk, bm, s, cus);
      if (!have || t < best_t) have = true, best_t = t, best_bm = bm, best_s = s;
    }
  }
  if (K % 128 == 0) {
    int rect_s = 1;
    for (int bn : {128, 192}) {
      const int64_t T = ((M + 127) / 128) * ((N + bn - 1) / bn);
      const double step_bytes = (128.0 + bn) * 128.0;
      const int smax = bn == 128 ? kFp8RectMaxSplit : 1;
      for (int s = 1; s <= smax && s * kFp8MinSliceSteps <= K / 128; ++s) {
        const int64_t units = T * s;
        const double steps = static_cast<double>((K / 128 + s - 1) / s);
        const double per_cu = static_cast<double>((units + cus - 1) / cus);
        double t = std::max(static_cast<double>(units) * steps * step_bytes / kL2Rate,
                            per_cu * steps * step_bytes / kCuRateRect) + kFixed;
        if (s > 1) t += (s + 1) * 4.0 * 128.0 * bn / kCuRateRect + kSplitLat;
        if (t < best_t) best_t = t, best_bm = -bn, rect_s = s;
      }
    }
    if (best_bm < 0) return plan_fp8_gemm_rect(M, N, rect_s, -best_bm);
  }
  GemmPlan p = plan_fp8_gemm_split(M, N, best_s, best_bm);
  // Whole 256x256 tiles in full waves and a partial last wave of R tiles:
  // that wave costs a full tile time on its CUs; as 4R 128x128 quarters (two
  // per CU) it takes about the time of one quarter, a little over half.
  const int T = p.tiles_m * p.tiles_n, R = T % cus;
  if (best_bm == 256 && best_s == 1 && T >= cus && R > 0 && 4 * R <= 2 * cus) {
    p.dp_tiles = T - R;
    p.sk_tiles = R;
    p.small = true;
  }
  return p;
}

// ydt: 0 bf16, 1 fp16, 2 fp32. `part` / `cnt`: plan.partial_bytes() of fp32
// partials and plan.counters() zeroed counters (left zero), when plan.split > 1.
void launch_fp8_gemm(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sx,
                     const float* sw, void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s) {
  const dim3 block(256);
  if (plan.rect && K % 128 == 0) {
    const dim3 grid(plan.dp_tiles + plan.sk_tiles * plan.split);
#define W8_FP8_ARGS A, B, (int)M, (int)N, (int)K, sx, sw, Y, plan.tiles_m, plan.tiles_n, plan.dp_tiles, plan.split, \
    part, cnt
    if (plan.bn == 192) {
      if (ydt == 0) k_fp8_gemm_rect<0, 3><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else if (ydt == 1) k_fp8_gemm_rect<1, 3><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else k_fp8_gemm_rect<2, 3><<<grid, block, 0, s>>>(W8_FP8_ARGS);
    } else {
      if (ydt == 0) k_fp8_gemm_rect<0, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else if (ydt == 1) k_fp8_gemm_rect<1, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else k_fp8_gemm_rect<2, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
    }
#undef W8_FP8_ARGS
    return;
  }
  if (K % kBK == 0) {
    constexpr int S = 4;
    if (plan.bm == 256 && plan.small) {
      // whole 256x256 tiles, then the leftover tiles as 128x128 quarters (a
      // second launch on the same stream, so it starts as the first ends)
      const dim3 grid(plan.dp_tiles), qgrid(4 * plan.sk_tiles);
#define W8_FP8_ARGS(Q) A, B, (int)M, (int)N, (int)K, sx, sw, Y, plan.tiles_m, plan.tiles_n, plan.dp_tiles, 1, part, \
    cnt, Q
      if (ydt == 0) {
        k_fp8_gemm_dma<0, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS(0));
        k_fp8_gemm_dma<0, S, 2><<<qgrid, block, 0, s>>>(W8_FP8_ARGS(1));
      } else if (ydt == 1) {
        k_fp8_gemm_dma<1, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS(0));
        k_fp8_gemm_dma<1, S, 2><<<qgrid, block, 0, s>>>(W8_FP8_ARGS(1));
      } else {
        k_fp8_gemm_dma<2, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS(0));
        k_fp8_gemm_dma<2, S, 2><<<qgrid, block, 0, s>>>(W8_FP8_ARGS(1));
      }
#undef W8_FP8_ARGS
      return;
    }
    const dim3 grid(plan.dp_tiles + plan.sk_tiles * plan.split);
#define W8_FP8_ARGS A, B, (int)M, (int)N, (int)K, sx, sw, Y, plan.tiles_m, plan.tiles_n, plan.dp_tiles, plan.split, \
    part, cnt, 0
    if (plan.bm == 256) {
      if (ydt == 0) k_fp8_gemm_dma<0, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else if (ydt == 1) k_fp8_gemm_dma<1, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else k_fp8_gemm_dma<2, S, 4><<<grid, block, 0, s>>>(W8_FP8_ARGS);
    } else {
      if (ydt == 0) k_fp8_gemm_dma<0, S, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else if (ydt == 1) k_fp8_gemm_dma<1, S, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
      else k_fp8_gemm_dma<2, S, 2><<<grid, block, 0, s>>>(W8_FP8_ARGS);
    }
#undef W8_FP8_ARGS
    return;
  }
  const int tiles_m = static_cast<int>((M + kFBM - 1) / kFBM);
  const int tiles_n = static_cast<int>((N + kFBN - 1) / kFBN);
  const dim3 grid(tiles_m * tiles_n);
  if (ydt == 0) k_fp8_gemm_any<0><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
  else if (ydt == 1) k_fp8_gemm_any<1><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
  else k_fp8_gemm_any<2><<<grid, block, 0, s>>>(A, B, (int)M, (int)N, (int)K, sx, sw, Y, tiles_m);
}

}  // namespace w8
