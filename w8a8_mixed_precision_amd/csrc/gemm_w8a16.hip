// FP8-E4M3 weight-only (W8A16) GEMM for gfx950: bf16 activations, E4M3
// weights dequantised between LDS and the MFMA.
//
//   W_deq[n,k] = rne_bf16(e4m3(wq[n,k]) * sw[n])    (the product is exact in fp32)
//   acc[m,n]   = sum_k x[m,k] * W_deq[n,k]           (v_mfma_f32_32x32x16_bf16, fp32 sums)
//   Y[m,n]     = acc rounded to the output type
//
// The weight-only loader of the "Qwen-Image-2.1 Text Encoder: FP8" card
// (sections "Format" and "How it was tested"): each weight is its FP8 value
// times the bf16 scale of its output channel, in bf16, and the linear runs in
// bf16. Here the weights stay 1 byte each in HBM and in LDS; every wave
// widens the fragments it multiplies (v_cvt_pk_f32_fp8, a multiply by the
// channel scale, v_cvt_pk_bf16_f32 round to nearest even).
//
// Tiling follows the FP8 W8A8 kernel: 2x2 waves with WT x WT 32x32 tiles each
// (WT = 4: 256x256 blocks, one per CU; 2: 128x128, two per CU), an LDS-DMA
// ring of S stages, split-K with fp32 partials summed in slice order. One K
// step is 64 values: 128-byte rows of A (bf16) and 64-byte rows of B (E4M3).
// It runs as two sub-steps of 32 values; in sub-step h the lanes of half
// fh = lane >> 5 take k = 32h + 16fh .. +16: A chunks 4h + 2fh and 4h + 2fh + 1
// (8 bf16 each, one per MFMA) and B chunk 2h + fh (16 codes, widened into the
// two matching bf16 fragments). Both operands use the same k, so every k of
// the step is multiplied exactly once.
//
// The plain 16-bit linear on 256x256 blocks takes K steps of 32 values
// instead: 64-byte rows of both operands (the int8 GEMM's layout), one
// sub-step per step, A and B chunks 2fh and 2fh + 1, through a 4-stage ring of
// 32 KB. It streams the same 32 KB per 1024 MFMA cycles as the int8 GEMM; the
// 64-value step would leave room for only two 64 KB stages, one step of
// look-ahead, too little to cover the load latency.
#include <algorithm>

#include "launch.h"
#include "tile.h"

namespace w8 {

// B operand kinds: E4M3 codes widened to bf16 with the channel scale (the
// weight-only FP8 linear), or 16-bit weights used as they are (the plain
// 16-bit linear: bf16 x bf16 or f16 x f16). A has B's 16-bit type.
enum : int { kBE4M3 = 0, kBBF16 = 1, kBF16 = 2 };

template <int WT, int BK>
struct W16Tile {
  static constexpr int BM = 64 * WT;                  // block rows = block columns
  static constexpr int kKS = BK != kBE4M3 && WT == 4 ? 32 : 64;   // K values per step
  static constexpr int kSub = kKS / 32;               // sub-steps per K step
  static constexpr int kARow = 2 * kKS;               // bytes of an A row per K step (16-bit)
  static constexpr int kBRow = BK == kBE4M3 ? kKS : 2 * kKS;   // bytes of a B row per K step
  static constexpr int kABytes = BM * kARow;          // A of one K step
  static constexpr int kStage = kABytes + BM * kBRow; // A then B
  static constexpr int kALoads = kABytes / 4096;      // DMA instructions per wave per step (A)
  static constexpr int kBLoads = BM * kBRow / 4096;   // ... (B)
  static constexpr int kLoads = kALoads + kBLoads;
  static constexpr int kMfma = 2 * WT * WT;           // MFMAs per wave per sub-step
  static constexpr int kBReads = BK == kBE4M3 ? WT : 2 * WT;   // 16-byte B reads per sub-step
  static constexpr int kReads = kBReads + 2 * WT;     // 16-byte LDS reads per wave per sub-step
  static constexpr int kChunks = 4 * WT * WT;         // 16-byte accumulator chunks per lane
  static constexpr int kPartBytes = BM * BM * 4;      // one fp32 partial
};
// Ring stages: 3 (E4M3 B: 144 KB at WT = 4, 72 KB at WT = 2, two blocks per
// CU); 16-bit B: 3 at WT = 2 (96 KB, one block per CU), 4 at WT = 4 (32-value
// steps, 128 KB).
template <int WT, int BK>
constexpr int w16_stages() { return BK == kBE4M3 ? 3 : (WT == 4 ? 4 : 3); }

// A rows: 8 chunks of 16 bytes, XOR-permuted by (row >> 1) & 7 so that the 32
// rows a half-wave reads at one chunk spread over the banks.
__device__ __forceinline__ int swz_a128(int row, int ch) { return row * 128 + ((ch ^ ((row >> 1) & 7)) << 4); }

// The target builtins behind plain functions (with template-dependent
// arguments the host compilation pass can drop the kernel templates).
// The operand loads are buffer loads into LDS: a per-lane byte offset that
// stays in one register for the whole loop plus the K step's offset in a
// scalar register (an address computed afresh for every load leaves the
// register allocator free to reuse its registers for fragment reads right
// after the load, and the compiler then waits for every load in flight).
__device__ __forceinline__ void w16_dma(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                 0);
}
__device__ __forceinline__ v16f mfma_f16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}
template <int BK>
__device__ __forceinline__ v16f mfma16(v4i a, v4i b, v16f c) {
  if constexpr (BK == kBF16) return mfma_f16(a, b, c);
  else return mfma_bf16(a, b, c);
}

// Eight E4M3 codes (bytes of w0, then w1) -> eight bf16 weights
// rne_bf16(value * s); the float product of a code and a bf16 scale is exact.
__device__ __forceinline__ v4i widen8(uint32_t w0, uint32_t w1, float s) {
  const v2f p0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);
  const v2f p1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);
  const v2f p2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);
  const v2f p3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);
  const float f[8] = {p0.x * s, p0.y * s, p1.x * s, p1.y * s, p2.x * s, p2.y * s, p3.x * s, p3.y * s};
  v8bf r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(f[e]);
  return __builtin_bit_cast(v4i, r);
}

// Fragments of one sub-step (16 bytes each, kept as plain vectors): a[i][q]
// (row block i, MFMA q), b[j][q], and for E4M3 the B chunks before widening.
template <int WT>
struct W16Frags {
  v4i a[WT][2];
  v4i b[WT][2];
  v4u raw[WT];
};

// Read number o (0 .. kReads-1) of a sub-step's fragments from stage `sl`: B
// first (E4M3 chunks still need widening), then A in consumption order.
template <int WT, int BK>
__device__ __forceinline__ void w16_read(W16Frags<WT>& F, const uint8_t* sl, int o, int h, int wm, int wn, int fr,
                                         int fh) {
  using T = W16Tile<WT, BK>;
  // byte offset of chunk (2h + fh) * 2 + q of a 16-bit row
  auto at16 = [](int row, int q, int h, int fh) {
    return T::kKS == 32 ? swz64(row, 2 * fh + q) : swz_a128(row, 4 * h + 2 * fh + q);
  };
  if (o < T::kBReads) {
    if constexpr (BK == kBE4M3) {
      const int row = wn * 32 * WT + 32 * o + fr;
      F.raw[o] = *reinterpret_cast<const v4u*>(sl + T::kABytes + swz64(row, 2 * h + fh));
    } else {
      const int j = o >> 1, q = o & 1;
      const int row = wn * 32 * WT + 32 * j + fr;
      F.b[j][q] = *reinterpret_cast<const v4i*>(sl + T::kABytes + at16(row, q, h, fh));
    }
  } else {
    const int a = o - T::kBReads, i = a >> 1, q = a & 1;
    const int row = wm * 32 * WT + 32 * i + fr;
    F.a[i][q] = *reinterpret_cast<const v4i*>(sl + at16(row, q, h, fh));
  }
}

template <int WT>
__device__ __forceinline__ void w16_widen(W16Frags<WT>& F, int j, float s) {
  F.b[j][0] = widen8(F.raw[j][0], F.raw[j][1], s);
  F.b[j][1] = widen8(F.raw[j][2], F.raw[j][3], s);
}

// DMA of K-step kt into its ring slot (past the last step the last step is
// loaded again into the slot just retired, which no later step reads, so every
// step issues the same number of loads).
template <int WT, int BK, int S>
__device__ __forceinline__ void w16_issue_one(uint8_t* lds, int kt, int nk, int d, __amdgpu_buffer_rsrc_t ra,
                                              __amdgpu_buffer_rsrc_t rb, const uint32_t* a_off,
                                              const uint32_t* b_off, int wave) {
  using T = W16Tile<WT, BK>;
  uint8_t* st = lds + (kt % S) * T::kStage;
  const uint32_t k0 = static_cast<uint32_t>(min(kt, nk - 1));
  if (d < T::kALoads)
    w16_dma(ra, st + (wave * T::kALoads + d) * 1024, a_off[d], k0 * static_cast<uint32_t>(T::kARow));
  else
    w16_dma(rb, st + T::kABytes + (wave * T::kBLoads + d - T::kALoads) * 1024, b_off[d - T::kALoads],
            k0 * static_cast<uint32_t>(T::kBRow));
}

// One sub-step: the wave's 2*WT*WT MFMAs on fragments C, while the next
// sub-step's fragments are read from stage `sn` (sub-step hn) into N and
// widened, and (DMA) the loads of K-step kt_dma go out into the retired slot.
// Each MFMA is followed by its share of the reads, widenings and loads;
// sched_barrier keeps that order.
template <int WT, int BK, int S, bool DMA>
__device__ __forceinline__ void w16_phase(const W16Frags<WT>& C, W16Frags<WT>& N, v16f (*acc)[WT], const uint8_t* sn,
                                          int hn, int wm, int wn, int fr, int fh, const float* sc, uint8_t* lds,
                                          int kt_dma, int nk, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          const uint32_t* a_off, const uint32_t* b_off, int wave) {
  using T = W16Tile<WT, BK>;
  constexpr int kT = T::kMfma;
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    const int i = t / (2 * WT), j = (t / 2) % WT, q = t & 1;
    acc[i][j] = mfma16<BK>(C.b[j][q], C.a[i][q], acc[i][j]);
#pragma unroll
    for (int o = t * T::kReads / kT; o < (t + 1) * T::kReads / kT; ++o)
      w16_read<WT, BK>(N, sn, o, hn, wm, wn, fr, fh);
    // widen E4M3 chunk j' at MFMA kT/2 + j' * kT/(2*WT), long after its read
    if constexpr (BK == kBE4M3) {
      if (t >= kT / 2 && (t - kT / 2) % (kT / (2 * WT)) == 0) {
        const int jw = (t - kT / 2) / (kT / (2 * WT));
        w16_widen<WT>(N, jw, sc[jw]);
      }
    }
    if constexpr (DMA) {
#pragma unroll
      for (int d = t * T::kLoads / kT; d < (t + 1) * T::kLoads / kT; ++d)
        w16_issue_one<WT, BK, S>(lds, kt_dma, nk, d, ra, rb, a_off, b_off, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// YDT: 0 bf16, 1 fp16, 2 fp32; BK: the B operand kind. sw: channel scales
// (E4M3 only; unused otherwise). Grid and split-K protocol of the FP8 W8A8
// kernel: blocks below dp_tiles own whole tiles; the rest are `split`
// K-slices of R = (gridDim.x - dp_tiles) / split tiles, whose fp32 partials go
// to their own slots of `part`; the last slice of a tile to arrive (counter in
// `cnt`, zero on entry and left zero) sums all partials in slice order.
template <int YDT, int WT, int BK>
__global__ __launch_bounds__(256, BK == kBE4M3 ? 4 / WT : 1) void k_w8a16_gemm(const uint16_t* __restrict__ A,
                                                            const uint8_t* __restrict__ B, int M, int N, int K,
                                                            const float* __restrict__ sw, void* __restrict__ Y,
                                                            int tiles_m, int tiles_n, int dp_tiles, int split,
                                                            float* __restrict__ part, int* __restrict__ cnt) {
  using T = W16Tile<WT, BK>;
  constexpr int S = w16_stages<WT, BK>();
  constexpr int BM = T::BM;
  // one LDS object (see the int8 kernel); the arrival flag lives past the
  // epilogue's area
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * T::kStage];
  static_assert(sizeof(lds) >= kEpiLds + 4, "epilogue LDS and arrival flag");
  int* const s_last = reinterpret_cast<int*>(lds + kEpiLds);

  constexpr int KS = T::kKS;
  const int nk_all = K / KS;
  int tm, tn, kb = 0, ke = nk_all;
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
    kb = piece * nk_all / split;
    ke = (piece + 1) * nk_all / split;
  }
  const int m0 = tm * BM, n0 = tn * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;

  // channel scales of the lane's B rows (output columns), one per column block
  float sc[WT];
#pragma unroll
  for (int j = 0; j < WT; ++j) sc[j] = BK == kBE4M3 ? sw[min(n0 + wn * 32 * WT + 32 * j + fr, N - 1)] : 1.0f;

  // DMA sources, as byte offsets into X and Wq8. 128-byte rows (16-bit, 64
  // values per step): load d of wave w covers rows (w*loads + d)*8 + lane/8,
  // LDS slot (lane & 7) holding chunk (lane & 7) ^ ((row >> 1) & 7). 64-byte
  // rows (E4M3 B, or 16-bit at 32 values per step): rows (w*loads + d)*16 +
  // lane/4, slot (lane & 3) holding chunk (lane & 3) ^ swz_term(row).
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A), 0, static_cast<int>(static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u),
      kRawBuffer);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(B), 0,
      static_cast<int>(static_cast<uint32_t>(N) * static_cast<uint32_t>(K) * (BK == kBE4M3 ? 1u : 2u)), kRawBuffer);
  // byte offset of this lane's 16-byte chunk for load d of a 16-bit operand
  auto off16 = [&](int row0, int rows, int d, int loads) -> uint32_t {
    int r, ch;
    if constexpr (KS == 32) {
      r = (wave * loads + d) * 16 + (lane >> 2);
      ch = (lane & 3) ^ swz_term(r);
    } else {
      r = (wave * loads + d) * 8 + (lane >> 3);
      ch = (lane & 7) ^ ((r >> 1) & 7);
    }
    return (static_cast<uint32_t>(min(row0 + r, rows - 1)) * static_cast<uint32_t>(K) + kb * KS) * 2u + ch * 16;
  };
  uint32_t a_off[T::kALoads], b_off[T::kBLoads];
#pragma unroll
  for (int d = 0; d < T::kALoads; ++d) a_off[d] = off16(m0, M, d, T::kALoads);
#pragma unroll
  for (int d = 0; d < T::kBLoads; ++d) {
    if constexpr (BK == kBE4M3) {
      const int r = (wave * T::kBLoads + d) * 16 + (lane >> 2);
      const int ch = (lane & 3) ^ swz_term(r);
      b_off[d] = static_cast<uint32_t>(min(n0 + r, N - 1)) * static_cast<uint32_t>(K) + kb * 64 + ch * 16;
    } else {                                    // 16-bit rows: the layout of A
      b_off[d] = off16(n0, N, d, T::kBLoads);
    }
  }
  const int nk = ke - kb;

  v16f acc[WT][WT];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int d = 0; d < T::kLoads; ++d) w16_issue_one<WT, BK, S>(lds, s, nk, d, ra, rb, a_off, b_off, wave);
  wait_vmcnt<(S - 1) * T::kLoads>();            // step 0 landed (this wave)
  block_barrier();                              // ... for every wave
  W16Frags<WT> f0, f1;
#pragma unroll
  for (int o = 0; o < T::kReads; ++o) w16_read<WT, BK>(f0, lds, o, 0, wm, wn, fr, fh);
  if constexpr (BK == kBE4M3) {
#pragma unroll
    for (int j = 0; j < WT; ++j) w16_widen<WT>(f0, j, sc[j]);
  }

  if constexpr (T::kSub == 1) {
    // one sub-step per K step: wait for step kt+1 (all waves) and for every
    // wave to be done reading step kt's slot, then multiply step kt while
    // reading step kt+1's fragments and loading step kt+S into the retired
    // slot. The last step runs the same code: its reads stay in the ring, and
    // its loads repeat the last step into its own slot, which no later step reads.
    auto body = [&](const W16Frags<WT>& C, W16Frags<WT>& Nx, int kt) {
      wait_lgkmcnt<0>();
      wait_vmcnt<(S - 2) * T::kLoads>();
      block_barrier();
      w16_phase<WT, BK, S, true>(C, Nx, acc, lds + ((kt + 1) % S) * T::kStage, 0, wm, wn, fr, fh, sc, lds, kt + S,
                                 nk, ra, rb, a_off, b_off, wave);
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      body(f0, f1, kt);
      body(f1, f0, kt + 1);
    }
    if (kt < nk) body(f0, f1, kt);
  } else {
  for (int kt = 0; kt < nk - 1; ++kt) {
    const uint8_t* sa = lds + (kt % S) * T::kStage;
    // sub-step 0 multiplies while sub-step 1's fragments are read
    w16_phase<WT, BK, S, false>(f0, f1, acc, sa, 1, wm, wn, fr, fh, sc, lds, 0, nk, ra, rb, a_off, b_off, wave);
    wait_lgkmcnt<0>();                          // this slot is fully read
    wait_vmcnt<(S - 2) * T::kLoads>();          // step kt+1 landed (this wave)
    block_barrier();                            // ... for every wave; slot kt retired
    // sub-step 1 multiplies while step kt+1's first fragments are read and
    // step kt+S is fetched into the retired slot
    w16_phase<WT, BK, S, true>(f1, f0, acc, lds + ((kt + 1) % S) * T::kStage, 0, wm, wn, fr, fh, sc, lds, kt + S,
                               nk, ra, rb, a_off, b_off, wave);
  }
  {
    const uint8_t* sa = lds + ((nk - 1) % S) * T::kStage;
#pragma unroll
    for (int o = 0; o < T::kReads; ++o) w16_read<WT, BK>(f1, sa, o, 1, wm, wn, fr, fh);
    if constexpr (BK == kBE4M3) {
#pragma unroll
      for (int j = 0; j < WT; ++j) w16_widen<WT>(f1, j, sc[j]);
    }
#pragma unroll
    for (int t = 0; t < T::kMfma; ++t) {
      const int i = t / (2 * WT), j = (t / 2) % WT, q = t & 1;
      acc[i][j] = mfma16<BK>(f0.b[j][q], f0.a[i][q], acc[i][j]);
    }
#pragma unroll
    for (int t = 0; t < T::kMfma; ++t) {
      const int i = t / (2 * WT), j = (t / 2) % WT, q = t & 1;
      acc[i][j] = mfma16<BK>(f1.b[j][q], f1.a[i][q], acc[i][j]);
    }
  }
  }
  wait_lgkmcnt<0>();
  wait_vmcnt<0>();                              // retire the trailing repeat loads
  block_barrier();                              // every wave is done with the ring

  if (slot >= 0) {
    // partial layout: 16-byte chunk c of wave w's accumulators at byte
    // ((w * kChunks + c) * 64 + lane) * 16, every access 1 KB contiguous
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
    // all slices' partials in slice order (this slice's own read back too),
    // one 32-row block at a time
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

  // Epilogue: Y = acc rounded to the output type, staged through LDS a 32-row
  // block at a time (element r of tile (i, j) of a lane is row
  // m0 + wm*32*WT + 32i + (lane&31), column n0 + wn*32*WT + 32j + 8(r>>2)
  // + 4(lane>>5) + (r&3): the weight fragment is the MFMA's first operand).
  constexpr int EB = YDT == 2 ? 4 : 2;
  constexpr int ROWB = 32 * WT * EB;
  constexpr int H = ROWB > 256 ? ROWB / 256 : 1;
  constexpr int PJ = WT / H;
  constexpr int RB = 32 * PJ * EB;
  const bool vec = (static_cast<int64_t>(N) * EB) % 16 == 0;
  char* const stg = reinterpret_cast<char*>(lds) + kEpiCols + wave * kStgWave;
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
          const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
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
      wave_lds_fence();
    }
  }
}

// ---------------------------------------------------------------------------
// Launch plan: block size (256 or 128) and K-slicing, all tiles alike, chosen
// by a model of measured MI355X timings (microseconds; 512-token text-encoder
// shapes, K = 4096 and 12288):
//  * a 256x256 block step (48 KB of operands, 2048 MFMA cycles per wave)
//    takes kW16Step256 on its CU;
//  * a lone 128x128 block step (24 KB) takes kW16Lat128 (latency-bound); two
//    blocks share a CU, which streams at most kW16CuRate bytes/us into LDS;
//  * all CUs together stream at most kW16L2Rate bytes/us from L2;
//  * K-slicing writes every slice's fp32 partial and re-reads them all for
//    the last slice (kW16PartRate bytes/us) after a latency kW16SplitLat;
//  * kW16Fixed per launch.
constexpr double kW16Step256 = 2.0;
constexpr double kW16Lat128 = 0.60;
constexpr double kW16CuRate = 46e3;
constexpr double kW16L2Rate = 10e6;
constexpr double kW16PartRate = 5e6;
constexpr double kW16SplitLat = 2.0;
constexpr double kW16Fixed = 3.0;
constexpr int kW16MinSliceSteps = 4;
constexpr int kW16MaxSplit = 16;

static double w16_plan_time(int64_t M, int64_t N, int64_t nk, int bm, int s, int cus) {
  const int64_t T = ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
  const int64_t units = T * s;
  const int64_t per_cu = (units + cus - 1) / cus;                          // blocks on the busiest CU
  const double steps = static_cast<double>((nk + s - 1) / s);
  const double step_bytes = 192.0 * bm;
  const double total = static_cast<double>(units) * steps * step_bytes;
  double t = total / kW16L2Rate;
  if (bm == 256) {
    t = std::max(t, static_cast<double>(per_cu) * steps * kW16Step256);
  } else {
    const double rounds = static_cast<double>((per_cu + 1) / 2);          // two blocks run together
    const double conc = static_cast<double>(std::min<int64_t>(per_cu, 2));
    t = std::max(t, rounds * steps * std::max(kW16Lat128, conc * step_bytes / kW16CuRate));
  }
  if (s > 1) {
    const double part = 4.0 * bm * bm;
    t += (static_cast<double>(units) + static_cast<double>(T) * s) * part / kW16PartRate + kW16SplitLat;
  }
  return t + kW16Fixed;
}

GemmPlan plan_w8a16_gemm_split(int64_t M, int64_t N, int split, int bm) {
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

GemmPlan plan_w8a16_gemm(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t nk = K / 64;
  double best_t = 0.0;
  int best_bm = 256, best_s = 1;
  bool have = false;
  for (int bm : {256, 128}) {
    for (int s = 1; s == 1 || (s <= kW16MaxSplit && s * kW16MinSliceSteps <= nk); ++s) {
      const double t = w16_plan_time(M, N, nk, bm, s, std::max(cus, 1));
      if (!have || t < best_t) have = true, best_t = t, best_bm = bm, best_s = s;
    }
  }
  return plan_w8a16_gemm_split(M, N, best_s, best_bm);
}

// Plain 16-bit linear. 256x256 blocks (32-value K steps): the tiles of the
// device's full waves run whole and the R leftover tiles of the last, partial
// wave (every tile when there are fewer than the CUs) run as `split` K-slices,
// so the tail costs 1/split of a tile plus the partial exchange. Model
// (microseconds, measured at 4352x16384 -> 4096): a 32-value step of a
// 256x256 block takes kL16Step on its CU while every CU streams, kL16TailStep
// in a sparse tail wave; the last slice of a cut tile reads the split fp32
// partials of 256 KB at kL16Part each, after kL16SplitLat. The 128x128 plan
// of the weight-only model (its byte terms scaled by 4/3 for the 16-bit B
// rows) is taken when it is cheaper (small outputs).
constexpr double kL16Step = 1.1;
constexpr double kL16TailStep = 0.75;
constexpr double kL16Part = 6.0;
constexpr double kL16SplitLat = 3.0;

GemmPlan plan_linear16_tail(int64_t M, int64_t N, int split, int cus) {
  GemmPlan p = plan_w8a16_gemm_split(M, N, 1, 256);
  const int T = p.tiles_m * p.tiles_n;
  if (split <= 1) return p;
  const int R = T % std::max(cus, 1);
  p.split = split;
  p.dp_tiles = T - R;
  p.sk_tiles = R;
  if (R == 0) p.split = 1;
  return p;
}

static double l16_tail_time(int64_t T, int64_t nk, int s, int cus) {
  const int64_t R = T % cus, full = T / cus;
  double t = static_cast<double>(full) * nk * kL16Step;
  if (R > 0) {
    const double rounds = static_cast<double>((R * s + cus - 1) / cus);
    t += rounds * static_cast<double>((nk + s - 1) / s) * (R * s >= cus ? kL16Step : kL16TailStep);
    if (s > 1) t += kL16SplitLat + s * kL16Part;
  }
  return t + kW16Fixed;
}

GemmPlan plan_linear16(int64_t M, int64_t N, int64_t K, int cus) {
  cus = std::max(cus, 1);
  const int64_t nk = K / 32;
  const int64_t T = ((M + 255) / 256) * ((N + 255) / 256);
  double best_t = 0.0;
  int best_s = 1;
  for (int s = 1; s == 1 || (s <= kW16MaxSplit && s * kW16MinSliceSteps <= nk); ++s) {
    const double t = l16_tail_time(T, nk, s, cus);
    if (s == 1 || t < best_t) best_t = t, best_s = s;
  }
  const int64_t nk64 = K / 64;
  double best128 = 0.0;
  int s128 = 1;
  for (int s = 1; s == 1 || (s <= kW16MaxSplit && s * kW16MinSliceSteps <= nk64); ++s) {
    const double t = w16_plan_time(M, N, nk64, 128, s, cus) * (4.0 / 3.0);
    if (s == 1 || t < best128) best128 = t, s128 = s;
  }
  if (best128 < best_t) return plan_w8a16_gemm_split(M, N, s128, 128);
  return plan_linear16_tail(M, N, best_s, cus);
}

// K % 64 == 0 (checked by the caller). ydt: 0 bf16, 1 fp16, 2 fp32. `part` /
// `cnt`: plan.partial_bytes() of fp32 partials and plan.counters() zeroed
// counters (left zero), when plan.split > 1. bk: kBE4M3 (B = E4M3 codes, sw
// their channel scales, A bf16), kBBF16 / kBF16 (B and A 16-bit, sw unused).
template <int BK>
static void launch_w16(const uint16_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sw, void* Y,
                       int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s) {
  const dim3 block(256);
  const dim3 grid(plan.dp_tiles + plan.sk_tiles * plan.split);
#define W8_W16_ARGS A, B, (int)M, (int)N, (int)K, sw, Y, plan.tiles_m, plan.tiles_n, plan.dp_tiles, plan.split, part, cnt
  if (plan.bm == 256) {
    if (ydt == 0) k_w8a16_gemm<0, 4, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
    else if (ydt == 1) k_w8a16_gemm<1, 4, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
    else k_w8a16_gemm<2, 4, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
  } else {
    if (ydt == 0) k_w8a16_gemm<0, 2, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
    else if (ydt == 1) k_w8a16_gemm<1, 2, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
    else k_w8a16_gemm<2, 2, BK><<<grid, block, 0, s>>>(W8_W16_ARGS);
  }
#undef W8_W16_ARGS
}

void launch_w8a16_gemm(const uint16_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, const float* sw,
                       void* Y, int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s) {
  launch_w16<kBE4M3>(A, B, M, N, K, sw, Y, ydt, plan, part, cnt, s);
}

// The plain 16-bit linear Y = X W^T (X and W both bf16, or both f16), on the
// same kernel with the 16-bit weights used as they are.
void launch_linear16(const uint16_t* A, const uint16_t* B, bool bf16, int64_t M, int64_t N, int64_t K, void* Y,
                     int ydt, const GemmPlan& plan, float* part, int* cnt, hipStream_t s) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(B);
  if (bf16) launch_w16<kBBF16>(A, b, M, N, K, nullptr, Y, ydt, plan, part, cnt, s);
  else launch_w16<kBF16>(A, b, M, N, K, nullptr, Y, ydt, plan, part, cnt, s);
}

}  // namespace w8
