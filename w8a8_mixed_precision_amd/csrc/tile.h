// Device helpers shared by the 256x256-tile GEMM kernels (int8 and FP8):
// LDS swizzle, XCD-aware tile order, explicit wait counters, barriers, and the
// staged row write-back of the epilogue. Internal to libw8mp.
#pragma once

#include "common.h"

namespace w8 {

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Block tile: 256 x 256 outputs, K step of 64 bytes (one 64-byte row segment
// of each operand per step). 4 waves as 2x2, each 128x128.
constexpr int kBM = 256, kBN = 256, kBK = 64;

// LDS byte offset of logical 16-byte chunk `ch` (0..3) of tile row `row`
// (64 bytes per row). The fragment reads take 32 consecutive rows at one
// chunk per half-wave; XOR-ing the chunk with (row >> 2) & 3 makes them free
// of bank conflicts on gfx950 (measured with the SQ_LDS_BANK_CONFLICT counter:
// 0% of the LDS-active cycles, against 50% for ((row >> 1) ^ (row >> 3)) & 3,
// 50% for (row >> 1) & 3 and 75% for row & 3 or no XOR).
__device__ __forceinline__ int swz_term(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz64(int row, int ch) { return row * kBK + ((ch ^ swz_term(row)) << 4); }

// XCD-aware block order: the hardware deals consecutive workgroups round-robin
// over the 8 XCDs; renumber so each XCD gets a contiguous range of ids, then
// walk tiles in groups of kGroupM tile-rows so blocks that run together on one
// XCD share A rows and B columns in that XCD's L2.
constexpr int kXcds = 8, kGroupM = 8;

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = (nblocks + kXcds - 1) / kXcds;
  const int tall = nblocks - (per - 1) * kXcds;  // XCDs that get `per` blocks
  const int xcd = bid % kXcds, local = bid / kXcds;
  return (xcd < tall) ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ void group_tile(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int in_group = kGroupM * tiles_n;
  const int g = id / in_group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = id % in_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  group_tile(xcd_remap(bid, nblocks), tiles_m, tiles_n, tm, tn);
}

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

// Lanes of a wave exchange data through LDS staging. The hardware runs a
// wave's LDS accesses in issue order, but the compiler reasons per thread and
// may move one lane's read ahead of another lane's write (or a write ahead of
// another lane's read) to the same bytes: a wavefront-scope fence keeps the
// program order, at no cost in instructions.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Epilogue staging. The 32x32 MFMA results give each lane one output row and
// 4 consecutive columns per group of 4 registers; stored directly, every store
// instruction would touch 32 rows (32 partial cache lines). Instead each wave
// stages 32 rows x 256 bytes in LDS and writes them back as whole rows,
// 16 lanes x 16 bytes per row, 4 rows per instruction.
constexpr int kStgPitch = 256 + 16;             // staged row: 256 bytes + pad
constexpr int kStgWave = 32 * kStgPitch;        // one wave's 32 staged rows
constexpr int kEpiCols = 2048;                  // column scales and bias, 256 floats each
constexpr int kEpiLds = kEpiCols + 4 * kStgWave;   // + 4 staging areas

// Writes the wave's 32 staged rows (RB bytes each: 256 or 128; EB bytes per
// element) to Y rows m_base.. and columns n_base.., clipped to [M, N). `vec`:
// rows of Y are 16-byte aligned (N * EB % 16 == 0), so whole chunks can be
// stored. One instruction covers 64 / (RB / 16) rows. All the lane's chunks
// are read from the staging area first (one LDS round trip), then stored.
template <int EB, int RB = 256>
__device__ __forceinline__ void flush_staged(const char* stg, char* __restrict__ y, int M, int N, int m_base,
                                             int n_base, int lane, bool vec) {
  static_assert(RB == 256 || RB == 128, "staged row bytes");
  constexpr int EPC = 16 / EB;                  // elements per 16-byte chunk
  constexpr int CPR = RB / 16;                  // chunks per staged row
  constexpr int RPI = 64 / CPR;                 // rows per instruction
  constexpr int T = 32 / RPI;                   // store instructions
  const int ch = lane % CPR;
  const int n = n_base + ch * EPC;
  uint4 v[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    v[t] = *reinterpret_cast<const uint4*>(stg + (RPI * t + lane / CPR) * kStgPitch + ch * 16);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = m_base + RPI * t + lane / CPR;
    if (m < M) {
      char* dst = y + (static_cast<int64_t>(m) * N + n) * EB;
      if (vec && n + EPC <= N) {
        *reinterpret_cast<uint4*>(dst) = v[t];
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

// Split-K partials are written and read through buffer instructions with the
// agent-scope coherence bit (sc1), the form the compiler itself uses for
// agent-scope atomic loads and stores: those accesses are coherent across XCDs
// on their own, without the whole-L2 write-back / invalidate that a
// device-scope fence performs. Partial layout: 16-byte chunk c (0..63) of wave
// w's 256 accumulators at byte ((w*64 + c)*64 + lane)*16, so every access is
// 1 KB contiguous.
constexpr int kSc1 = 16;                        // cache-policy bit sc1
constexpr int kNt = 2;                          // cache-policy bit nt: streaming (non-temporal) access
constexpr int kRawBuffer = 0x00020000;          // word 3 of a raw buffer descriptor (32-bit data format)
constexpr int kPartWords = kBM * kBN;           // one 256x256 partial, 4-byte words

// Buffer descriptor of partial `slot` of `bytes` bytes (slots are contiguous).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(void* part, int slot, int bytes = kPartWords * 4) {
  return __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(part) + static_cast<int64_t>(slot) * bytes, 0, bytes,
                                           kRawBuffer);
}

// Operand rows for the LDS-DMA K loops. Each wave loads 16 rows per
// instruction, 4 lanes (16 bytes each) per 64-byte row segment; the rows a
// lane loads are 16 apart, so with the swizzle (row >> 2) & 3 its chunk is the
// same for all of them and one byte offset per lane serves every load of both
// operands. The descriptor covers rows r0.. of a K-contiguous int8 matrix with
// R rows (at most `rows` of them) from byte k_off of each row on; a load past
// the last valid row reads zeros (the buffer range check), and every offset
// stays below rows * K, within 32 bits for any K the library accepts.
struct DmaSrc {
  __amdgpu_buffer_rsrc_t a, b;   // the tile's rows of A and of B
  uint32_t voff;                 // this lane's offset: row and swizzled chunk
  int rows16;                    // bytes between the 16-row groups of a wave: 16 K
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const int8_t* P, int r0, int R, int K, int k_off,
                                                               int rows) {
  const int valid = min(R - r0, rows);
  const uint32_t n = valid > 0 ? static_cast<uint32_t>(valid) * static_cast<uint32_t>(K) - k_off : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(P) + static_cast<int64_t>(r0) * K + k_off, 0, n,
                                           kRawBuffer);
}

// rows_per_wave: 64 (256-row tiles) or 32 (128-row blocks).
__device__ __forceinline__ DmaSrc dma_src(const int8_t* A, const int8_t* B, int m0, int n0, int M, int N, int K,
                                          int k_off, int rows, int wave, int lane) {
  DmaSrc d;
  d.a = operand_rsrc(A, m0, M, K, k_off, rows);
  d.b = operand_rsrc(B, n0, N, K, k_off, rows);
  const int r = wave * (rows / 4) + (lane >> 2);
  d.voff = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + (((lane & 3) ^ swz_term(r)) << 4);
  d.rows16 = 16 * K;
  return d;
}

// Load i (16 rows) of this wave's share of operand A or B at byte k0 of the
// K range into LDS at dst (1 KB: the 16 rows' 64-byte segments). The row goes
// into the per-lane offset and k0 into the scalar one. The range check covers
// their sum (measured: with a descriptor spanning one row and the row's start
// in the scalar offset, every row past the first read as zeros); for a row
// inside the descriptor, row * K + k0 plus the chunk stays below its range.
__device__ __forceinline__ void dma_a(const DmaSrc& d, int8_t* dst, int i, int k0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.a, dst, 16, d.voff + i * d.rows16, k0, 0, 0);
}
__device__ __forceinline__ void dma_b(const DmaSrc& d, int8_t* dst, int i, int k0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.b, dst, 16, d.voff + i * d.rows16, k0, 0, 0);
}

}  // namespace w8
