// Row quantisation kernels of libw8mp (gfx950).
//
//  k_int8_rows       one pass over each row: outlier-column flags (|x| > t),
//                    the provisional scale s' = max |x| over the elements with
//                    |x| <= t, and int8 codes with it. Without flags (t = inf)
//                    it is the rowwise weight quantiser.
//  k_outlier_fixup   the outlier set from the flags; zero the codes of the
//                    outlier columns, gather those columns of X (XO) and of Wq
//                    as 16-bit values (WO), and re-encode the rare rows whose
//                    scale must change.
//  k_fp8_rows        per-row (or static) scale and E4M3 codes.
//
// The LLM.int8 decomposition ("Image21-INT8" card, section "Quantization":
// threshold 6.0, outliers in floating point): a row's scale ignores every
// column that is an outlier column in ANY row of the call. One pass cannot
// know that set, so the row pass takes s' over |x| <= t. The true scale
// differs from s' only when s' is reached in outlier columns alone; the
// fix-up sees exactly those values when it gathers XO, so it re-encodes a row
// when its largest gathered |x| <= t equals s'.
//
// Both 16-bit formats store a sign bit and a magnitude whose bit patterns
// order like the magnitudes, so maxima and threshold tests run on packed
// 16-bit integers (bits & 0x7FFF): |x| > t exactly when the magnitude bits
// exceed those of the largest representable value <= t. Non-finite values
// have the largest patterns: with a finite t they are outliers.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "produce.h"

namespace w8 {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short ss2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}

// per 16-bit half: 0xFFFF where the magnitude m exceeds t2's half, else 0
// (t - m as a signed 16-bit difference is negative exactly then; both are
// 15-bit magnitudes)
__device__ __forceinline__ uint32_t pk_gt_mask(uint32_t m, uint32_t t2) {
  const ss2 d = __builtin_bit_cast(ss2, t2) - __builtin_bit_cast(ss2, m);
  return __builtin_bit_cast(uint32_t, static_cast<ss2>(d >> static_cast<short>(15)));
}

// 8 codes of one 16-byte chunk: q = rne(fl32(x * r)) as a byte. Adding
// 1.5 * 2^23 rounds fl32(x * r) (|.| <= 127.x) to the nearest integer, ties
// to even, and leaves it in the low mantissa bits. A row scale below
// 127/FLT_MAX makes r = +inf: then every non-zero x saturates to +-127 and
// zero stays 0. (Outlier elements, |x| > t, get arbitrary bytes here: the
// fix-up zeroes every code of an outlier column.)
template <bool BF16>
__device__ __forceinline__ uint2 encode8(const uint4& v, float r) {
#pragma clang fp contract(off)  // the product is rounded before the add: no FMA
  float f[8];
  unpack8<BF16>(v, f);
  uint32_t b[8];
  if (__builtin_isinf(r)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = f[j] > 0.0f ? 0x7Fu : (f[j] < 0.0f ? 0x81u : 0u);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = f[j] * r;
      b[j] = __float_as_uint(p + 12582912.0f) & 0xFFu;
    }
  }
  return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}

// Packed maximum of the magnitudes <= t of one chunk; the columns of the
// magnitudes > t get this call's stamp in their flag word (a plain store: many
// rows flag the same few columns, and equal plain stores need no atomics).
template <bool ACT>
__device__ __forceinline__ uint32_t chunk_scan(const uint4& v, uint32_t t2, uint32_t* __restrict__ flags, int c,
                                               uint32_t stamp) {
  uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
  if constexpr (ACT) {
    uint32_t gt[4], any = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gt[i] = pk_gt_mask(w[i], t2);
      any |= gt[i];
      w[i] &= ~gt[i];
    }
    if (any) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (gt[i] & 0xFFFFu) flags[8 * c + 2 * i] = stamp;
        if (gt[i] >> 16) flags[8 * c + 2 * i + 1] = stamp;
      }
    }
  }
  return pk_max_u16(pk_max_u16(w[0], w[1]), pk_max_u16(w[2], w[3]));
}

template <bool BF16>
__device__ __forceinline__ float decode_mag(uint32_t bits) {
  if constexpr (BF16) return __uint_as_float(bits << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

template <bool BF16>
__device__ __forceinline__ uint32_t mag_bits(float s) {   // s is a value of the 16-bit format
  if constexpr (BF16) return __float_as_uint(s) >> 16;
  else return __builtin_bit_cast(uint16_t, static_cast<_Float16>(s));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}

// --------------------------------------------------------------------------
// Row pass, register form (K <= 16384): W = ceil(K / 4096) waves per row, each
// covering a 4096-column slice, 8 chunks of 8 elements per lane; a block of NW
// waves holds NW/W rows per iteration. With W == 1 the row reduction stays
// inside one wave (no LDS, no barrier).
//
// With a producer (PROD != kProdNone) the loaded values are H, and X is made
// from them in registers (produce.h) before anything else; RMSNorm first
// reduces the row's sum of squares and stores the row's rstd for the fix-up.
// flags: one word per column; a column with some |x| > t gets `stamp`.
// This wave's share of row group row0 (row row0 + wave / W, part wave % W):
// up to 8 chunks of 8 values per lane.
template <int W>
__device__ __forceinline__ void rows_load(const uint16_t* __restrict__ X, int64_t rows, int K, int64_t row0,
                                          uint4 (&v)[8]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = row0 + wave / W;
  const int part = wave % W;
  const int nch = K >> 3;
  if (row < rows) {
    const uint4* xr = reinterpret_cast<const uint4*>(X + row * K);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = part * 512 + lane + 64 * i;
      if (c < nch) v[i] = xr[c];
    }
  }
}

// The row pass over one row group whose chunks rows_load put in v.
template <bool BF16, int W, int NW, bool ACT, int PROD>
__device__ __forceinline__ void rows_process(uint4 (&v)[8], int64_t rows, int K, uint32_t tbits,
                                             int8_t* __restrict__ q, float* __restrict__ sx,
                                             uint32_t* __restrict__ flags, uint32_t stamp, const ProdArgs& pa,
                                             int64_t row0, uint32_t* red, double* red64, const uint16_t* gelu) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = row0 + wave / W;
  const bool valid = row < rows;
  const int part = wave % W;
  const int nch = K >> 3;
  const uint32_t t2 = tbits | (tbits << 16);
  if constexpr (PROD != kProdNone) {
    float rstd = 0.0f;
    if constexpr (PROD == kProdRms) {
      double ss = 0.0;
      if (valid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = part * 512 + lane + 64 * i;
          if (c < nch) ss += sumsq8<BF16>(v[i]);
        }
      }
      ss = wave_sum_f64(ss);
      if constexpr (W > 1) {
        if (lane == 0) red64[wave] = ss;
        __syncthreads();
        const int w0 = (wave / W) * W;
        ss = red64[w0];
#pragma unroll
        for (int w = 1; w < W; ++w) ss += red64[w0 + w];
      }
      rstd = rms_rstd(ss, K, pa.eps);
      if (valid && part == 0 && lane == 0) pa.rstd[row] = rstd;
    }
    if (valid) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = part * 512 + lane + 64 * i;
        if (c < nch) v[i] = produce8<BF16, PROD>(v[i], c, rstd, pa, gelu);
      }
    }
  }
  uint32_t mx = 0;
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = part * 512 + lane + 64 * i;
      if (c < nch) mx = pk_max_u16(mx, chunk_scan<ACT>(v[i], t2, flags, c, stamp));
    }
  }
  mx = wave_max_u32(max(mx & 0xFFFFu, mx >> 16));
  if constexpr (W > 1) {
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const int w0 = (wave / W) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) mx = max(mx, red[w0 + w]);
    __syncthreads();                             // red and red64 are reused by the next iteration
  }
  if (!valid) return;
  const float s = decode_mag<BF16>(mx);
  const float r = s > 0.0f ? 127.0f / s : 0.0f;   // IEEE division; an all-zero row codes to 0
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = part * 512 + lane + 64 * i;
    if (c < nch) qr[c] = encode8<BF16>(v[i], r);
  }
  if (part == 0 && lane == 0) sx[row] = s;
}

template <bool BF16, int W, bool ACT, int PROD>
__global__ __launch_bounds__(256) void k_int8_rows(const uint16_t* __restrict__ X, int64_t rows, int K,
                                                   uint32_t tbits, int8_t* __restrict__ q, float* __restrict__ sx,
                                                   uint32_t* __restrict__ flags, uint32_t stamp, ProdArgs pa) {
  __shared__ uint32_t red[4];
  __shared__ double red64[4];
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (4 / W);
  uint4 v[8];
  rows_load<W>(X, rows, K, row0, v);
  rows_process<BF16, W, 4, ACT, PROD>(v, rows, K, tbits, q, sx, flags, stamp, pa, row0, red, red64, nullptr);
}

// The GELU-fused row pass: X = gelu(H) from the format's table, copied once
// into LDS by each block (128 KB, so one block of 8 waves per CU); the blocks
// then walk the row groups grid-stride, each wave loading its share of the
// next group before it works on the current one, so two groups' loads are in
// flight per CU (one group alone leaves the pass latency-bound).
constexpr int kGeluWaves = 8;

template <bool BF16, int W>
__global__ __launch_bounds__(64 * kGeluWaves) void k_int8_rows_gelu(const uint16_t* __restrict__ X, int64_t rows,
                                                                    int K, uint32_t tbits, int8_t* __restrict__ q,
                                                                    float* __restrict__ sx,
                                                                    uint32_t* __restrict__ flags, uint32_t stamp) {
  __shared__ __attribute__((aligned(16))) uint16_t gtab[65536];
  __shared__ uint32_t red[kGeluWaves];
  __shared__ double red64[kGeluWaves];
  constexpr int kRows = kGeluWaves / W;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kRows;
  const ProdArgs none{nullptr, nullptr, nullptr, 0.0f, nullptr};
  uint4 v[8], vn[8];
  int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  rows_load<W>(X, rows, K, row0, v);              // in flight while the table is copied
  gelu_table_to_lds<BF16>(gtab);
  __syncthreads();
  for (; row0 < rows; row0 += stride) {
    rows_load<W>(X, rows, K, row0 + stride, vn);  // the next group (nothing past the last row)
    rows_process<BF16, W, kGeluWaves, true, kProdGelu>(v, rows, K, tbits, q, sx, flags, stamp, none, row0, red, red64,
                                                       gtab);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = vn[i];
  }
}

// Row pass, streaming form for K > 16384: one block per row, two passes.
template <bool BF16, bool ACT>
__global__ __launch_bounds__(256) void k_int8_rows_long(const uint16_t* __restrict__ X, int K, uint32_t tbits,
                                                        int8_t* __restrict__ q, float* __restrict__ sx,
                                                        uint32_t* __restrict__ flags, uint32_t stamp) {
  __shared__ uint32_t red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const uint32_t t2 = tbits | (tbits << 16);
  const uint4* xr = reinterpret_cast<const uint4*>(X + row * K);
  uint32_t mx = 0;
#pragma unroll 4
  for (int c = threadIdx.x; c < nch; c += 256) mx = pk_max_u16(mx, chunk_scan<ACT>(xr[c], t2, flags, c, stamp));
  mx = wave_max_u32(max(mx & 0xFFFFu, mx >> 16));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = decode_mag<BF16>(mx);
  const float r = s > 0.0f ? 127.0f / s : 0.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
#pragma unroll 4
  for (int c = threadIdx.x; c < nch; c += 256) qr[c] = encode8<BF16>(xr[c], r);
  if (threadIdx.x == 0) sx[row] = s;
}

// --------------------------------------------------------------------------
// Block roles: blocks [0, xblocks) take kFixRows rows of X each; the rest take
// kFixWRows rows of Wq each (only when WO != nullptr). X blocks are small so
// that the rare rows to re-encode (a full pass over the row each, about 12 us
// on one CU with a GELU producer at K = 16384) seldom share a block. Every block rebuilds the
// ascending outlier list from the flags (a bit mask and its popcount prefix in
// LDS), then spreads (row, outlier slot) pairs over all threads, so the
// scattered loads of a block are all in flight together. Dynamic LDS: mask
// words, their exclusive popcount prefix, and the outlier list (up to kOcap
// entries; a larger set takes the per-row loops). A column is an outlier
// column when its flag word holds this call's stamp. XO and WO are written
// only when the padded outlier count fits their kOutCap columns; beyond that
// the GEMM gathers the outlier columns itself.
constexpr int kFixRows = 16;
constexpr int kFixWRows = 64;
constexpr int kOcap = 4096;
constexpr int kGatherUnroll = 8;

size_t outlier_fixup_lds_bytes(int K) {
  return static_cast<size_t>(2) * ((K + 31) / 32) * 4 + static_cast<size_t>(kOcap) * 4;
}

//
// With a producer, X is never stored: the gathers read H and make X values from
// it (with the row's rstd from the row pass), and re-encoded rows are made
// from H again.
template <bool BF16, int PROD>
__global__ __launch_bounds__(256) void k_outlier_fixup(
    const uint16_t* __restrict__ X, int M, int K, uint32_t tbits, const uint32_t* __restrict__ colflag,
    uint32_t stamp, int8_t* __restrict__ q, float* __restrict__ sx, int* __restrict__ O, int* __restrict__ nO_out,
    uint16_t* __restrict__ XO, const int8_t* __restrict__ Wq, int N, uint16_t* __restrict__ WO, int xblocks,
    ProdArgs pa) {
  extern __shared__ uint32_t smem[];
  __shared__ int scan_tot[4];
  __shared__ float fred[4];
  __shared__ uint32_t somax[kFixRows];       // per row: largest gathered magnitude <= t
  __shared__ float ssx[kFixRows];            // per row: provisional scale
  __shared__ float srstd[kFixRows];          // per row: RMSNorm rstd (producer kProdRms)
  __shared__ uint64_t sredo[1];              // rows to re-encode (bit r: row r of the block)
  const int nwords = (K + 31) >> 5;
  uint32_t* smask = smem;
  int* spre = reinterpret_cast<int*>(smem + nwords);
  int* sO = reinterpret_cast<int*>(smem + 2 * nwords);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // column flags -> bit mask in LDS, exclusive prefix of popcounts
  // (block scan in 256-word tiles)
  int carry = 0;
  for (int base = 0; base < nwords; base += 256) {
    const int w = base + tid;
    uint32_t bits = 0u;
    if (w < nwords) {
      if (32 * w + 32 <= K) {
        const uint4* fp = reinterpret_cast<const uint4*>(colflag + 32 * w);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 a = fp[i];
          bits |= (a.x == stamp ? 1u : 0u) << (4 * i);
          bits |= (a.y == stamp ? 1u : 0u) << (4 * i + 1);
          bits |= (a.z == stamp ? 1u : 0u) << (4 * i + 2);
          bits |= (a.w == stamp ? 1u : 0u) << (4 * i + 3);
        }
      } else {
        for (int j = 0; 32 * w + j < K; ++j) bits |= (colflag[32 * w + j] == stamp ? 1u : 0u) << j;
      }
      smask[w] = bits;
    }
    const int v = __popc(bits);
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) scan_tot[wave] = incl;
    __syncthreads();
    int wpre = 0;
    for (int i = 0; i < wave; ++i) wpre += scan_tot[i];
    if (w < nwords) spre[w] = carry + wpre + incl - v;
    carry += scan_tot[0] + scan_tot[1] + scan_tot[2] + scan_tot[3];
    __syncthreads();
  }
  const int nO = carry;
  const int P = (nO + 31) & ~31;
  const bool listed = nO <= kOcap;
  if (P > kOutCap) XO = nullptr, WO = nullptr;    // the GEMM gathers the outlier columns itself
  const uint16_t* gelu = gelu_table_global<BF16>();

  // ascending outlier list: in LDS for this block, in global memory from block 0
  for (int w = tid; w < nwords; w += 256) {
    uint32_t bits = smask[w];
    int j = spre[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (listed) sO[j] = 32 * w + b;
      if (blockIdx.x == 0 && O) O[j] = 32 * w + b;
      ++j;
    }
  }
  if (blockIdx.x == 0 && tid == 0) *nO_out = nO;
  if (nO == 0) return;
  if (tid < kFixRows) somax[tid] = 0u;
  const bool xblock = static_cast<int>(blockIdx.x) < xblocks;
  if (xblock && tid < kFixRows && static_cast<int>(blockIdx.x) * kFixRows + tid < M) {
    ssx[tid] = sx[blockIdx.x * kFixRows + tid];
    if constexpr (PROD == kProdRms) srstd[tid] = pa.rstd[blockIdx.x * kFixRows + tid];
  }
  __syncthreads();

  if (xblock) {
    const int r0 = blockIdx.x * kFixRows;
    const int rows = min(kFixRows, M - r0);
    // zero the codes of the outlier columns, gather X's outlier columns, and
    // note per row the largest gathered magnitude <= t
    auto take = [&](int r, int64_t m, int k) -> uint16_t {
      const uint16_t v = static_cast<uint16_t>(produce1<BF16, PROD>(X[m * K + k], k,
                                                                   PROD == kProdRms ? srstd[r] : 0.0f, pa, gelu));
      q[m * K + k] = 0;
      const uint32_t mag = v & 0x7FFFu;
      if (mag <= tbits) atomicMax(&somax[r], mag);
      return v;
    };
    if (listed) {
      // 8 entries per thread per round: all 8 loads go out before any store
      // (loads of padding entries read X[0] and are discarded), so a round
      // costs one memory latency, not eight
      const int total = rows * P;
      for (int base = 0; base < total; base += 256 * kGatherUnroll) {
        uint16_t v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
          const int idx = base + tid + 256 * u;
          const int r = idx / P, j = idx - r * P;
          const bool live = idx < total && j < nO;
          v[u] = X[live ? static_cast<int64_t>(r0 + r) * K + sO[j] : 0];
        }
        // the producer's values first, then the stores: with GELU every value
        // is a table load, and stores in between would hold each load back
        // until the stores before it (the compiler cannot tell the table from
        // the outputs)
        uint16_t pv[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
          const int idx = base + tid + 256 * u;
          const int r = idx / P, j = idx - r * P;
          pv[u] = idx < total && j < nO
                      ? static_cast<uint16_t>(
                            produce1<BF16, PROD>(v[u], sO[j], PROD == kProdRms ? srstd[r] : 0.0f, pa, gelu))
                      : uint16_t{0};
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
          const int idx = base + tid + 256 * u;
          if (idx >= total) break;
          const int r = idx / P, j = idx - r * P;
          const int64_t m = r0 + r;
          const uint16_t val = pv[u];
          if (j < nO) {
            q[m * K + sO[j]] = 0;
            const uint32_t mag = val & 0x7FFFu;
            if (mag <= tbits) atomicMax(&somax[r], mag);
          }
          if (XO) XO[m * P + j] = val;
        }
      }
    } else {
      for (int r = 0; r < rows; ++r) {
        const int64_t m = r0 + r;
        for (int w = tid; w < nwords; w += 256) {
          uint32_t bits = smask[w];
          int j = spre[w];
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            const uint16_t v = take(r, m, 32 * w + b);
            if (XO) XO[m * P + j] = v;
            ++j;
          }
        }
        if (XO)
          for (int j = nO + tid; j < P; j += 256) XO[m * P + j] = 0;
      }
    }
    __syncthreads();
    // A row whose provisional scale is also reached in an outlier column may
    // have a smaller true scale: recompute it over the non-outlier columns
    // and re-encode the whole row. The rows are tested all at once (one lane
    // per row, one wave's ballot); the loop visits only the rows found,
    // instead of paying two dependent LDS reads for every row.
    static_assert(kFixRows <= 64, "one ballot bit per row");
    if (wave == 0) {
      bool redo = false;
      if (lane < rows) {
        const float sp = ssx[lane];
        redo = sp > 0.0f && somax[lane] == mag_bits<BF16>(sp);
      }
      const uint64_t m = __ballot(redo);
      if (lane == 0) sredo[0] = m;
    }
    __syncthreads();
    for (uint64_t todo = sredo[0]; todo != 0; todo &= todo - 1) {
      const int r = __builtin_ctzll(todo);       // block-uniform
      const int64_t rowoff = static_cast<int64_t>(r0 + r) * K;
      const uint4* xr = reinterpret_cast<const uint4*>(X + rowoff);
      uint2* qr = reinterpret_cast<uint2*>(q + rowoff);
      const int nch = K >> 3;
      const float rr_std = PROD == kProdRms ? srstd[r] : 0.0f;
      float best = 0.0f;
      // the 8 codes of chunk c (outlier columns 0) with reciprocal scale rr
      auto code8 = [&](const float (&f)[8], int c, float rr) {
        const uint32_t ob = (smask[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int code = ((ob >> j) & 1u) ? 0 : absmax_code(f[j], rr);
          const uint32_t bb = static_cast<uint32_t>(code) & 0xFFu;
          if (j < 4) lo |= bb << (8 * j);
          else hi |= bb << (8 * (j - 4));
        }
        qr[c] = make_uint2(lo, hi);
      };
      auto chunk_best = [&](const float (&f)[8], int c) {
        const uint32_t ob = (smask[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!((ob >> j) & 1u)) best = fmaxf(best, fabsf(f[j]));
      };
      if constexpr (PROD != kProdNone) {
        // K <= 16384 with a producer: the row's X is made once and held in
        // registers (8 chunks per thread) for both passes. All 8 chunks of H
        // are loaded first, then all their producer values made (with GELU,
        // 64 independent table loads): one memory latency for each step
        // rather than two per chunk.
        uint4 xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + 256 * i;
          xv[i] = c < nch ? xr[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + 256 * i;
          if (c < nch) xv[i] = produce8<BF16, PROD>(xv[i], c, rr_std, pa, gelu);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + 256 * i;
          if (c < nch) {
            float f[8];
            unpack8<BF16>(xv[i], f);
            chunk_best(f, c);
          }
        }
        best = block_max256(best, fred);
        const float rr = 127.0f / best;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = tid + 256 * i;
          if (c < nch) {
            float f[8];
            unpack8<BF16>(xv[i], f);
            code8(f, c, rr);
          }
        }
      } else {
#pragma unroll 8
        for (int c = tid; c < nch; c += 256) {
          float f[8];
          unpack8<BF16>(xr[c], f);
          chunk_best(f, c);
        }
        best = block_max256(best, fred);
        const float rr = 127.0f / best;
#pragma unroll 8
        for (int c = tid; c < nch; c += 256) {
          float f[8];
          unpack8<BF16>(xr[c], f);
          code8(f, c, rr);
        }
      }
      if (tid == 0) sx[r0 + r] = best;
    }
  } else if (WO) {
    const int r0 = (blockIdx.x - xblocks) * kFixWRows;
    const int rows = min(kFixWRows, N - r0);
    auto cvt = [](int8_t v) -> uint16_t {
      const float f = static_cast<float>(v);  // |v| <= 127: exact in both 16-bit types
      return BF16 ? static_cast<uint16_t>(__float_as_uint(f) >> 16) : f32_to_f16_bits(f);
    };
    if (listed) {
      // as for XO: the round's loads go out together (padding reads Wq[0])
      const int total = rows * P;
      for (int base = 0; base < total; base += 256 * kGatherUnroll) {
        int8_t v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
          const int idx = base + tid + 256 * u;
          const int r = idx / P, j = idx - r * P;
          const bool live = idx < total && j < nO;
          v[u] = Wq[live ? static_cast<int64_t>(r0 + r) * K + sO[j] : 0];
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
          const int idx = base + tid + 256 * u;
          if (idx >= total) break;
          const int r = idx / P, j = idx - r * P;
          WO[static_cast<int64_t>(r0 + r) * P + j] = j < nO ? cvt(v[u]) : uint16_t(0);
        }
      }
    } else {
      for (int r = 0; r < rows; ++r) {
        const int64_t n = r0 + r;
        for (int w = tid; w < nwords; w += 256) {
          uint32_t bits = smask[w];
          int j = spre[w];
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            WO[n * P + j++] = cvt(Wq[n * K + 32 * w + b]);
          }
        }
        for (int j = nO + tid; j < P; j += 256) WO[n * P + j] = 0;
      }
    }
  }
}

// --------------------------------------------------------------------------
// FP8 rows. MODE 0: dynamic activation scale fl32(amax/448); MODE 1: static
// scale *act_scale; MODE 2: weight scale bf16(fl32(amax/448)).
template <bool BF16, int CPT, int MODE>
__global__ __launch_bounds__(256) void k_fp8_rows(const uint16_t* __restrict__ X, int K,
                                                  const float* __restrict__ act_scale,
                                                  uint8_t* __restrict__ xq, float* __restrict__ sx) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(X + row * K);
  uint2* qr = reinterpret_cast<uint2*>(xq + row * K);
  const int tid = threadIdx.x;

  auto code_chunk = [&](const uint4& v, int c, float s) {
    float f[8];
    unpack8<BF16>(v, f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = (s == 0.0f) ? 0u : e4m3_code(f[j] / s);  // IEEE division
      if (j < 4) lo |= b << (8 * j);
      else hi |= b << (8 * (j - 4));
    }
    qr[c] = make_uint2(lo, hi);
  };
  auto chunk_absmax = [&](const uint4& v) {
    float f[8];
    unpack8<BF16>(v, f);
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
    return a;
  };
  auto finish_scale = [&](float amax) {
    if constexpr (MODE == 1) {
      return *act_scale;
    } else {
      const float s = amax / 448.0f;
      if constexpr (MODE == 2) return __uint_as_float(bf16_rne_bits(s) << 16);
      return s;
    }
  };

  if constexpr (CPT > 0) {
    uint4 v[CPT];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) v[i] = xr[c];
    }
    if constexpr (MODE != 1) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = tid + 256 * i;
        if (c < nch) amax = fmaxf(amax, chunk_absmax(v[i]));
      }
      amax = block_max256(amax, red);
    }
    const float s = finish_scale(amax);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) code_chunk(v[i], c, s);
    }
    if (tid == 0) sx[row] = s;
  } else {
    float amax = 0.0f;
    if constexpr (MODE != 1) {
      for (int c = tid; c < nch; c += 256) amax = fmaxf(amax, chunk_absmax(xr[c]));
      amax = block_max256(amax, red);
    }
    const float s = finish_scale(amax);
    for (int c = tid; c < nch; c += 256) code_chunk(xr[c], c, s);
    if (tid == 0) sx[row] = s;
  }
}

// --------------------------------------------------------------------------
// Host-side launchers (called by the ABI layer after validation).

template <bool BF16, bool ACT, int PROD>
static void launch_int8_rows_t(const uint16_t* X, int64_t rows, int K, uint32_t tbits, int8_t* q, float* sx,
                               uint32_t* flags, uint32_t stamp, const ProdArgs& pa, hipStream_t s) {
  const dim3 block(256);
  auto blocks = [&](int rpb) { return dim3(static_cast<unsigned>((rows + rpb - 1) / rpb)); };
  if constexpr (PROD == kProdGelu) {
    // one block per CU at most (the 128 KB table fills the LDS)
    const int W = K <= 4096 ? 1 : (K <= 8192 ? 2 : 4);
    const int64_t groups = (rows + kGeluWaves / W - 1) / (kGeluWaves / W);
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(groups, std::max(device_cus(), 1))));
    const dim3 gblock(64 * kGeluWaves);
    if (W == 1) k_int8_rows_gelu<BF16, 1><<<grid, gblock, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp);
    else if (W == 2) k_int8_rows_gelu<BF16, 2><<<grid, gblock, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp);
    else k_int8_rows_gelu<BF16, 4><<<grid, gblock, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp);
  } else if (K <= 4096) {
    k_int8_rows<BF16, 1, ACT, PROD><<<blocks(4), block, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp, pa);
  } else if (K <= 8192) {
    k_int8_rows<BF16, 2, ACT, PROD><<<blocks(2), block, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp, pa);
  } else if (K <= 16384) {
    k_int8_rows<BF16, 4, ACT, PROD><<<blocks(1), block, 0, s>>>(X, rows, K, tbits, q, sx, flags, stamp, pa);
  } else if constexpr (PROD == kProdNone) {
    k_int8_rows_long<BF16, ACT><<<dim3(static_cast<unsigned>(rows)), block, 0, s>>>(X, K, tbits, q, sx, flags,
                                                                                    stamp);
  }
}

template <bool BF16>
static void launch_int8_rows_b(const uint16_t* X, int64_t rows, int K, uint32_t tbits, int8_t* q, float* sx,
                               uint32_t* flags, uint32_t stamp, int prod, const ProdArgs& pa, hipStream_t s) {
  if (!flags) launch_int8_rows_t<BF16, false, kProdNone>(X, rows, K, tbits, q, sx, flags, stamp, pa, s);
  else if (prod == kProdRms) launch_int8_rows_t<BF16, true, kProdRms>(X, rows, K, tbits, q, sx, flags, stamp, pa, s);
  else if (prod == kProdGelu) launch_int8_rows_t<BF16, true, kProdGelu>(X, rows, K, tbits, q, sx, flags, stamp, pa, s);
  else launch_int8_rows_t<BF16, true, kProdNone>(X, rows, K, tbits, q, sx, flags, stamp, pa, s);
}

// flags == nullptr: weight pass (no threshold, no producer). A producer needs
// K <= 16384 (checked by the caller).
void launch_int8_rows(const void* X, bool bf16, int64_t rows, int K, uint32_t tbits, int8_t* q, float* sx,
                      uint32_t* flags, uint32_t stamp, int prod, const ProdArgs& pa, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (bf16) launch_int8_rows_b<true>(x, rows, K, tbits, q, sx, flags, stamp, prod, pa, s);
  else launch_int8_rows_b<false>(x, rows, K, tbits, q, sx, flags, stamp, prod, pa, s);
}

// X = producer(H) written out (the parity export, and the GELU before the
// 16-bit down-projection of the block driver). RMSNorm: one block per row.
template <bool BF16, int PROD>
__global__ __launch_bounds__(256) void k_produce(const uint16_t* __restrict__ H, int K, ProdArgs pa,
                                                 uint16_t* __restrict__ X) {
  __shared__ double red64[4];
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const uint4* hr = reinterpret_cast<const uint4*>(H + row * K);
  uint4* xr = reinterpret_cast<uint4*>(X + row * K);
  float rstd = 0.0f;
  if constexpr (PROD == kProdRms) {
    double ss = 0.0;
    for (int c = threadIdx.x; c < nch; c += 256) ss += sumsq8<BF16>(hr[c]);
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0) red64[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = ((red64[0] + red64[1]) + red64[2]) + red64[3];
    rstd = rms_rstd(ss, K, pa.eps);
  }
  for (int c = threadIdx.x; c < nch; c += 256) xr[c] = produce8<BF16, PROD>(hr[c], c, rstd, pa, nullptr);
}

// GELU is elementwise: each block copies the table into LDS and then maps
// 16-byte chunks of the whole array, grid-stride, four chunks in flight per
// thread.
template <bool BF16>
__global__ __launch_bounds__(512) void k_produce_gelu(const uint16_t* __restrict__ H, int64_t nchunks,
                                                      uint16_t* __restrict__ X) {
  __shared__ __attribute__((aligned(16))) uint16_t gtab[65536];
  gelu_table_to_lds<BF16>(gtab);
  __syncthreads();
  const uint4* h = reinterpret_cast<const uint4*>(H);
  uint4* x = reinterpret_cast<uint4*>(X);
  const ProdArgs none{nullptr, nullptr, nullptr, 0.0f, nullptr};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; c + 3 * stride < nchunks; c += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = h[c + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[c + u * stride] = produce8<BF16, kProdGelu>(v[u], 0, 0.0f, none, gtab);
  }
  for (; c < nchunks; c += stride) x[c] = produce8<BF16, kProdGelu>(h[c], 0, 0.0f, none, gtab);
}

void launch_produce(const void* H, bool bf16, int64_t M, int K, int prod, const ProdArgs& pa, void* X,
                    hipStream_t s) {
  const uint16_t* h = static_cast<const uint16_t*>(H);
  uint16_t* x = static_cast<uint16_t*>(X);
  if (prod == kProdGelu) {
    const int64_t nchunks = M * K / 8;
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>((nchunks + 511) / 512, std::max(device_cus(), 1))));
    if (bf16) k_produce_gelu<true><<<grid, dim3(512), 0, s>>>(h, nchunks, x);
    else k_produce_gelu<false><<<grid, dim3(512), 0, s>>>(h, nchunks, x);
    return;
  }
  const dim3 grid(static_cast<unsigned>(M)), block(256);
  if (bf16) {
    if (prod == kProdRms) k_produce<true, kProdRms><<<grid, block, 0, s>>>(h, K, pa, x);
    else k_produce<true, kProdNone><<<grid, block, 0, s>>>(h, K, pa, x);
  } else {
    if (prod == kProdRms) k_produce<false, kProdRms><<<grid, block, 0, s>>>(h, K, pa, x);
    else k_produce<false, kProdNone><<<grid, block, 0, s>>>(h, K, pa, x);
  }
}

template <bool BF16, int PROD>
static void launch_fixup_t(const uint16_t* X, int64_t M, int K, uint32_t tbits, const uint32_t* colflag,
                           uint32_t stamp, int8_t* q,
                           float* sx, int* O, int* nO, uint16_t* XO, const int8_t* Wq, int64_t N, uint16_t* WO,
                           const ProdArgs& pa, hipStream_t s) {
  const int xblocks = static_cast<int>((M + kFixRows - 1) / kFixRows);
  const int wblocks = WO ? static_cast<int>((N + kFixWRows - 1) / kFixWRows) : 0;
  const size_t lds = outlier_fixup_lds_bytes(K);
  const dim3 grid(xblocks + wblocks), block(256);
  k_outlier_fixup<BF16, PROD><<<grid, block, lds, s>>>(X, (int)M, K, tbits, colflag, stamp, q, sx, O, nO, XO, Wq,
                                                       (int)N, WO, xblocks, pa);
}

void launch_outlier_fixup(const void* X, bool bf16, int64_t M, int K, uint32_t tbits, const uint32_t* colflag,
                          uint32_t stamp, int8_t* q, float* sx, int* O, int* nO, uint16_t* XO, const int8_t* Wq, int64_t N,
                          uint16_t* WO, int prod, const ProdArgs& pa, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
#define W8_FIX_ARGS x, M, K, tbits, colflag, stamp, q, sx, O, nO, XO, Wq, N, WO, pa, s
  if (bf16) {
    if (prod == kProdRms) launch_fixup_t<true, kProdRms>(W8_FIX_ARGS);
    else if (prod == kProdGelu) launch_fixup_t<true, kProdGelu>(W8_FIX_ARGS);
    else launch_fixup_t<true, kProdNone>(W8_FIX_ARGS);
  } else {
    if (prod == kProdRms) launch_fixup_t<false, kProdRms>(W8_FIX_ARGS);
    else if (prod == kProdGelu) launch_fixup_t<false, kProdGelu>(W8_FIX_ARGS);
    else launch_fixup_t<false, kProdNone>(W8_FIX_ARGS);
  }
#undef W8_FIX_ARGS
}

template <bool BF16, int MODE>
static void launch_fp8_rows_t(const uint16_t* X, int64_t rows, int K, const float* act_scale, uint8_t* xq,
                              float* sx, hipStream_t s) {
  const int nch = K >> 3;
  const dim3 grid(static_cast<unsigned>(rows)), block(256);
  if (nch <= 256)
    k_fp8_rows<BF16, 1, MODE><<<grid, block, 0, s>>>(X, K, act_scale, xq, sx);
  else if (nch <= 512)
    k_fp8_rows<BF16, 2, MODE><<<grid, block, 0, s>>>(X, K, act_scale, xq, sx);
  else if (nch <= 1024)
    k_fp8_rows<BF16, 4, MODE><<<grid, block, 0, s>>>(X, K, act_scale, xq, sx);
  else if (nch <= 2048)
    k_fp8_rows<BF16, 8, MODE><<<grid, block, 0, s>>>(X, K, act_scale, xq, sx);
  else
    k_fp8_rows<BF16, 0, MODE><<<grid, block, 0, s>>>(X, K, act_scale, xq, sx);
}

// mode: 0 dynamic activation, 1 static activation, 2 weight
void launch_fp8_rows(const void* X, bool bf16, int64_t rows, int K, const float* act_scale, uint8_t* xq,
                     float* sx, int mode, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (bf16) {
    if (mode == 0) launch_fp8_rows_t<true, 0>(x, rows, K, act_scale, xq, sx, s);
    else if (mode == 1) launch_fp8_rows_t<true, 1>(x, rows, K, act_scale, xq, sx, s);
    else launch_fp8_rows_t<true, 2>(x, rows, K, act_scale, xq, sx, s);
  } else {
    if (mode == 0) launch_fp8_rows_t<false, 0>(x, rows, K, act_scale, xq, sx, s);
    else if (mode == 1) launch_fp8_rows_t<false, 1>(x, rows, K, act_scale, xq, sx, s);
    else launch_fp8_rows_t<false, 2>(x, rows, K, act_scale, xq, sx, s);
  }
}

}  // namespace w8
