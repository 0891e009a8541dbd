// Row quantisation kernels of libw8mp (gfx950).
//
//  k_clear            zero the outlier-column flags
//  k_int8_rows        one pass over a row: absmax over the elements with
//                     |x| <= t and its column, outlier-column flags (|x| > t),
//                     int8 codes with that provisional scale. With t = +inf it
//                     is the rowwise weight quantiser.
//  k_outlier_fixup    outlier list, zero codes in outlier columns, gather the
//                     outlier columns of X and Wq for the 16-bit side product,
//                     and redo the rare rows whose provisional absmax sat in an
//                     outlier column.
//  k_fp8_rows         per-row (or static) scale and E4M3 codes.
//
// The LLM.int8 decomposition ("Image21-INT8" card, section "Quantization":
// threshold 6.0, outliers in floating point): a row's scale must ignore every
// column that is an outlier column in ANY row of the call. One pass cannot know
// that set, so k_int8_rows takes the max over |x| <= t. That equals the true
// scale unless the max sat in a column another row made an outlier;
// k_outlier_fixup detects exactly those rows through the recorded column and
// re-encodes them once the whole set is known.
#include "common.h"

namespace w8 {

// --------------------------------------------------------------------------
__global__ void k_clear(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// --------------------------------------------------------------------------
// Row pass, register-resident form: W waves per row (W = 1, 2, 4), each wave
// covering a 4096-element slice, 8 chunks of 8 elements per lane; a block of
// 256 threads therefore holds 4/W rows. With W == 1 the row reduction stays
// inside one wave (no LDS, no barrier).
//
// Outlier columns are flagged with a plain byte store of 1 into colflag[k]
// (cleared before the pass): many rows flag the same few columns, and equal
// plain stores need no read-modify-write.
template <bool BF16, int W, bool WEIGHT>
__global__ __launch_bounds__(256) void k_int8_rows(const uint16_t* __restrict__ X, int64_t rows, int K, float t,
                                                   int8_t* __restrict__ q, float* __restrict__ sx,
                                                   int* __restrict__ amax_col, uint8_t* __restrict__ colflag) {
  constexpr int kRows = 4 / W;
  __shared__ MaxLoc red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRows + wave / W;
  const bool valid = row < rows;
  const int part = wave % W;
  const int nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(X + (valid ? row : 0) * K);
  uint2* qr = reinterpret_cast<uint2*>(q + (valid ? row : 0) * K);

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = part * 512 + lane + 64 * i;
    if (valid && c < nch) v[i] = xr[c];
  }
  MaxLoc best{0.0f, -1};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = part * 512 + lane + 64 * i;
    if (!(valid && c < nch)) continue;
    float f[8];
    unpack8<BF16>(v[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(f[j]);
      if (a > t) {
        if (!WEIGHT) colflag[8 * c + j] = 1;
      } else if (a > best.v) {
        best.v = a;
        best.k = 8 * c + j;
      }
    }
  }
  best = wave_maxloc(best);
  if constexpr (W > 1) {
    if (lane == 0) red[wave] = best;
    __syncthreads();
    const int w0 = (wave / W) * W;
    best = red[w0];
#pragma unroll
    for (int w = 1; w < W; ++w) best = maxloc_pick(best, red[w0 + w]);
  }
  const float r = 127.0f / best.v;  // IEEE division; +inf for an all-zero row
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = part * 512 + lane + 64 * i;
    if (!(valid && c < nch)) continue;
    float f[8];
    unpack8<BF16>(v[i], f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int code = (fabsf(f[j]) > t) ? 0 : absmax_code(f[j], r);
      const uint32_t b = static_cast<uint32_t>(code) & 0xFFu;
      if (j < 4) lo |= b << (8 * j);
      else hi |= b << (8 * (j - 4));
    }
    qr[c] = make_uint2(lo, hi);
  }
  if (valid && part == 0 && lane == 0) {
    sx[row] = best.v;
    if (!WEIGHT) amax_col[row] = best.k;
  }
}

// Row pass, streaming form for K > 16384: one block per row, two passes.
template <bool BF16, bool WEIGHT>
__global__ __launch_bounds__(256) void k_int8_rows_long(const uint16_t* __restrict__ X, int K, float t,
                                                        int8_t* __restrict__ q, float* __restrict__ sx,
                                                        int* __restrict__ amax_col, uint8_t* __restrict__ colflag) {
  __shared__ MaxLoc red[4];
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(X + row * K);
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
  MaxLoc best{0.0f, -1};
#pragma unroll 4
  for (int c = threadIdx.x; c < nch; c += 256) {
    float f[8];
    unpack8<BF16>(xr[c], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(f[j]);
      if (a > t) {
        if (!WEIGHT) colflag[8 * c + j] = 1;
      } else if (a > best.v) {
        best.v = a;
        best.k = 8 * c + j;
      }
    }
  }
  const MaxLoc b = block_maxloc256(best, red);
  const float r = 127.0f / b.v;
#pragma unroll 4
  for (int c = threadIdx.x; c < nch; c += 256) {
    float f[8];
    unpack8<BF16>(xr[c], f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int code = (fabsf(f[j]) > t) ? 0 : absmax_code(f[j], r);
      const uint32_t bb = static_cast<uint32_t>(code) & 0xFFu;
      if (j < 4) lo |= bb << (8 * j);
      else hi |= bb << (8 * (j - 4));
    }
    qr[c] = make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) {
    sx[row] = b.v;
    if (!WEIGHT) amax_col[row] = b.k;
  }
}

// --------------------------------------------------------------------------
// Block roles: blocks [0, xblocks) take kFixRows rows of X each; the rest take
// kFixRows rows of Wq each (only when WO != nullptr). Every block rebuilds the
// ascending outlier list from the mask in LDS (prefix of popcounts), then
// spreads (row, outlier slot) pairs over all threads, so the scattered loads
// of a block are all in flight together. Dynamic LDS: mask words, their
// exclusive popcount prefix, and the outlier list (up to kOcap entries; a
// larger set takes the per-row loop at the end).
constexpr int kFixRows = 64;
constexpr int kOcap = 4096;

size_t outlier_fixup_lds_bytes(int K) {
  return static_cast<size_t>(2) * ((K + 31) / 32) * 4 + static_cast<size_t>(kOcap) * 4;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_outlier_fixup(
    const uint16_t* __restrict__ X, int M, int K, const uint8_t* __restrict__ colflag,
    int8_t* __restrict__ q, float* __restrict__ sx, const int* __restrict__ amax_col,
    int* __restrict__ O, int* __restrict__ nO_out, uint16_t* __restrict__ XO,
    const int8_t* __restrict__ Wq, int N, uint16_t* __restrict__ WO, int xblocks) {
  extern __shared__ uint32_t smem[];
  __shared__ int scan_tot[4];
  __shared__ float fred[4];
  __shared__ int sredo[kFixRows];
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
      const uint4* fp = reinterpret_cast<const uint4*>(colflag + 32 * w);  // K % 32 == 0 region
      const int avail = min(32, K - 32 * w);
      if (avail == 32) {
        const uint4 a = fp[0], b = fp[1];
        const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) bits |= ((wd[i] >> (8 * j)) & 1u) << (4 * i + j);
      } else {
        for (int j = 0; j < avail; ++j) bits |= static_cast<uint32_t>(colflag[32 * w + j] & 1u) << j;
      }
    }
    if (w < nwords) smask[w] = bits;
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
  __syncthreads();

  if (static_cast<int>(blockIdx.x) < xblocks) {
    const int r0 = blockIdx.x * kFixRows;
    const int rows = min(kFixRows, M - r0);
    if (tid < rows) {
      const int c = amax_col[r0 + tid];
      sredo[tid] = (c >= 0) && ((smask[c >> 5] >> (c & 31)) & 1u);
    }
    if (listed) {
      // zero the codes of the outlier columns and gather X's outlier columns
#pragma unroll 8
      for (int idx = tid; idx < rows * P; idx += 256) {
        const int r = idx / P, j = idx - r * P;
        const int64_t m = r0 + r;
        uint16_t v = 0;
        if (j < nO) {
          const int k = sO[j];
          v = X[m * K + k];
          q[m * K + k] = 0;
        }
        if (XO) XO[m * P + j] = v;
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
            q[m * K + 32 * w + b] = 0;
            if (XO) XO[m * P + j] = X[m * K + 32 * w + b];
            ++j;
          }
        }
        if (XO)
          for (int j = nO + tid; j < P; j += 256) XO[m * P + j] = 0;
      }
    }
    __syncthreads();
    // Rows whose provisional absmax sat in an outlier column: recompute the
    // scale over the non-outlier columns and re-encode the whole row.
    for (int r = 0; r < rows; ++r) {
      if (!sredo[r]) continue;
      const int64_t rowoff = static_cast<int64_t>(r0 + r) * K;
      const uint4* xr = reinterpret_cast<const uint4*>(X + rowoff);
      uint2* qr = reinterpret_cast<uint2*>(q + rowoff);
      const int nch = K >> 3;
      float best = 0.0f;
#pragma unroll 8
      for (int c = tid; c < nch; c += 256) {
        float f[8];
        unpack8<BF16>(xr[c], f);
        const uint32_t ob = (smask[c >> 2] >> ((c & 3) * 8)) & 0xFFu;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!((ob >> j) & 1u)) best = fmaxf(best, fabsf(f[j]));
      }
      best = block_max256(best, fred);
      const float rr = 127.0f / best;
#pragma unroll 8
      for (int c = tid; c < nch; c += 256) {
        float f[8];
        unpack8<BF16>(xr[c], f);
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
      }
      if (tid == 0) sx[r0 + r] = best;
    }
  } else if (WO) {
    const int r0 = (blockIdx.x - xblocks) * kFixRows;
    const int rows = min(kFixRows, N - r0);
    auto cvt = [](int8_t v) -> uint16_t {
      const float f = static_cast<float>(v);  // |v| <= 127: exact in both 16-bit types
      return BF16 ? static_cast<uint16_t>(__float_as_uint(f) >> 16) : f32_to_f16_bits(f);
    };
    if (listed) {
#pragma unroll 8
      for (int idx = tid; idx < rows * P; idx += 256) {
        const int r = idx / P, j = idx - r * P;
        const int64_t n = r0 + r;
        WO[n * P + j] = (j < nO) ? cvt(Wq[n * K + sO[j]]) : uint16_t(0);
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

template <bool BF16, bool WEIGHT>
static void launch_int8_rows_t(const uint16_t* X, int64_t rows, int K, float t, int8_t* q, float* sx,
                               int* amax_col, uint8_t* colflag, hipStream_t s) {
  const dim3 block(256);
  auto blocks = [&](int rpb) { return dim3(static_cast<unsigned>((rows + rpb - 1) / rpb)); };
  if (K <= 4096)
    k_int8_rows<BF16, 1, WEIGHT><<<blocks(4), block, 0, s>>>(X, rows, K, t, q, sx, amax_col, colflag);
  else if (K <= 8192)
    k_int8_rows<BF16, 2, WEIGHT><<<blocks(2), block, 0, s>>>(X, rows, K, t, q, sx, amax_col, colflag);
  else if (K <= 16384)
    k_int8_rows<BF16, 4, WEIGHT><<<blocks(1), block, 0, s>>>(X, rows, K, t, q, sx, amax_col, colflag);
  else
    k_int8_rows_long<BF16, WEIGHT><<<dim3(static_cast<unsigned>(rows)), block, 0, s>>>(X, K, t, q, sx, amax_col,
                                                                                       colflag);
}

void launch_clear(uint32_t* p, int n, hipStream_t s) {
  const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  k_clear<<<dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s>>>(p, n);
}

void launch_int8_rows(const void* X, bool bf16, int64_t rows, int K, float t, int8_t* q, float* sx,
                      int* amax_col, uint8_t* colflag, bool weight, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (bf16) {
    if (weight) launch_int8_rows_t<true, true>(x, rows, K, t, q, sx, amax_col, colflag, s);
    else launch_int8_rows_t<true, false>(x, rows, K, t, q, sx, amax_col, colflag, s);
  } else {
    if (weight) launch_int8_rows_t<false, true>(x, rows, K, t, q, sx, amax_col, colflag, s);
    else launch_int8_rows_t<false, false>(x, rows, K, t, q, sx, amax_col, colflag, s);
  }
}

void launch_outlier_fixup(const void* X, bool bf16, int64_t M, int K, const uint8_t* colflag, int8_t* q,
                          float* sx, const int* amax_col, int* O, int* nO, uint16_t* XO,
                          const int8_t* Wq, int64_t N, uint16_t* WO, hipStream_t s) {
  const int xblocks = static_cast<int>((M + kFixRows - 1) / kFixRows);
  const int wblocks = WO ? static_cast<int>((N + kFixRows - 1) / kFixRows) : 0;
  const size_t lds = outlier_fixup_lds_bytes(K);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const dim3 grid(xblocks + wblocks), block(256);
  if (bf16)
    k_outlier_fixup<true><<<grid, block, lds, s>>>(x, (int)M, K, colflag, q, sx, amax_col, O, nO, XO, Wq,
                                                   (int)N, WO, xblocks);
  else
    k_outlier_fixup<false><<<grid, block, lds, s>>>(x, (int)M, K, colflag, q, sx, amax_col, O, nO, XO, Wq,
                                                    (int)N, WO, xblocks);
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
