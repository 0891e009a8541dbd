// Row quantisation kernels of libw8mp (gfx950).
//
//  k_clear            zero the outlier-column bit mask (and the outlier count)
//  k_int8_rows        one pass over a row: absmax over the elements with
//                     |x| <= t and its column, outlier-column bits (|x| > t),
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
// One 256-thread block per row. A thread owns 16-byte chunks c = tid + 256*i.
// CPT > 0: the row stays in registers (K <= 2048*CPT); CPT == 0: two passes.
template <bool BF16, int CPT, bool WEIGHT>
__global__ __launch_bounds__(256) void k_int8_rows(const uint16_t* __restrict__ X, int K, float t,
                                                   int8_t* __restrict__ q, float* __restrict__ sx,
                                                   int* __restrict__ amax_col,
                                                   uint32_t* __restrict__ mask) {
  __shared__ MaxLoc red[4];
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(X + row * K);
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
  const int tid = threadIdx.x;

  MaxLoc best{0.0f, -1};
  auto scan_chunk = [&](const uint4& v, int c) {
    float f[8];
    unpack8<BF16>(v, f);
    uint32_t obits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(f[j]);
      if (a > t) {
        obits |= 1u << j;
      } else if (a > best.v) {
        best.v = a;
        best.k = 8 * c + j;
      }
    }
    if (!WEIGHT && obits) atomicOr(&mask[c >> 2], obits << ((c & 3) * 8));
  };
  auto code_chunk = [&](const uint4& v, int c, float r) {
    float f[8];
    unpack8<BF16>(v, f);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int code = (fabsf(f[j]) > t) ? 0 : absmax_code(f[j], r);
      const uint32_t b = static_cast<uint32_t>(code) & 0xFFu;
      if (j < 4) lo |= b << (8 * j);
      else hi |= b << (8 * (j - 4));
    }
    qr[c] = make_uint2(lo, hi);
  };

  if constexpr (CPT > 0) {
    uint4 v[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) v[i] = xr[c];
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) scan_chunk(v[i], c);
    }
    const MaxLoc b = block_maxloc256(best, red);
    const float r = 127.0f / b.v;  // IEEE division; +inf for an all-zero row
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < nch) code_chunk(v[i], c, r);
    }
    if (tid == 0) {
      sx[row] = b.v;
      if (!WEIGHT) amax_col[row] = b.k;
    }
  } else {
    for (int c = tid; c < nch; c += 256) scan_chunk(xr[c], c);
    const MaxLoc b = block_maxloc256(best, red);
    const float r = 127.0f / b.v;
    for (int c = tid; c < nch; c += 256) code_chunk(xr[c], c, r);
    if (tid == 0) {
      sx[row] = b.v;
      if (!WEIGHT) amax_col[row] = b.k;
    }
  }
}

// --------------------------------------------------------------------------
// Block roles: blocks [0, xblocks) take ROWS rows of X each; the rest take ROWS
// rows of Wq each (only when WO != nullptr). Dynamic LDS: mask words and their
// exclusive popcount prefix (2 * nwords ints).
constexpr int kFixRows = 16;

template <bool BF16>
__global__ __launch_bounds__(256) void k_outlier_fixup(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ mask,
    int8_t* __restrict__ q, float* __restrict__ sx, const int* __restrict__ amax_col,
    int* __restrict__ O, int* __restrict__ nO_out, uint16_t* __restrict__ XO,
    const int8_t* __restrict__ Wq, int N, uint16_t* __restrict__ WO, int xblocks) {
  extern __shared__ uint32_t smem[];
  __shared__ int scan_tot[4];
  __shared__ float fred[4];
  const int nwords = (K + 31) >> 5;
  uint32_t* smask = smem;
  int* spre = reinterpret_cast<int*>(smem + nwords);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // mask -> LDS, exclusive prefix of popcounts (block scan in 256-word tiles)
  int carry = 0;
  for (int base = 0; base < nwords; base += 256) {
    const int w = base + tid;
    const uint32_t bits = (w < nwords) ? mask[w] : 0u;
    if (w < nwords) smask[w] = bits;
    int v = __popc(bits);
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

  if (blockIdx.x == 0) {
    for (int w = tid; w < nwords; w += 256) {
      uint32_t bits = smask[w];
      int j = spre[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        if (O) O[j] = 32 * w + b;
        ++j;
      }
    }
    if (tid == 0) *nO_out = nO;
  }
  if (nO == 0) return;

  if (static_cast<int>(blockIdx.x) < xblocks) {
    const int r0 = blockIdx.x * kFixRows;
    for (int m = r0; m < min(r0 + kFixRows, M); ++m) {
      const int64_t rowoff = static_cast<int64_t>(m) * K;
      const int c = amax_col[m];
      const bool redo = (c >= 0) && ((smask[c >> 5] >> (c & 31)) & 1u);
      if (redo) {
        // The provisional absmax sat in an outlier column: recompute the
        // scale over the non-outlier columns and re-encode the whole row.
        float best = 0.0f;
        for (int k = tid; k < K; k += 256) {
          if (!((smask[k >> 5] >> (k & 31)) & 1u)) best = fmaxf(best, fabsf(to_f32<BF16>(X[rowoff + k])));
        }
        best = block_max256(best, fred);
        const float r = 127.0f / best;
        for (int k = tid; k < K; k += 256) {
          const bool out = (smask[k >> 5] >> (k & 31)) & 1u;
          q[rowoff + k] = out ? 0 : static_cast<int8_t>(absmax_code(to_f32<BF16>(X[rowoff + k]), r));
        }
        if (tid == 0) sx[m] = best;
      } else {
        for (int w = tid; w < nwords; w += 256) {
          uint32_t bits = smask[w];
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            q[rowoff + 32 * w + b] = 0;
          }
        }
      }
      if (XO) {
        uint16_t* xo = XO + static_cast<int64_t>(m) * P;
        for (int w = tid; w < nwords; w += 256) {
          uint32_t bits = smask[w];
          int j = spre[w];
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            xo[j++] = X[rowoff + 32 * w + b];
          }
        }
        for (int j = nO + tid; j < P; j += 256) xo[j] = 0;
      }
    }
  } else if (WO) {
    const int r0 = (blockIdx.x - xblocks) * kFixRows;
    for (int n = r0; n < min(r0 + kFixRows, N); ++n) {
      const int8_t* wr = Wq + static_cast<int64_t>(n) * K;
      uint16_t* wo = WO + static_cast<int64_t>(n) * P;
      for (int w = tid; w < nwords; w += 256) {
        uint32_t bits = smask[w];
        int j = spre[w];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          const float v = static_cast<float>(wr[32 * w + b]);  // |v| <= 127: exact in 16 bits
          wo[j++] = BF16 ? static_cast<uint16_t>(__float_as_uint(v) >> 16) : f32_to_f16_bits(v);
        }
      }
      for (int j = nO + tid; j < P; j += 256) wo[j] = 0;
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
                               int* amax_col, uint32_t* mask, hipStream_t s) {
  const int nch = K >> 3;
  const dim3 grid(static_cast<unsigned>(rows)), block(256);
  if (nch <= 256)
    k_int8_rows<BF16, 1, WEIGHT><<<grid, block, 0, s>>>(X, K, t, q, sx, amax_col, mask);
  else if (nch <= 512)
    k_int8_rows<BF16, 2, WEIGHT><<<grid, block, 0, s>>>(X, K, t, q, sx, amax_col, mask);
  else if (nch <= 1024)
    k_int8_rows<BF16, 4, WEIGHT><<<grid, block, 0, s>>>(X, K, t, q, sx, amax_col, mask);
  else if (nch <= 2048)
    k_int8_rows<BF16, 8, WEIGHT><<<grid, block, 0, s>>>(X, K, t, q, sx, amax_col, mask);
  else
    k_int8_rows<BF16, 0, WEIGHT><<<grid, block, 0, s>>>(X, K, t, q, sx, amax_col, mask);
}

void launch_clear(uint32_t* p, int n, hipStream_t s) {
  const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  k_clear<<<dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s>>>(p, n);
}

void launch_int8_rows(const void* X, bool bf16, int64_t rows, int K, float t, int8_t* q, float* sx,
                      int* amax_col, uint32_t* mask, bool weight, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  if (bf16) {
    if (weight) launch_int8_rows_t<true, true>(x, rows, K, t, q, sx, amax_col, mask, s);
    else launch_int8_rows_t<true, false>(x, rows, K, t, q, sx, amax_col, mask, s);
  } else {
    if (weight) launch_int8_rows_t<false, true>(x, rows, K, t, q, sx, amax_col, mask, s);
    else launch_int8_rows_t<false, false>(x, rows, K, t, q, sx, amax_col, mask, s);
  }
}

size_t outlier_fixup_lds_bytes(int K) { return static_cast<size_t>(2) * ((K + 31) / 32) * 4; }

void launch_outlier_fixup(const void* X, bool bf16, int64_t M, int K, const uint32_t* mask, int8_t* q,
                          float* sx, const int* amax_col, int* O, int* nO, uint16_t* XO,
                          const int8_t* Wq, int64_t N, uint16_t* WO, hipStream_t s) {
  const int xblocks = static_cast<int>((M + kFixRows - 1) / kFixRows);
  const int wblocks = WO ? static_cast<int>((N + kFixRows - 1) / kFixRows) : 0;
  const size_t lds = outlier_fixup_lds_bytes(K);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const dim3 grid(xblocks + wblocks), block(256);
  if (bf16)
    k_outlier_fixup<true><<<grid, block, lds, s>>>(x, (int)M, K, mask, q, sx, amax_col, O, nO, XO, Wq,
                                                   (int)N, WO, xblocks);
  else
    k_outlier_fixup<false><<<grid, block, lds, s>>>(x, (int)M, K, mask, q, sx, amax_col, O, nO, XO, Wq,
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
