// Device side of the producers fused into the int8 row pass, the outlier
// fix-up and the GEMM's outlier gather (internal to libw8mp). X is the value
// a separate producer op would store in H's 16-bit type:
//
//  * RMSNorm (Zhang and Sennrich, 2019) with the x(1+scale)+shift modulation of
//    adaptive layer norm (Peebles and Xie, "Scalable Diffusion Models with
//    Transformers", 2023), a fixed sequence of float32 operations, each
//    rounded to nearest even and none contracted into an FMA:
//      ss   = sum_k h^2 (float64; each square is exact)
//      rstd = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))))
//      x    = fl32(fl32(h * rstd) * fl32(gamma * fl32(1 + scale))) [+ shift]
//    then rounded to nearest even in H's type. The float64 sum of squares is
//    added in this kernel's order; it can differ from the exactly rounded sum
//    in the last bit, which moves rstd only when fl32(ss / K) sits at a
//    rounding boundary.
//  * GELU, tanh form (Hendrycks and Gimpel, 2016):
//      gelu(h) = 0.5 h (1 + tanh u),  u = sqrt(2/pi) (h + 0.044715 h^3),
//    correctly rounded in H's type. X depends on the 16-bit pattern of h
//    alone, so it is read from a table of all 65536 results per format, made
//    at build time by gelu_table_gen.cpp (kGeluF16, kGeluBF16). Kernels that
//    map many elements copy the format's 128 KB table into LDS; the rest read
//    it from global memory.
#pragma once

#include "common.h"
#include "producer.h"

namespace w8 {

#include "gelu_table.inc"

template <bool BF16>
__device__ __forceinline__ const uint16_t* gelu_table_global() {
  if constexpr (BF16) return kGeluBF16;
  else return kGeluF16;
}

// fl32(gamma[k] * fl32(1 + scale[k])), the modulated gain of column k
__device__ __forceinline__ float rms_gain(const ProdArgs& pa, int k) {
#pragma clang fp contract(off)
  const float g = pa.gamma ? pa.gamma[k] : 1.0f;
  const float one_plus = pa.scale ? 1.0f + pa.scale[k] : 1.0f;
  return g * one_plus;
}

__device__ __forceinline__ float rms_apply(float h, float rstd, float gain, const ProdArgs& pa, int k) {
#pragma clang fp contract(off)
  float x = h * rstd;
  x = x * gain;
  if (pa.shift) x = x + pa.shift[k];
  return x;
}

// rstd from the float64 sum of squares of a row of K values
__device__ __forceinline__ float rms_rstd(double ss, int K, float eps) {
#pragma clang fp contract(off)
  const float ms = static_cast<float>(ss / static_cast<double>(K));
  const float v = ms + eps;
  return 1.0f / __builtin_sqrtf(v);
}

template <bool BF16>
__device__ __forceinline__ uint32_t round16(float x) {
  if constexpr (BF16) return bf16_rne_bits(x);
  else return f32_to_f16_bits(x);
}

// One element of X from one 16-bit value of H in column k. `gelu`: the GELU
// table of the format (LDS or global memory).
template <bool BF16, int PROD>
__device__ __forceinline__ uint32_t produce1(uint32_t hbits, int k, float rstd, const ProdArgs& pa,
                                             const uint16_t* gelu) {
  if constexpr (PROD == kProdNone) {
    return hbits;
  } else if constexpr (PROD == kProdGelu) {
    return gelu[hbits & 0xFFFFu];
  } else {
    const float h = to_f32<BF16>(hbits);
    return round16<BF16>(rms_apply(h, rstd, rms_gain(pa, k), pa, k));
  }
}

// produce1 with the producer chosen at run time (the rare paths that are not
// specialised per producer); GELU from the global table.
template <bool BF16>
__device__ __forceinline__ uint32_t produce1_any(int prod, uint32_t hbits, int k, float rstd, const ProdArgs& pa) {
  if (prod == kProdGelu) return gelu_table_global<BF16>()[hbits & 0xFFFFu];
  if (prod == kProdRms) return produce1<BF16, kProdRms>(hbits, k, rstd, pa, nullptr);
  return hbits;
}

// Eight consecutive floats of an optional [K] vector (16-byte aligned).
__device__ __forceinline__ void load8(const float* v, int c, float (&out)[8], float dflt) {
  if (v) {
    const float4 a = reinterpret_cast<const float4*>(v)[2 * c];
    const float4 b = reinterpret_cast<const float4*>(v)[2 * c + 1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = dflt;
  }
}

// Eight elements of X (chunk c: columns 8c .. 8c+7) from eight of H; the
// RMSNorm vectors are read as 16-byte loads, the same values produce1 reads.
template <bool BF16, int PROD>
__device__ __forceinline__ uint4 produce8(const uint4& hv, int c, float rstd, const ProdArgs& pa,
                                          const uint16_t* gelu) {
#pragma clang fp contract(off)
  if constexpr (PROD == kProdNone) {
    return hv;
  } else if constexpr (PROD == kProdGelu) {
    const uint32_t w[4] = {hv.x, hv.y, hv.z, hv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = static_cast<uint32_t>(gelu[w[i] & 0xFFFFu]) | (static_cast<uint32_t>(gelu[w[i] >> 16]) << 16);
    return make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    float h[8];
    unpack8<BF16>(hv, h);
    uint32_t b[8];
    float g[8], sc[8], sh[8];
    load8(pa.gamma, c, g, 1.0f);
    load8(pa.scale, c, sc, 0.0f);
    load8(pa.shift, c, sh, 0.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gain = g[j] * (pa.scale ? 1.0f + sc[j] : 1.0f);
      float x = h[j] * rstd;
      x = x * gain;
      if (pa.shift) x = x + sh[j];
      b[j] = round16<BF16>(x);
    }
    return make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
  }
}

// Partial float64 sum of squares of the eight values of a chunk.
template <bool BF16>
__device__ __forceinline__ double sumsq8(const uint4& hv) {
  float f[8];
  unpack8<BF16>(hv, f);
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += static_cast<double>(f[j]) * static_cast<double>(f[j]);
  return s;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Copies the format's GELU table (65536 patterns, 128 KB) into LDS; every
// thread of the block takes part, and the caller synchronises afterwards.
template <bool BF16>
__device__ __forceinline__ void gelu_table_to_lds(uint16_t* lds_tab) {
  const uint4* src = reinterpret_cast<const uint4*>(gelu_table_global<BF16>());
  uint4* dst = reinterpret_cast<uint4*>(lds_tab);
  for (int i = threadIdx.x; i < 65536 * 2 / 16; i += blockDim.x) dst[i] = src[i];
}

}  // namespace w8
