// The op that produces X, fused into the int8 row pass and the outlier fix-up
// (internal to libw8mp). Each producer is a fixed sequence of float32
// operations, every one rounded to nearest even and none contracted into an
// FMA, so the 16-bit X it yields is one well-defined value per element:
//
//  * RMSNorm (Zhang and Sennrich, 2019) with the x(1+scale)+shift modulation of
//    adaptive layer norm (Peebles and Xie, "Scalable Diffusion Models with
//    Transformers", 2023):
//      ss   = sum_k h^2 (float64, each square exact)
//      rstd = fl32(1 / fl32(sqrt(fl32(fl32(ss / K) + eps))))
//      x    = fl32(fl32(h * rstd) * fl32(gamma * fl32(1 + scale))) [+ shift]
//  * GELU, tanh form (Hendrycks and Gimpel, 2016), evaluated as
//      h / (1 + exp(-2u)),  u = sqrt(2/pi) (h + 0.044715 h^3),
//    equal to 0.5 h (1 + tanh u) and accurate for negative h, with exp32 below.
//
// X = the float32 result rounded to nearest even in the 16-bit type of H.
#pragma once

#include "common.h"

namespace w8 {

enum : int { kProdNone = 0, kProdRms = 1, kProdGelu = 2 };

struct ProdArgs {
  const float* gamma;   // [K] or null (1)
  const float* scale;   // [K] or null (0)
  const float* shift;   // [K] or null (no addition)
  float eps;
  float* rstd;          // [M]: written by the row pass, read by the fix-up (RMSNorm)
};

// exp(x) = 2^k p(r): k = rint(x log2 e), r = x - k ln2 in two parts (Cody and
// Waite, 1980; the high part has 9 significant bits, so k * LN2_HI is exact),
// p = the degree-6 Taylor polynomial of exp on |r| <= ln(2)/2 by Horner's rule.
// About 2 ulp; +inf past FLT_MAX, 0 below the subnormals.
__device__ __forceinline__ float exp32(float x) {
#pragma clang fp contract(off)
  constexpr float kLog2e = 0x1.715476p+0f;
  constexpr float kLn2Hi = 0x1.63p-1f;
  constexpr float kLn2Lo = -0x1.bd0106p-13f;
  const float k = __builtin_rintf(x * kLog2e);
  float r = x - k * kLn2Hi;
  r = r - k * kLn2Lo;
  float p = 0x1.6c16c2p-10f;                    // 1/720
  p = p * r + 0x1.111112p-7f;                   // 1/120
  p = p * r + 0x1.555556p-5f;                   // 1/24
  p = p * r + 0x1.555556p-3f;                   // 1/6
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const int ki = static_cast<int>(fminf(fmaxf(k, -300.0f), 300.0f));
  return __builtin_ldexpf(p, ki);
}

__device__ __forceinline__ float gelu32(float h) {
#pragma clang fp contract(off)
  constexpr float kC = 0x1.988454p-1f;          // sqrt(2/pi)
  constexpr float kA = 0x1.6e4e26p-5f;          // 0.044715
  const float h3 = (h * h) * h;
  const float inner = h + kA * h3;
  const float u = kC * inner;
  const float e = exp32(u * -2.0f);
  const float den = 1.0f + e;
  return h / den;                               // IEEE division
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

// One element of X from one 16-bit value of H in column k.
template <bool BF16, int PROD>
__device__ __forceinline__ uint32_t produce1(uint32_t hbits, int k, float rstd, const ProdArgs& pa) {
  if constexpr (PROD == kProdNone) {
    return hbits;
  } else {
    const float h = to_f32<BF16>(hbits);
    if constexpr (PROD == kProdGelu) return round16<BF16>(gelu32(h));
    else return round16<BF16>(rms_apply(h, rstd, rms_gain(pa, k), pa, k));
  }
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
__device__ __forceinline__ uint4 produce8(const uint4& hv, int c, float rstd, const ProdArgs& pa) {
#pragma clang fp contract(off)
  if constexpr (PROD == kProdNone) {
    return hv;
  } else {
    float h[8];
    unpack8<BF16>(hv, h);
    uint32_t b[8];
    if constexpr (PROD == kProdGelu) {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = round16<BF16>(gelu32(h[j]));
    } else {
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

}  // namespace w8
