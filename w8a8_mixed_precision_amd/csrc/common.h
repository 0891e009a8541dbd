// Internal helpers of libw8mp's gfx950 kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- 16-bit storage <-> fp32 ------------------------------------------------

template <bool BF16>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (BF16) {
    return __uint_as_float(bits16 << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  }
}

// Unpack the eight 16-bit values of a 16-byte chunk.
template <bool BF16>
__device__ __forceinline__ void unpack8(const uint4& v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = to_f32<BF16>(w[i] & 0xFFFFu);
    f[2 * i + 1] = to_f32<BF16>(w[i] >> 16);
  }
}

// fp32 -> bf16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x, a float32 value, rounded to fp16 (v_cvt_f16_f32, RNE). The empty asm
// hides where x came from: otherwise instruction selection may fuse an FMA
// producing x with this conversion into one mixed-precision FMA
// (v_fma_mixlo_f16), which rounds the exact result once, to fp16, and so
// differs from rounding x in about one result in 10^5, for some elements of
// a kernel and not others.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  __asm__("" : "+v"(x));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// The pair (a, b), float32 values, each rounded to fp16 as f32_to_f16_bits
// does, packed a | b << 16: one v_cvt_pk_f16_f32 (gfx950) instead of two
// conversions and an OR. Equal to the two scalar conversions for every pair
// of float32 bit patterns (w8dbg_cvt_f16_pair_check).
typedef float w8_f2 __attribute__((ext_vector_type(2)));
typedef _Float16 w8_h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_f16x2_bits(float a, float b) {
  w8_f2 v{a, b};
  __asm__("" : "+v"(v));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, w8_h2));
}

// ---- integer code of the symmetric absmax int8 scheme ----------------------
// q = clamp(rne(fl32(x * r)), -127, 127), 0 for x == 0 (r may be +inf).
__device__ __forceinline__ int absmax_code(float x, float r) {
  if (x == 0.0f) return 0;
  float p = __builtin_rintf(x * r);
  p = fminf(fmaxf(p, -127.0f), 127.0f);
  return static_cast<int>(p);
}

// ---- OCP E4M3FN encode: RNE, saturating at +-448, sign of zero kept ---------
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                 // below 2^-6: grid of 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {                                    // normal: keep 3 mantissa bits, RNE
    const uint32_t au = __float_as_uint(a);
    const uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);
    code = ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));
  }
  return sign | code;
}

// ---- wave / block reductions ------------------------------------------------

// Max of |x| with the column it came from; -1 column means "none".
struct MaxLoc {
  float v;
  int k;
};

__device__ __forceinline__ MaxLoc maxloc_pick(MaxLoc a, MaxLoc b) {
  // larger value wins; on a tie the smaller column (any choice would be valid)
  if (b.v > a.v || (b.v == a.v && b.k >= 0 && (a.k < 0 || b.k < a.k))) return b;
  return a;
}

__device__ __forceinline__ MaxLoc wave_maxloc(MaxLoc x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    MaxLoc o;
    o.v = __shfl_xor(x.v, off, kWave);
    o.k = __shfl_xor(x.k, off, kWave);
    x = maxloc_pick(x, o);
  }
  return x;
}

// Block-wide max-with-location for a 256-thread block; result on every thread.
__device__ __forceinline__ MaxLoc block_maxloc256(MaxLoc x, MaxLoc* red /*[4] in LDS*/) {
  x = wave_maxloc(x);
  const int wave = threadIdx.x / kWave;
  __syncthreads();  // red may still be read by a previous reduction
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  MaxLoc r = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) r = maxloc_pick(r, red[w]);
  return r;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float block_max256(float x, float* red /*[4] in LDS*/) {
  x = wave_max(x);
  const int wave = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

}  // namespace w8
