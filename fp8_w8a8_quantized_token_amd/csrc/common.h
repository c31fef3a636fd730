// Device helpers shared by the gfx950 kernels of the FP8 W8A8 library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w8a8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;

// 16-byte global load with the non-temporal hint (data read exactly once).
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Plain 16-byte global load (data other workgroups may re-read from cache).
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs;
// NaN maps to a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> OCP E4M3 code, saturating at +-448, round to nearest even, sign of
// zero kept. Built from the E4M3 bit layout (sign | 4-bit exponent, bias 7 |
// 3-bit mantissa; subnormals are k * 2^-9):
//  * |v| < 2^-6: the result is k * 2^-9 with k = rne(|v| * 2^9) in 0..8; the
//    code of k * 2^-9 is k itself (k = 8 is the smallest normal, code 0x08);
//  * otherwise: round the fp32 mantissa to 3 bits (RNE on the bit pattern,
//    a carry moves into the exponent) and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), kE4M3Max);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
  }
  return code | sign;
}

// Max over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// |x| maximum of the 8 bf16 values packed in a 16-byte word.
__device__ __forceinline__ float absmax8_bf16(const uint4& w) {
  float m = 0.0f;
  const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_to_f32(p[i] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_to_f32(p[i] >> 16)));
  }
  return m;
}

// Quantize the 8 bf16 values of a 16-byte word with scale s (true fp32
// division per element) into 8 E4M3 codes packed little-endian in a uint2.
__device__ __forceinline__ uint2 quant8_bf16(const uint4& w, float s) {
  const uint32_t p[4] = {w.x, w.y, w.z, w.w};
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = e4m3_encode(bf16_to_f32(p[i] & 0xffffu) / s);
    const uint32_t hi = e4m3_encode(bf16_to_f32(p[i] >> 16) / s);
    c[i] = lo | (hi << 8);
  }
  return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
}

}  // namespace fp8w8a8
