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

// x / s rounded to nearest fp32, from y = RN(1/s) computed once per group:
// q0 = RN(x*y), r = x - q0*s (exact, one fma), q1 = RN(q0 + r*y). Checked
// exhaustively on the host against IEEE division for every positive bf16 x
// and every scale s = RN(max(a, 1e-10)/448) from a bf16 absmax a >= x
// (532,668,480 pairs): the E4M3 code of q1 equals that of RN(x/s) in every
// case (the quotients themselves differ only deep in the underflow range,
// where both encode to zero). The sign is taken from x, which is the sign of
// the true quotient (s > 0) also when it rounds to zero.
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
  const float q0 = __fmul_rn(x, y);
  const float r = __fmaf_rn(-q0, s, x);
  const float q1 = __fmaf_rn(r, y, q0);
  return __builtin_copysignf(q1, x);
}

// Two fp32 values -> two OCP E4M3 codes (saturating at +-448, round to
// nearest even, signed zero kept): clamp, then the packed hardware convert,
// which rounds to nearest even and handles the E4M3 subnormal range; it was
// checked against a bit-level E4M3 encoder on every fifth fp32 pattern in
// [-448, 448] and on every E4M3 midpoint +-2 ulp. The two codes land in the
// low (HI = false) or high 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ int e4m3_pack2(float a, float b, int old) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
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

// Quantize the 8 bf16 values of a 16-byte word with scale s (y = RN(1/s))
// into 8 E4M3 codes packed little-endian in a uint2.
__device__ __forceinline__ uint2 quant8_bf16(const uint4& w, float s, float y) {
  const uint32_t p[4] = {w.x, w.y, w.z, w.w};
  float q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = div_by_scale(bf16_to_f32(p[i] & 0xffffu), s, y);
    q[2 * i + 1] = div_by_scale(bf16_to_f32(p[i] >> 16), s, y);
  }
  int lo = e4m3_pack2<false>(q[0], q[1], 0);
  lo = e4m3_pack2<true>(q[2], q[3], lo);
  int hi = e4m3_pack2<false>(q[4], q[5], 0);
  hi = e4m3_pack2<true>(q[6], q[7], hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// Smallest power of two >= s, for a positive normal fp32 s.
__device__ __forceinline__ float pow2_ceil(float s) {
  uint32_t b = __float_as_uint(s);
  if (b & 0x007FFFFFu) b = (b & 0xFF800000u) + 0x00800000u;
  return __uint_as_float(b);
}

// Nearest bf16 (ties to even) of a double, without double rounding: the
// conversion to fp32 is made round-to-odd (inexact results get their last bit
// set after truncation), which keeps 16 guard bits for the bf16 rounding.
__device__ __forceinline__ uint32_t bf16_of_f64(double d) {
  const float f = (float)d;  // round to nearest
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {
    if (fabs(back) > fabs(d)) b -= 1u;  // rounded away from zero: step back
    b |= 1u;
  }
  return f32_to_bf16(__uint_as_float(b));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 (a in the low half), round to nearest even: the
// packed hardware convert of gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// silu(g) * u in fp32: e^-g as 2^(-g log2 e) on the hardware exp2 (within 1
// ulp), then the reciprocal (1 ulp) and two products. Relative error at most
// (1.23 |g| + 7) 2^-24 for g >= -16: the exponent -g log2 e is off by its
// rounding (2^-24 relative) plus that of the fp32 log2 e (0.22 2^-24), which
// 2^x turns into 1.23 |g| 2^-24 of e^-g and at most as much of the result;
// the other steps cost 7 2^-24 together. For g > 16.6 the e^-g term is below
// half an ulp of 1 and its error drops out.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  const float t = __builtin_amdgcn_exp2f(g * -1.44269504088896340736f);
  return (g * __builtin_amdgcn_rcpf(1.0f + t)) * u;
}

// True where the fp32 value y = silu_mul_f32(g, u) may round to a different
// bf16 than the exact product: y lies within 48 fp32 ulps of a bf16 rounding
// midpoint (low 16 bits near 0x8000; the relative bound above is under
// 1.23 |g| + 7 ulps of y, an ulp being at least 2^-24 of |y|: at most 27 ulps
// for g >= -16), or g < -16, outside that bound. A window scaled with |g|
// sends fewer values to the fp64 path but measured slower: its per-value
// arithmetic costs more than the redo it saves.
__device__ __forceinline__ bool silu_needs_f64(float g, float y) {
  const uint32_t low = __float_as_uint(y) & 0xFFFFu;
  return !(g >= -16.0f) || (low - (0x8000u - 48u)) <= 96u;
}

// bf16 bits of silu(g) * u from fp64 (exp in fp64 within 1 ulp, IEEE
// division): correctly rounded unless the exact value lies within ~2^-50
// relative of a bf16 midpoint.
static __device__ __noinline__ uint32_t silu_mul_bf16_f64(float g, float u) {
  const double gd = (double)g;
  return bf16_of_f64(gd / (1.0 + exp(-gd)) * (double)u);
}

// 8 gate and 8 up bf16 values -> 8 bf16 values of silu(gate) * up, correctly
// rounded. All eight fp32 evaluations run first, straight-line; the few that
// sit too close to a bf16 rounding midpoint (about 1 in 700 on normal data)
// are redone in fp64 behind one branch per 8 values.
__device__ __forceinline__ uint4 silu_mul8(const uint4& g, const uint4& u) {
  const uint32_t gp[4] = {g.x, g.y, g.z, g.w};
  const uint32_t up[4] = {u.x, u.y, u.z, u.w};
  float gf[8], uf[8], y[8];
  bool redo = false;  // a lane mask: the per-value tests are repeated in the rare branch
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gf[i] = bf16_to_f32((i & 1) ? (gp[i >> 1] >> 16) : (gp[i >> 1] & 0xffffu));
    uf[i] = bf16_to_f32((i & 1) ? (up[i >> 1] >> 16) : (up[i >> 1] & 0xffffu));
    y[i] = silu_mul_f32(gf[i], uf[i]);
    redo = redo || silu_needs_f64(gf[i], y[i]);
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
  if (redo) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (silu_needs_f64(gf[i], y[i])) {
        const uint32_t b = silu_mul_bf16_f64(gf[i], uf[i]);
        o[i >> 1] = (i & 1) ? ((o[i >> 1] & 0xffffu) | (b << 16)) : ((o[i >> 1] & 0xffff0000u) | b);
      }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace fp8w8a8
