// Dynamic FP8 (OCP E4M3) activation quantization kernels for gfx950.
//
// Per-token-group quantization with row-padded, column-major scales follows
// the PR 27896 digest ("Remove the per-call padding overhead of the FP8
// blockwise GEMM", sections "Implementation" and "Key source excerpts"): one
// fp32 scale per (row, group of G columns), scale = max(absmax, eps) / 448,
// codes = E4M3(x / scale) clamped to +-448, scale (m, g) stored at g*M_pad + m,
// rows at or beyond M untouched. Per-token quantization is the same with one
// group per row.
//
// All kernels here are HBM-bound streaming kernels: 2 bytes read (4 with
// SiLU-and-mul) and 1 byte written per element, plus 4 bytes per group. Every
// thread owns 16 elements (16-byte loads, one 16-byte store) so global
// accesses are 128-bit and contiguous across lanes.
#include "common.h"
#include "kernels.h"

namespace fp8w8a8 {

// ---------------------------------------------------------------------------
// Variants named by the quantizer's kernel call on the same page
// (fuse_silu_and_mul, scale_ue8m0 flags) and by the A100 dtype page (a static
// FP8 quantization kernel), whose bodies the pages do not show. Readings:
//  * SiLU-and-mul: the input row is [gate | up] (2K values); the row that is
//    quantized is y = bf16(silu(gate) * up), silu(g) = g / (1 + e^-g), so the
//    fused call equals SiLU-and-mul (bf16 out) followed by the quantizer.
//  * UE8M0: each fp32 scale is rounded up to a power of two.
//  * Static: a given fp32 scale, codes E4M3(clamp(x / s)), no scale written.
// ---------------------------------------------------------------------------

// The 16 values of unit u of a row as bf16: the input itself, or (SiLU-and-mul)
// silu(gate) * up from the two halves of a 2K-wide row.
template <int FLAGS>
__device__ __forceinline__ void load_unit(const uint16_t* xr, int64_t K, int64_t u, uint4& v0,
                                          uint4& v1) {
  const uint4* src = reinterpret_cast<const uint4*>(xr + u * 16);
  if constexpr ((FLAGS & kQuantSiluMul) != 0) {
    const uint4* up = reinterpret_cast<const uint4*>(xr + K + u * 16);
    const uint4 g0 = load16_nt(src), g1 = load16_nt(src + 1);
    const uint4 u0 = load16_nt(up), u1 = load16_nt(up + 1);
    v0 = silu_mul8(g0, u0);
    v1 = silu_mul8(g1, u1);
  } else {
    v0 = load16_nt(src);
    v1 = load16_nt(src + 1);
  }
}

// Scale of a group from its absmax: fp32 (absmax floored at eps) / 448,
// rounded up to a power of two for UE8M0.
template <int FLAGS>
__device__ __forceinline__ float group_scale(float amax, float eps) {
  const float s = fmaxf(amax, eps) / kE4M3Max;
  return (FLAGS & kQuantUe8m0) != 0 ? pow2_ceil(s) : s;
}

// ---------------------------------------------------------------------------
// Per-token: one workgroup per row; the row's 16-element units are spread over
// the workgroup's threads and kept in registers (UNITS per thread), the row
// absmax is reduced wave-wise then across waves through LDS, and the codes are
// produced from the registers, so the row is read from HBM once.
// ---------------------------------------------------------------------------
template <int UNITS, int FLAGS>
__global__ __launch_bounds__((FLAGS & kQuantSiluMul) != 0 ? 1024 : 256) void quant_per_token_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, float eps) {
  __shared__ float wave_part[16];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;
  const int units = (int)(K >> 4);
  const int nthr = blockDim.x;

  uint4 v[UNITS][2];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < UNITS; ++i) {
    const int u = threadIdx.x + i * nthr;
    if (u < units) {
      load_unit<FLAGS>(xr, K, u, v[i][0], v[i][1]);
      amax = fmaxf(amax, fmaxf(absmax8_bf16(v[i][0]), absmax8_bf16(v[i][1])));
    }
  }
  amax = wave_max(amax);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) wave_part[wave] = amax;
  __syncthreads();
  float m = wave_part[0];
  for (int w = 1; w < (nthr >> 6); ++w) m = fmaxf(m, wave_part[w]);
  const float s = group_scale<FLAGS>(m, eps);
  const float y = 1.0f / s;
  if (threadIdx.x == 0) scale[row] = s;
#pragma unroll
  for (int i = 0; i < UNITS; ++i) {
    const int u = threadIdx.x + i * nthr;
    if (u < units) {
      const uint2 lo = quant8_bf16(v[i][0], s, y);
      const uint2 hi = quant8_bf16(v[i][1], s, y);
      *reinterpret_cast<uint4*>(qr + (int64_t)u * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

// Rows longer than 256 threads x 8 units: two passes over the row (the second
// pass re-reads it from cache; SiLU-and-mul is evaluated again, to the same bits).
template <int FLAGS>
__global__ __launch_bounds__(256) void quant_per_token_long_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, float eps) {
  __shared__ float wave_part[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;
  const int64_t units = K >> 4;
  float amax = 0.0f;
  for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
    uint4 v0, v1;
    load_unit<FLAGS>(xr, K, u, v0, v1);
    amax = fmaxf(amax, fmaxf(absmax8_bf16(v0), absmax8_bf16(v1)));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = amax;
  __syncthreads();
  float m = wave_part[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, wave_part[w]);
  const float s = group_scale<FLAGS>(m, eps);
  const float y = 1.0f / s;
  if (threadIdx.x == 0) scale[row] = s;
  for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
    uint4 v0, v1;
    load_unit<FLAGS>(xr, K, u, v0, v1);
    const uint2 lo = quant8_bf16(v0, s, y);
    const uint2 hi = quant8_bf16(v1, s, y);
    *reinterpret_cast<uint4*>(qr + u * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---------------------------------------------------------------------------
// Per-token-group: one thread per 16-element unit, TPG = G/16 consecutive
// threads per group (aligned, so a group never straddles a wavefront and its
// absmax is an xor-shuffle reduction over TPG lanes). Units are numbered
// row-major over [M, K/16]; a group never straddles a row since G divides K.
// ---------------------------------------------------------------------------
// MASKED: grid y runs over experts; expert e quantizes the first masked_m[e]
// rows (clamped to [0, M]) of its own slab and leaves the rest untouched.
template <int TPG, int FLAGS, bool MASKED = false>
__global__ __launch_bounds__(256) void quant_group_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, int64_t m_pad, float eps, MaskArgs mask) {
  const int64_t units_per_row = K >> 4;
  if constexpr (MASKED) {
    const int64_t e = blockIdx.y;
    int64_t rows = mask.masked_m[e];
    rows = rows < 0 ? 0 : (rows > M ? M : rows);
    if ((int64_t)blockIdx.x * blockDim.x >= rows * units_per_row) return;  // whole block past the rows
    M = rows;
    x += e * mask.x_es;
    q += e * mask.q_es;
    scale += e * mask.s_es;
  }
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = u < M * units_per_row;
  const int64_t row = live ? u / units_per_row : 0;
  const int64_t col_unit = live ? u - row * units_per_row : 0;

  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
  if (live) load_unit<FLAGS>(x + row * ldx, K, col_unit, v0, v1);
  float amax = fmaxf(absmax8_bf16(v0), absmax8_bf16(v1));
#pragma unroll
  for (int off = TPG / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = group_scale<FLAGS>(amax, eps);
  const float y = 1.0f / s;
  if (live) {
    const uint2 lo = quant8_bf16(v0, s, y);
    const uint2 hi = quant8_bf16(v1, s, y);
    *reinterpret_cast<uint4*>(q + row * ldq + col_unit * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    if ((col_unit & (TPG - 1)) == 0) {
      const int64_t g = col_unit / TPG;
      scale[g * m_pad + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Static per-tensor quantization: one thread per 16-element unit, the scale
// read from device memory, codes from IEEE fp32 division x / s (the scale is
// arbitrary here, so the reciprocal-and-correction sequence of the dynamic
// kernels, checked only for scales derived from a bf16 absmax, is not used).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint2 quant8_bf16_div(const uint4& w, float s) {
  const uint32_t p[4] = {w.x, w.y, w.z, w.w};
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __fdiv_rn(bf16_to_f32(p[i] & 0xffffu), s);
    r[2 * i + 1] = __fdiv_rn(bf16_to_f32(p[i] >> 16), s);
  }
  int lo = e4m3_pack2<false>(r[0], r[1], 0);
  lo = e4m3_pack2<true>(r[2], r[3], lo);
  int hi = e4m3_pack2<false>(r[4], r[5], 0);
  hi = e4m3_pack2<true>(r[6], r[7], hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

__global__ __launch_bounds__(256) void quant_static_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, const float* __restrict__ scale,
    uint8_t* __restrict__ q, int64_t ldq) {
  const int64_t units_per_row = K >> 4;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= M * units_per_row) return;
  const int64_t row = u / units_per_row;
  const int64_t col_unit = u - row * units_per_row;
  const float s = scale[0];
  const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + col_unit * 16);
  const uint4 v0 = load16_nt(src), v1 = load16_nt(src + 1);
  const uint2 lo = quant8_bf16_div(v0, s);
  const uint2 hi = quant8_bf16_div(v1, s);
  *reinterpret_cast<uint4*>(q + row * ldq + col_unit * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// ---------------------------------------------------------------------------
// Launchers (arguments already validated by the C ABI layer).
// ---------------------------------------------------------------------------
namespace {

template <int FLAGS>
void launch_per_token_flags(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* scale, float eps, hipStream_t stream) {
  const int64_t units = K >> 4;
  // threads: a multiple of 64, enough to keep UNITS <= 8, at most 256 -- or,
  // with SiLU-and-mul, whose per-element work is several times larger, at most
  // 1024 while there are too few rows to fill the chip, so that a short batch
  // of long rows still spreads over many waves
  const int cap = (FLAGS & kQuantSiluMul) != 0 && M < 1024 ? 1024 : 256;
  int threads = (int)((units + 63) / 64) * 64;
  if (threads > cap) threads = cap;
  const int64_t per = (units + threads - 1) / threads;
  const dim3 grid((unsigned)M), block((unsigned)threads);
  if (per <= 1)
    hipLaunchKernelGGL((quant_per_token_kernel<1, FLAGS>), grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 2)
    hipLaunchKernelGGL((quant_per_token_kernel<2, FLAGS>), grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 4)
    hipLaunchKernelGGL((quant_per_token_kernel<4, FLAGS>), grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 8)
    hipLaunchKernelGGL((quant_per_token_kernel<8, FLAGS>), grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else
    hipLaunchKernelGGL((quant_per_token_long_kernel<FLAGS>), grid, dim3(256), 0, stream, x, K, ldx, q, ldq, scale, eps);
}

template <int FLAGS, bool MASKED>
void launch_group_flags(const uint16_t* x, int64_t experts, int64_t M, int64_t K, int64_t ldx,
                        int group_size, int64_t m_pad, uint8_t* q, int64_t ldq, float* scale,
                        float eps, const MaskArgs& mask, hipStream_t stream) {
  const int64_t units = M * (K >> 4);
  const dim3 block(256), grid((unsigned)((units + 255) / 256), (unsigned)(MASKED ? experts : 1));
  switch (group_size) {
    case 16:
      hipLaunchKernelGGL((quant_group_kernel<1, FLAGS, MASKED>), grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps, mask);
      break;
    case 32:
      hipLaunchKernelGGL((quant_group_kernel<2, FLAGS, MASKED>), grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps, mask);
      break;
    case 64:
      hipLaunchKernelGGL((quant_group_kernel<4, FLAGS, MASKED>), grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps, mask);
      break;
    default:
      hipLaunchKernelGGL((quant_group_kernel<8, FLAGS, MASKED>), grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps, mask);
      break;
  }
}

template <bool MASKED>
void launch_group_any(const uint16_t* x, int64_t experts, int64_t M, int64_t K, int64_t ldx,
                      int group_size, int64_t m_pad, uint8_t* q, int64_t ldq, float* scale,
                      float eps, int flags, const MaskArgs& mask, hipStream_t stream) {
  switch (flags & (kQuantSiluMul | kQuantUe8m0)) {
    case 0:
      launch_group_flags<0, MASKED>(x, experts, M, K, ldx, group_size, m_pad, q, ldq, scale, eps, mask, stream);
      break;
    case kQuantSiluMul:
      launch_group_flags<kQuantSiluMul, MASKED>(x, experts, M, K, ldx, group_size, m_pad, q, ldq, scale,
                                                eps, mask, stream);
      break;
    case kQuantUe8m0:
      launch_group_flags<kQuantUe8m0, MASKED>(x, experts, M, K, ldx, group_size, m_pad, q, ldq, scale,
                                              eps, mask, stream);
      break;
    default:
      launch_group_flags<kQuantSiluMul | kQuantUe8m0, MASKED>(x, experts, M, K, ldx, group_size, m_pad,
                                                              q, ldq, scale, eps, mask, stream);
      break;
  }
}

}  // namespace

hipError_t launch_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale, float eps, int flags,
                                  hipStream_t stream) {
  switch (flags & (kQuantSiluMul | kQuantUe8m0)) {
    case 0: launch_per_token_flags<0>(x, M, K, ldx, q, ldq, scale, eps, stream); break;
    case kQuantSiluMul: launch_per_token_flags<kQuantSiluMul>(x, M, K, ldx, q, ldq, scale, eps, stream); break;
    case kQuantUe8m0: launch_per_token_flags<kQuantUe8m0>(x, M, K, ldx, q, ldq, scale, eps, stream); break;
    default:
      launch_per_token_flags<kQuantSiluMul | kQuantUe8m0>(x, M, K, ldx, q, ldq, scale, eps, stream);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_per_token_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                        int group_size, int64_t m_pad, uint8_t* q, int64_t ldq,
                                        float* scale, float eps, int flags, hipStream_t stream) {
  const MaskArgs none{};
  launch_group_any<false>(x, 1, M, K, ldx, group_size, m_pad, q, ldq, scale, eps, flags, none, stream);
  return hipGetLastError();
}

hipError_t launch_quant_per_token_group_masked(const uint16_t* x, int64_t experts, int64_t M,
                                               int64_t K, int64_t ldx, int group_size,
                                               int64_t m_pad, uint8_t* q, int64_t ldq, float* scale,
                                               float eps, int flags, const MaskArgs& mask,
                                               hipStream_t stream) {
  launch_group_any<true>(x, experts, M, K, ldx, group_size, m_pad, q, ldq, scale, eps, flags, mask,
                         stream);
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* scale, uint8_t* q, int64_t ldq, hipStream_t stream) {
  const int64_t units = M * (K >> 4);
  const dim3 block(256), grid((unsigned)((units + 255) / 256));
  hipLaunchKernelGGL(quant_static_kernel, grid, block, 0, stream, x, M, K, ldx, scale, q, ldq);
  return hipGetLastError();
}

}  // namespace fp8w8a8
