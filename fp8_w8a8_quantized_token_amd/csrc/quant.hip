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
// Both kernels are HBM-bound streaming kernels: 2 bytes read and 1 byte
// written per element (plus 4 bytes per group). Every thread owns 16 elements
// (two 16-byte loads, one 16-byte store) so global accesses are 128-bit and
// contiguous across lanes.
#include "common.h"
#include "kernels.h"

namespace fp8w8a8 {

// ---------------------------------------------------------------------------
// Per-token: one workgroup per row; the row's 16-element units are spread over
// the workgroup's threads and kept in registers (UNITS per thread), the row
// absmax is reduced wave-wise then across waves through LDS, and the codes are
// produced from the registers, so the row is read from HBM once.
// ---------------------------------------------------------------------------
template <int UNITS>
__global__ __launch_bounds__(256) void quant_per_token_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, float eps) {
  __shared__ float wave_part[4];
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
      const uint4* src = reinterpret_cast<const uint4*>(xr + (int64_t)u * 16);
      v[i][0] = load16_nt(src);
      v[i][1] = load16_nt(src + 1);
      amax = fmaxf(amax, fmaxf(absmax8_bf16(v[i][0]), absmax8_bf16(v[i][1])));
    }
  }
  amax = wave_max(amax);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) wave_part[wave] = amax;
  __syncthreads();
  float m = wave_part[0];
  for (int w = 1; w < (nthr >> 6); ++w) m = fmaxf(m, wave_part[w]);
  const float s = fmaxf(m, eps) / kE4M3Max;
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
// pass re-reads it from cache).
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
    const uint4* src = reinterpret_cast<const uint4*>(xr + u * 16);
    amax = fmaxf(amax, fmaxf(absmax8_bf16(src[0]), absmax8_bf16(src[1])));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = amax;
  __syncthreads();
  float m = wave_part[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, wave_part[w]);
  const float s = fmaxf(m, eps) / kE4M3Max;
  const float y = 1.0f / s;
  if (threadIdx.x == 0) scale[row] = s;
  for (int64_t u = threadIdx.x; u < units; u += blockDim.x) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + u * 16);
    const uint2 lo = quant8_bf16(src[0], s, y);
    const uint2 hi = quant8_bf16(src[1], s, y);
    *reinterpret_cast<uint4*>(qr + u * 16) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// ---------------------------------------------------------------------------
// Per-token-group: one thread per 16-element unit, TPG = G/16 consecutive
// threads per group (aligned, so a group never straddles a wavefront and its
// absmax is an xor-shuffle reduction over TPG lanes). Units are numbered
// row-major over [M, K/16]; a group never straddles a row since G divides K.
// ---------------------------------------------------------------------------
template <int TPG>
__global__ __launch_bounds__(256) void quant_group_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, int64_t m_pad, float eps) {
  const int64_t units_per_row = K >> 4;
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = u < M * units_per_row;
  const int64_t row = live ? u / units_per_row : 0;
  const int64_t col_unit = live ? u - row * units_per_row : 0;

  uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
  if (live) {
    const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + col_unit * 16);
    v0 = load16_nt(src);
    v1 = load16_nt(src + 1);
  }
  float amax = fmaxf(absmax8_bf16(v0), absmax8_bf16(v1));
#pragma unroll
  for (int off = TPG / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = fmaxf(amax, eps) / kE4M3Max;
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
// Launchers (arguments already validated by the C ABI layer).
// ---------------------------------------------------------------------------
hipError_t launch_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale, float eps,
                                  hipStream_t stream) {
  const int64_t units = K >> 4;
  // threads: a multiple of 64, at most 256, enough to keep UNITS <= 8
  int threads = (int)((units + 63) / 64) * 64;
  if (threads > 256) threads = 256;
  const int64_t per = (units + threads - 1) / threads;
  const dim3 grid((unsigned)M), block((unsigned)threads);
  if (per <= 1)
    hipLaunchKernelGGL(quant_per_token_kernel<1>, grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 2)
    hipLaunchKernelGGL(quant_per_token_kernel<2>, grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 4)
    hipLaunchKernelGGL(quant_per_token_kernel<4>, grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else if (per <= 8)
    hipLaunchKernelGGL(quant_per_token_kernel<8>, grid, block, 0, stream, x, K, ldx, q, ldq, scale, eps);
  else
    hipLaunchKernelGGL(quant_per_token_long_kernel, grid, dim3(256), 0, stream, x, K, ldx, q, ldq, scale, eps);
  return hipGetLastError();
}

hipError_t launch_quant_per_token_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                        int group_size, int64_t m_pad, uint8_t* q, int64_t ldq,
                                        float* scale, float eps, hipStream_t stream) {
  const int64_t units = M * (K >> 4);
  const dim3 block(256), grid((unsigned)((units + 255) / 256));
  switch (group_size) {
    case 16:
      hipLaunchKernelGGL(quant_group_kernel<1>, grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps);
      break;
    case 32:
      hipLaunchKernelGGL(quant_group_kernel<2>, grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps);
      break;
    case 64:
      hipLaunchKernelGGL(quant_group_kernel<4>, grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps);
      break;
    default:
      hipLaunchKernelGGL(quant_group_kernel<8>, grid, block, 0, stream, x, M, K, ldx, q, ldq, scale, m_pad, eps);
      break;
  }
  return hipGetLastError();
}

}  // namespace fp8w8a8
