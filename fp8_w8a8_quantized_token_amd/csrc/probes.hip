// Measurement probes for gfx950: the ceilings the GEMM and quantizer kernels
// are compared with. None of them is part of the linear itself.
//
//  * stream_read_kernel: reads a buffer once from HBM (16-byte non-temporal
//    loads, U per lane in flight), the read-only ceiling of the weight stream
//    of the small-M GEMMs.
//  * l2_feed_kernel: every workgroup re-reads the same L2-resident window,
//    with register loads or with LDS-DMA loads (global_load_lds_dwordx4, the
//    form the panel-ring GEMM tiles use): the per-compute-unit feed rate from
//    L2.
//  * panel_feed_kernel: the panel tiles' LDS-DMA feed (64-row panels, 128
//    bytes per row and stage) alone, with LDS reads of the landed stages,
//    with a barrier per stage, or both.
//  * mfma_probe_kernel: back-to-back independent 32x32x64 FP8 MFMAs: the
//    dense FP8 matrix rate and, from it, the clock the matrix cores ran at.
//
// Every probe folds what it reads into a value that is stored only when it
// equals a key the host passes (never met in practice), so no load or MFMA
// can be removed by the compiler, and only vector stores write memory.
#include "common.h"
#include "kernels.h"

namespace fp8w8a8 {

namespace {
constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 8;
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* src, int64_t n16,
                                                                    uint32_t* sink, uint32_t key) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * kProbeThreads * kReadUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kProbeThreads * kReadUnroll + threadIdx.x; base < n16;
       base += step) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kProbeThreads;
      v[u] = load16_nt(src + (i < n16 ? i : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == key) sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

// A [rows][row_bytes] matrix read once in pieces of `piece` bytes per row:
// workgroup w owns rows [w R, w R + R) and walks the row length in steps of
// `piece` bytes, each step reading its R rows' pieces (one 1 KB load
// instruction covers 1024 / piece rows); kReadUnroll instructions of a lane in
// flight. piece = 128 is the access pattern of the panel-ring GEMM tiles'
// weight panels, piece >= 1024 that of the weight-streaming kernel.
__global__ __launch_bounds__(kProbeThreads) void strided_read_kernel(const uint8_t* src, int64_t row_bytes,
                                                                     int rows_per_wg, int piece,
                                                                     uint32_t* sink, uint32_t key) {
  uint32_t acc = 0;
  const int tid = threadIdx.x;
  const int lanes_per_row = piece / 16;       // lanes covering one row's piece
  const int rows_per_inst = 1024 / piece;     // rows per 64-lane instruction
  const int wave = tid >> 6, lane = tid & 63;
  const int inst_per_step = rows_per_wg / rows_per_inst;  // instructions per K step (all waves)
  const uint8_t* base = src + (int64_t)blockIdx.x * rows_per_wg * row_bytes;
  const int64_t total = (row_bytes / piece) * inst_per_step;  // instructions of this workgroup
  for (int64_t i0 = wave; i0 < total; i0 += 4 * kReadUnroll) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      int64_t i = i0 + 4 * u;
      i = i < total ? i : total - 1;
      const int64_t step = i / inst_per_step;
      const int r = (int)(i % inst_per_step) * rows_per_inst + lane / lanes_per_row;
      v[u] = load16_nt(base + (int64_t)r * row_bytes + step * piece + (lane % lanes_per_row) * 16);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == key) sink[blockIdx.x * kProbeThreads + tid] = acc;
}

// DMA == 0: register loads; DMA == 1: LDS-DMA loads into a 16-slot ring of
// 1 KB per wave (at most 15 slots in flight per wave, so a slot's previous
// load has landed before it is issued into again).
template <int DMA>
__global__ __launch_bounds__(kProbeThreads) void l2_feed_kernel(const uint8_t* src, int64_t window,
                                                                int reps, uint32_t* sink, uint32_t key) {
  uint32_t acc = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n1k = window / 1024;  // 1 KB pieces of the window
  if constexpr (DMA == 0) {
    for (int r = 0; r < reps; ++r) {
      for (int64_t p = wave; p < n1k; p += 4 * kReadUnroll) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
          int64_t q = p + 4 * u;
          q = q < n1k ? q : n1k - 1;
          v[u] = load16(src + q * 1024 + lane * 16);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      }
    }
  } else {
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][16][1024];
    const uint32_t base = (uint32_t)(uintptr_t)&ring[wave][0][0];
    int slot = 0;
    int64_t issued = 0;
    for (int r = 0; r < reps; ++r) {
      for (int64_t p = wave; p < n1k; p += 4) {
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(base + (uint32_t)slot * 1024);
        const uint8_t* g = src + p * 1024 + lane * 16;
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0v) : "memory", "m0");
        slot = (slot + 1) & 15;
        ++issued;
        // keep at most 15 pieces of this wave in flight
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (15 << 8));
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    acc = *reinterpret_cast<const uint32_t*>(&ring[wave][lane & 15][0]) + (uint32_t)issued;
  }
  if (acc == key) sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

// The panel tiles' feed pattern without their arithmetic: a workgroup of
// four waves streams 64-row panels (8 rows x 128 bytes per LDS-DMA
// instruction, two per wave) of its own L2-resident row block, stage s
// taking the rows' bytes [128 (s mod row_bytes / 128), +128), into an
// 8-slot ring with at most six stages in flight per wave. MODE bit 0: after
// each stage's wait every wave also reads 32 rows (4 KB) of the stage that
// landed six stages back from LDS (the tiles' two readers per panel row);
// bit 1: a workgroup barrier after each stage's wait.
template <int MODE>
__global__ __launch_bounds__(kProbeThreads) void panel_feed_kernel(const uint8_t* src, uint32_t row_bytes,
                                                                   int panels, int stages, uint32_t* sink,
                                                                   uint32_t key) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[8][8192];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(blockIdx.x % panels) * 64u;
  const uint32_t cols = row_bytes / 128;
  const uint32_t lds0 = (uint32_t)(uintptr_t)&ring[0][0];
  uint32_t acc = 0;
  for (int s = 0; s < stages; ++s) {
    const uint32_t col = (uint32_t)s % cols;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t row = base + (uint32_t)(wave * 2 + i) * 8 + (lane >> 3);
      const uint32_t off = row * row_bytes + col * 128 + (lane & 7) * 16;
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(s & 7) * 8192 + (wave * 2 + i) * 1024);
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(src), "s"(m0v)
                   : "memory", "m0");
    }
    __builtin_amdgcn_s_waitcnt(12 | (7 << 4) | (15 << 8));  // vmcnt <= 12: six stages in flight
    if (MODE & 2) __syncthreads();
    if (MODE & 1) {
      const uint8_t* slot = &ring[(s + 2) & 7][(wave & 1) * 4096];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(slot + r * 1024 + lane * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  acc ^= *reinterpret_cast<const uint32_t*>(&ring[lane & 7][wave * 16]);
  if (acc == key) sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float* sink, uint32_t key) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // E4M3 codes of 0.5 and 0.25 with the lane folded into the low bits
    a[i] = 0x30303030 + (lane & 1);
    b[i] = 0x28282828 + ((lane >> 1) & 1);
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (__float_as_uint(s) == key) sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// LDS read rate: every lane reads 16 bytes per step (ds_read_b128), the 64
// lanes of a wave one contiguous 1 KB row of a 64 KB buffer (conflict-free),
// the row moving with the step and the wave; THREADS threads per workgroup.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void lds_read_kernel(int iters, uint32_t* sink, uint32_t key) {
  __shared__ __attribute__((aligned(16))) uint4 buf[4096];  // 64 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4096; i += THREADS) buf[i] = make_uint4(i, i ^ 0x55u, i + 7u, ~i);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint4 v = buf[(((it * 8 + u) * 5 + wave) & 63) * 64 + lane];
      acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
    }
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == key) sink[blockIdx.x * THREADS + tid] = r;
}

hipError_t launch_probe_lds(int iters, int threads, uint32_t* sink, int workgroups, hipStream_t stream) {
  if (threads == 512)
    hipLaunchKernelGGL(lds_read_kernel<512>, dim3((unsigned)workgroups), dim3(512), 0, stream, iters, sink,
                       0x9E3779B9u);
  else
    hipLaunchKernelGGL(lds_read_kernel<256>, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, sink,
                       0x9E3779B9u);
  return hipGetLastError();
}

// One pass over `bytes` in 1 KB pieces (a wave's 64 lanes x 16 bytes), piece
// i of workgroup w at (i * gridDim.x + w) * 1 KB... strided by wave: each
// wave of THREADS / 64 keeps U pieces in flight, into registers (DMA == 0)
// or into a U-slot LDS ring of its own by LDS-DMA (DMA == 1, waiting before a
// slot is reused). For the scaling of the read rate with waves per compute
// unit and copies in flight per wave.
template <int THREADS, int U, int DMA>
__global__ __launch_bounds__(THREADS) void wave_read_kernel(const uint8_t* src, int64_t pieces, uint32_t* sink,
                                                            uint32_t key) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  constexpr int NWV = THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * NWV;
  uint32_t acc = 0;
  int64_t p0 = (int64_t)blockIdx.x * NWV + wave;
  if constexpr (DMA == 0) {
    for (; p0 < pieces; p0 += stride * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t q = p0 + u * stride;
        q = q < pieces ? q : pieces - 1;
        v[u] = load16_nt(src + q * 1024 + lane * 16);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  } else {
    const uint32_t base = (uint32_t)(uintptr_t)ring + (uint32_t)wave * U * 1024;
    int slot = 0;
    for (; p0 < pieces; p0 += stride) {
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(base + (uint32_t)slot * 1024);
      const uint8_t* g = src + p0 * 1024 + lane * 16;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0v) : "memory", "m0");
      slot = slot + 1 == U ? 0 : slot + 1;
      // at most U - 1 of this wave's pieces in flight: the slot issued next
      // has landed
      __builtin_amdgcn_s_waitcnt(((U - 1) & 15) | (((U - 1) >> 4) << 14) | (7 << 4) | (15 << 8));
    }
    __builtin_amdgcn_s_waitcnt(0);
    acc = *reinterpret_cast<const uint32_t*>(ring + wave * U * 1024 + (lane & 15) * 16);
  }
  if (acc == key) sink[blockIdx.x * THREADS + threadIdx.x] = acc;
}

template <int THREADS, int U, int DMA>
hipError_t launch_wave_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  auto kern = wave_read_kernel<THREADS, U, DMA>;
  const size_t lds = DMA ? (size_t)(THREADS / 64) * U * 1024 : 0;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)workgroups), dim3(THREADS), lds, stream,
                     static_cast<const uint8_t*>(src), (int64_t)(bytes / 1024), sink, 0x9E3779B9u);
  return hipGetLastError();
}

hipError_t launch_probe_wave_read(const void* src, size_t bytes, int threads, int depth, int dma, uint32_t* sink,
                                  int workgroups, hipStream_t stream) {
#define FP8_WAVE_READ(T, U)                                                           \
  if (threads == T && depth == U)                                                     \
    return dma ? launch_wave_read<T, U, 1>(src, bytes, sink, workgroups, stream)      \
               : launch_wave_read<T, U, 0>(src, bytes, sink, workgroups, stream);
  FP8_WAVE_READ(256, 4) FP8_WAVE_READ(256, 8) FP8_WAVE_READ(256, 16)
  FP8_WAVE_READ(512, 4) FP8_WAVE_READ(512, 8) FP8_WAVE_READ(512, 16)
  FP8_WAVE_READ(1024, 4) FP8_WAVE_READ(1024, 8)
#undef FP8_WAVE_READ
  return hipErrorInvalidValue;
}

// One MFMA per wave on given operands, D = W X^T + C, in the operand layout
// the GEMM kernels use. FORM 0: V_MFMA_F32_16X16X128_F8F6F4, W and X [16][128]
// E4M3 codes, C and D [16][16] fp32 (element [n][m]: row n of W, row m of X);
// lane l supplies row l % 16 and the K bytes [32 (l / 16), +32) of both
// operands and owns D[4 (l / 16) + v][l % 16]. FORM 1:
// V_MFMA_F32_32X32X64_F8F6F4, W and X [32][64], C and D [32][32]; lane l
// supplies row l % 32 and K bytes [32 (l / 32), +32) and owns
// D[8 q + 4 (l / 32) + v][l % 32] in accumulator 4 q + v. Shows the matrix
// core's own rounding of an FP8 dot product and of its addition to C.
template <int FORM>
__global__ __launch_bounds__(64) void mfma_dot_probe_kernel(const uint8_t* w, const uint8_t* x, const float* c,
                                                            float* d) {
  constexpr int R = FORM == 0 ? 16 : 32, KD = FORM == 0 ? 128 : 64;
  const int lane = threadIdx.x, r = lane % R, g = lane / R;
  const size_t op = (size_t)blockIdx.x * R * KD, mat = (size_t)blockIdx.x * R * R;
  const uint4* wp = reinterpret_cast<const uint4*>(w + op + (size_t)r * KD + 32 * g);
  const uint4* xp = reinterpret_cast<const uint4*>(x + op + (size_t)r * KD + 32 * g);
  const uint4 w0 = wp[0], w1 = wp[1], x0 = xp[0], x1 = xp[1];
  i32x8 wv, xv;
  wv[0] = (int)w0.x; wv[1] = (int)w0.y; wv[2] = (int)w0.z; wv[3] = (int)w0.w;
  wv[4] = (int)w1.x; wv[5] = (int)w1.y; wv[6] = (int)w1.z; wv[7] = (int)w1.w;
  xv[0] = (int)x0.x; xv[1] = (int)x0.y; xv[2] = (int)x0.z; xv[3] = (int)x0.w;
  xv[4] = (int)x1.x; xv[5] = (int)x1.y; xv[6] = (int)x1.z; xv[7] = (int)x1.w;
  if constexpr (FORM == 0) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    f32x4v acc;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = c[mat + (size_t)(4 * g + v) * R + r];
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, xv, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) d[mat + (size_t)(4 * g + v) * R + r] = acc[v];
  } else {
    typedef float f32x16v __attribute__((ext_vector_type(16)));
    f32x16v acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = c[mat + (size_t)(8 * (i >> 2) + 4 * g + (i & 3)) * R + r];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, xv, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[mat + (size_t)(8 * (i >> 2) + 4 * g + (i & 3)) * R + r] = acc[i];
  }
}

hipError_t launch_probe_mfma_dot(const void* w, const void* x, const float* c, float* d, int count, int form,
                                 hipStream_t stream) {
  if (form == 0)
    hipLaunchKernelGGL(mfma_dot_probe_kernel<0>, dim3((unsigned)count), dim3(64), 0, stream,
                       static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(x), c, d);
  else
    hipLaunchKernelGGL(mfma_dot_probe_kernel<1>, dim3((unsigned)count), dim3(64), 0, stream,
                       static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(x), c, d);
  return hipGetLastError();
}

hipError_t launch_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint4*>(src), (int64_t)(bytes / 16), sink, 0x9E3779B9u);
  return hipGetLastError();
}

hipError_t launch_probe_strided_read(const void* src, int64_t rows, int64_t row_bytes, int rows_per_wg,
                                     int piece, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(strided_read_kernel, dim3((unsigned)(rows / rows_per_wg)), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint8_t*>(src), row_bytes, rows_per_wg, piece, sink, 0x9E3779B9u);
  return hipGetLastError();
}

hipError_t launch_probe_l2_feed(const void* src, size_t window, int reps, int dma, uint32_t* sink,
                                int workgroups, hipStream_t stream) {
  if (dma)
    hipLaunchKernelGGL(l2_feed_kernel<1>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint8_t*>(src), (int64_t)window, reps, sink, 0x9E3779B9u);
  else
    hipLaunchKernelGGL(l2_feed_kernel<0>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint8_t*>(src), (int64_t)window, reps, sink, 0x9E3779B9u);
  return hipGetLastError();
}

hipError_t launch_probe_panel_feed(const void* src, uint32_t row_bytes, int panels, int stages, int mode,
                                   uint32_t* sink, int workgroups, hipStream_t stream) {
  const uint8_t* b = static_cast<const uint8_t*>(src);
  const dim3 grid((unsigned)workgroups), block(kProbeThreads);
  switch (mode) {
    case 0: hipLaunchKernelGGL(panel_feed_kernel<0>, grid, block, 0, stream, b, row_bytes, panels, stages, sink, 0x9E3779B9u); break;
    case 1: hipLaunchKernelGGL(panel_feed_kernel<1>, grid, block, 0, stream, b, row_bytes, panels, stages, sink, 0x9E3779B9u); break;
    case 2: hipLaunchKernelGGL(panel_feed_kernel<2>, grid, block, 0, stream, b, row_bytes, panels, stages, sink, 0x9E3779B9u); break;
    default: hipLaunchKernelGGL(panel_feed_kernel<3>, grid, block, 0, stream, b, row_bytes, panels, stages, sink, 0x9E3779B9u); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, float* sink, int workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream, iters,
                     sink, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace fp8w8a8
