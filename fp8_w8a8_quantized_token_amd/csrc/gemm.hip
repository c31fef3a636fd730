// FP8 (OCP E4M3) scaled GEMM kernels for gfx950 (CDNA4).
//
// Channelwise (PR 34331 digest, "Tune FP8 GEMM Triton tiles on L40S and enable
// them by default", "Key source excerpts", apply_fp8_linear):
//   out[m,n] = bf16(a_scale[m] * b_scale[n] * sum_k A[m,k] B[n,k] + bias[n])
// Blockwise (PR 27896 digest, "Remove the per-call padding overhead of the FP8
// blockwise GEMM", "Key source excerpts"): one activation scale per (row,
// 128-wide K block) and one weight scale per 128x128 block,
//   out[m,n] = bf16(sum_kb a_scale[m,kb] b_scale[n/128,kb] sum_{k in kb} A B + bias[n])
//
// Both use V_MFMA_F32_16X16X128_F8F6F4 with E4M3 operands and fp32
// accumulators. One MFMA is exactly one 128-deep K block, so the blockwise
// kernel promotes each block's MFMA result into the fp32 accumulator with its
// scale product (one FMA per accumulator element per block).
//
// Operand roles: the weight fragment is the MFMA's first operand and the
// activation fragment the second, so the 16x16 result tile is out^T: lane l
// holds m = l % 16 and four consecutive n = 4*(l/16) + r, which makes the
// epilogue store 4 contiguous bf16 (8 bytes) per lane.
//
// K ordering inside an MFMA: lane group g = l/16 supplies 32 bytes of K for
// its row. The hardware pairs A and B bytes that sit in the same lane group
// and register slot, so any assignment of K bytes to (group, slot) that is the
// same for both operands yields the same dot product; the kernels give group g
// the bytes [32g, 32g + 32) of each 128-byte K block.
#include "common.h"
#include "kernels.h"

namespace fp8w8a8 {

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& w, const i32x8& x, const f32x4& c) {
  // format selectors 0/0 = E4M3 for both operands; zero scale operands select
  // the unscaled V_MFMA_F32_16X16X128_F8F6F4
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 join(const uint4& lo, const uint4& hi) {
  i32x8 r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Store the 4 outputs a lane owns: row m, columns n..n+3 (bf16).
template <int KIND>
__device__ __forceinline__ void store_out4(const GemmArgs& p, int64_t m, int64_t n, f32x4 v,
                                           float sa_m) {
  if (m >= p.M || n >= p.N) return;
  float o[4];
  if (n + 3 < p.N) {
    if (KIND == kChannelwise) {
      const float4 sb = *reinterpret_cast<const float4*>(p.sb + n);
      o[0] = v[0] * sa_m * sb.x; o[1] = v[1] * sa_m * sb.y;
      o[2] = v[2] * sa_m * sb.z; o[3] = v[3] * sa_m * sb.w;
    } else {
      o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    }
    if (p.bias) {
      const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
      o[0] += bf16_to_f32(bb.x & 0xffffu); o[1] += bf16_to_f32(bb.x >> 16);
      o[2] += bf16_to_f32(bb.y & 0xffffu); o[3] += bf16_to_f32(bb.y >> 16);
    }
    const uint2 packed = make_uint2(f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16),
                                    f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16));
    *reinterpret_cast<uint2*>(p.out + m * p.ldc + n) = packed;
  } else {
    for (int r = 0; r < 4 && n + r < p.N; ++r) {
      float x = v[r];
      if (KIND == kChannelwise) x = x * sa_m * p.sb[n + r];
      if (p.bias) x += bf16_to_f32(p.bias[n + r]);
      p.out[m * p.ldc + n + r] = (uint16_t)f32_to_bf16(x);
    }
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel: BM x BN block tile, 128-deep K steps, WM x WN waves, each wave
// a (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA tiles. A and B K-slices are
// staged through LDS, double buffered: global loads of step k+1 are issued
// into registers before the MFMAs of step k and written to the other LDS
// buffer after them, with one barrier per step. LDS rows are 128 bytes made of
// eight 16-byte chunks; chunk c of row r is stored at position c ^ (r & 7), so
// the 16 lanes that read one chunk column of 16 consecutive rows hit distinct
// bank groups.
// Split-K: blockIdx.y selects a K range; every split writes its fp32 partial
// tile to the workspace, and the last split to arrive (arrival counter per
// tile) sums the partials in split order -- deterministic -- applies the
// epilogue and re-arms the counter to zero.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int KIND>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 128;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int A_CH = BM * 8 / NT;
  constexpr int B_CH = BN * 8 / NT;
  static_assert(A_CH >= 1 && B_CH >= 1 && BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/threads");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const a_lds = lds;                  // [2][BM][128]
  uint8_t* const b_lds = lds + 2 * BM * BK;    // [2][BN][128]
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int split = blockIdx.y;
  const int64_t kt_all = (p.K + BK - 1) / BK;
  const int64_t kt_begin = (int64_t)split * p.k_tiles_per_split;
  int64_t kt_end = kt_begin + p.k_tiles_per_split;
  if (kt_end > kt_all) kt_end = kt_all;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[A_CH], rb[B_CH];
  float sa_nxt[TM], sb_nxt[TN];

  auto gload = [&](int64_t kt) {
    const int64_t k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      const int64_t gm = m0 + r, gk = k0 + c * 16;
      ra[i] = (gm < p.M && gk < p.K)
                  ? load16(p.a + gm * p.lda + gk)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      const int64_t gn = n0 + r, gk = k0 + c * 16;
      rb[i] = (gn < p.N && gk < p.K)
                  ? load16(p.b + gn * p.ldb + gk)
                  : make_uint4(0, 0, 0, 0);
    }
    if (KIND == kBlockwise) {
      const int64_t kb_all = p.K / BK;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WTM + i * 16 + (lane & 15);
        sa_nxt[i] = (m < p.M) ? p.sa[kt * p.sa_ld + m] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WTN + j * 16;
        sb_nxt[j] = (n < p.N) ? p.sb[(n / 128) * kb_all + kt] : 0.0f;
      }
    }
  };
  auto swrite = [&](int buf) {
    uint8_t* ab = a_lds + buf * BM * BK;
    uint8_t* bb = b_lds + buf * BN * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(ab + r * BK + ((c ^ (r & 7)) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id >> 3, c = id & 7;
      *reinterpret_cast<uint4*>(bb + r * BK + ((c ^ (r & 7)) << 4)) = rb[i];
    }
  };

  float sa_cur[TM], sb_cur[TN];
  if (kt_begin < kt_end) {
    gload(kt_begin);
    swrite(0);
  }
  __syncthreads();

  const int g = lane >> 4;
  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (int)((kt - kt_begin) & 1);
    const bool has_next = kt + 1 < kt_end;
    if (KIND == kBlockwise) {
#pragma unroll
      for (int i = 0; i < TM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
      for (int j = 0; j < TN; ++j) sb_cur[j] = sb_nxt[j];
    }
    if (has_next) gload(kt + 1);

    const uint8_t* ab = a_lds + buf * BM * BK;
    const uint8_t* bb = b_lds + buf * BN * BK;
    i32x8 af[TM], bf[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * 16 + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(ab + r * BK + (((2 * g) ^ (r & 7)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(ab + r * BK + (((2 * g + 1) ^ (r & 7)) << 4));
      af[i] = join(lo, hi);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = wn * WTN + j * 16 + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(bb + r * BK + (((2 * g) ^ (r & 7)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(bb + r * BK + (((2 * g + 1) ^ (r & 7)) << 4));
      bf[j] = join(lo, hi);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (KIND == kChannelwise) {
          acc[i][j] = mfma_fp8(bf[j], af[i], acc[i][j]);
        } else {
          const f32x4 t = mfma_fp8(bf[j], af[i], f32x4{0.f, 0.f, 0.f, 0.f});
          const float sc = sa_cur[i] * sb_cur[j];
          acc[i][j] += t * sc;
        }
      }

    if (has_next) swrite(buf ^ 1);
    __syncthreads();
  }

  if (p.split_k > 1) {
    // partial layout: [tile][split][TM*TN][NT] float4 (register order)
    f32x4* part = reinterpret_cast<f32x4*>(p.ws_part) +
                  ((tile * p.split_k) * (TM * TN)) * NT;
    f32x4* mine = part + (int64_t)split * (TM * TN) * NT;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mine[(i * TN + j) * NT + tid] = acc[i][j];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int old = atomicAdd(p.ws_count + tile, 1);
      last_flag = (old == p.split_k - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        f32x4 s = part[(i * TN + j) * NT + tid];
        for (int sp = 1; sp < p.split_k; ++sp) s += part[((int64_t)sp * TM * TN + i * TN + j) * NT + tid];
        acc[i][j] = s;
      }
    if (tid == 0) p.ws_count[tile] = 0;
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 16 + (lane & 15);
    const float sa_m = (KIND == kChannelwise && m < p.M) ? p.sa[m] : 1.0f;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 16 + 4 * g;
      store_out4<KIND>(p, m, n, acc[i][j], sa_m);
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny kernel for M <= 16*MT: the weight is read exactly once, straight into
// registers (no LDS staging: each weight byte feeds one MFMA). A workgroup owns
// one 16-wide column tile of the output; its W waves split K into 512-byte
// chunks (wave w takes chunks w, w+W, ...), each lane loading four 32-byte
// pieces of its weight row per chunk. The W partial 16x16 tiles are summed
// through LDS in wave order (deterministic) and wave 0 runs the epilogue.
// The activation rows (at most 32) stay cache-resident and are re-read per
// chunk; lanes whose row is >= M load nothing.
// ---------------------------------------------------------------------------
template <int MT, int W, int KIND>
__global__ __launch_bounds__(W * 64) void gemm_skinny_kernel(GemmArgs p) {
  __shared__ f32x4 red[W][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nrow = n0 + (lane & 15);
  const bool n_ok = nrow < p.N;
  const int64_t kc_all = (p.K + 511) / 512;
  const int64_t kb_all = p.K / 128;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* brow = p.b + nrow * p.ldb;
  for (int64_t kc = wave; kc < kc_all; kc += W) {
    uint4 bq[4][2];
    uint4 aq[MT][4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t off = kc * 512 + j * 128 + g * 32;
      const bool k0 = off < p.K, k1 = off + 16 < p.K;
      bq[j][0] = (n_ok && k0) ? load16_nt(brow + off)
                              : make_uint4(0, 0, 0, 0);
      bq[j][1] = (n_ok && k1) ? load16_nt(brow + off + 16)
                              : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int64_t m = t * 16 + (lane & 15);
        const bool m_ok = m < p.M;
        const uint8_t* arow = p.a + m * p.lda;
        aq[t][j][0] = (m_ok && k0) ? load16(arow + off) : make_uint4(0, 0, 0, 0);
        aq[t][j][1] = (m_ok && k1) ? load16(arow + off + 16) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8 bf = join(bq[j][0], bq[j][1]);
      if (KIND == kChannelwise) {
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = mfma_fp8(bf, join(aq[t][j][0], aq[t][j][1]), acc[t]);
      } else {
        const int64_t kb = kc * 4 + j;
        if (kb < kb_all) {
          const float sb = p.sb[(n0 / 128) * kb_all + kb];
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const int64_t m = t * 16 + (lane & 15);
            const float sa = (m < p.M) ? p.sa[kb * p.sa_ld + m] : 0.0f;
            const f32x4 r = mfma_fp8(bf, join(aq[t][j][0], aq[t][j][1]), f32x4{0.f, 0.f, 0.f, 0.f});
            acc[t] += r * (sa * sb);
          }
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    f32x4 s = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) s += red[w][t][lane];
    const int64_t m = t * 16 + (lane & 15);
    const float sa_m = (KIND == kChannelwise && m < p.M) ? p.sa[m] : 1.0f;
    store_out4<KIND>(p, m, n0 + 4 * g, s, sa_m);
  }
}

// ---------------------------------------------------------------------------
// Variant table and launch.
// ---------------------------------------------------------------------------
namespace {
constexpr int kSkinnyWaves = 8;

template <int BM, int BN, int WM, int WN, int KIND>
hipError_t launch_tile(const GemmArgs& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const size_t lds = (size_t)2 * (BM + BN) * 128;
  auto kern = gemm_tile_kernel<BM, BN, WM, WN, KIND>;
  static bool lds_attr_set = false;  // per instantiation; setting it twice is harmless
  if (lds > 65536 && !lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)p.split_k), dim3(WM * WN * 64), lds,
                     stream, p);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(int variant, const GemmArgs& p, hipStream_t stream) {
  switch (variant) {
    case 0: {  // FP8_VARIANT_SKINNY
      const dim3 grid((unsigned)((p.N + 15) / 16)), block(kSkinnyWaves * 64);
      if (p.M <= 16)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, kSkinnyWaves, KIND>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<2, kSkinnyWaves, KIND>), grid, block, 0, stream, p);
      return hipGetLastError();
    }
    case 1: return launch_tile<64, 64, 2, 2, KIND>(p, stream);
    case 2: return launch_tile<128, 128, 2, 2, KIND>(p, stream);
    case 3: return launch_tile<256, 128, 4, 2, KIND>(p, stream);
    case 4: return launch_tile<256, 256, 2, 4, KIND>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

VariantInfo variant_info(int variant) {
  switch (variant) {
    case 0: return {32, 16, 512, kSkinnyWaves, true};
    case 1: return {64, 64, 128, 4, true};
    case 2: return {128, 128, 128, 4, true};
    case 3: return {256, 128, 128, 8, true};
    case 4: return {256, 256, 128, 8, true};
    default: return {0, 0, 0, 0, false};
  }
}

int64_t variant_tiles(int variant, int64_t M, int64_t N) {
  const VariantInfo v = variant_info(variant);
  if (!v.exists) return 0;
  if (variant == 0) return (N + 15) / 16;
  return ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
}

size_t variant_workspace_bytes(int variant, int split_k, int64_t M, int64_t N) {
  if (split_k <= 1 || variant == 0) return 0;
  const VariantInfo v = variant_info(variant);
  const int64_t tiles = variant_tiles(variant, M, N);
  return kCounterBytes + (size_t)tiles * split_k * v.bm * v.bn * sizeof(float);
}

hipError_t launch_gemm(int kind, int variant, const GemmArgs& p, hipStream_t stream) {
  return kind == kChannelwise ? launch_kind<kChannelwise>(variant, p, stream)
                              : launch_kind<kBlockwise>(variant, p, stream);
}

}  // namespace fp8w8a8
