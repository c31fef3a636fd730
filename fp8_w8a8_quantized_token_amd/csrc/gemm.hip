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
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace fp8w8a8 {

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& w, const i32x8& x, const f32x4& c) {
  // format selectors 0/0 = E4M3 for both operands; zero scale operands select
  // the unscaled V_MFMA_F32_16X16X128_F8F6F4
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}

// The same with E8M0 block scales applied by the matrix core (gfx950's
// block-scaled MFMA): every product is multiplied by 2^(ew - 127) 2^(ex - 127),
// ew the exponent of the first operand's row (the weight row n), ex that of the
// second's (the activation row m). Each lane passes, in the low byte, the
// exponent for its row and the 32-deep K piece it supplies (lane group l / 16);
// with one scale per 128-deep block all four pieces of a row pass the same one.
__device__ __forceinline__ f32x4 mfma_fp8_e8(const i32x8& w, const i32x8& x, const f32x4& c, int ew,
                                             int ex) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, ew, 0, ex);
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
    const uint2 packed = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    *reinterpret_cast<uint2*>(p.out + m * p.ldc + n) = packed;
  } else {
    for (int r = 0; r < 4 && n + r < p.N; ++r) {
      float x = v[r];
      if (KIND == kChannelwise) x = x * sa_m * p.sb[n + r];
      if (p.bias) x += bf16_to_f32(p.bias[n + r]);
      p.out[m * p.ldc + n + r] = (uint16_t)pack_bf16x2(x, 0.0f);
    }
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// pack_out4 (below) with the weight scales of columns n..n+3 passed in
// (channelwise; columns >= N give unspecified values).
template <int KIND>
__device__ __forceinline__ uint2 pack_out4s(const GemmArgs& p, int64_t n, f32x4 v, float sa_m, float4 sb) {
  float o[4] = {v[0], v[1], v[2], v[3]};
  if (KIND == kChannelwise) {
    o[0] = o[0] * sa_m * sb.x; o[1] = o[1] * sa_m * sb.y;
    o[2] = o[2] * sa_m * sb.z; o[3] = o[3] * sa_m * sb.w;
  }
  if (p.bias) {
    if (n + 3 < p.N) {
      const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
      o[0] += bf16_to_f32(bb.x & 0xffffu); o[1] += bf16_to_f32(bb.x >> 16);
      o[2] += bf16_to_f32(bb.y & 0xffffu); o[3] += bf16_to_f32(bb.y >> 16);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < p.N) o[r] += bf16_to_f32(p.bias[n + r]);
    }
  }
  return make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}

// Scale (channelwise), add the bias and round to bf16 the 4 outputs a lane
// owns at columns n..n+3 of row m; columns >= N give unspecified values.
template <int KIND>
__device__ __forceinline__ uint2 pack_out4(const GemmArgs& p, int64_t n, f32x4 v, float sa_m) {
  float o[4] = {v[0], v[1], v[2], v[3]};
  if (n + 3 < p.N) {
    if (KIND == kChannelwise) {
      const float4 sb = *reinterpret_cast<const float4*>(p.sb + n);
      o[0] = o[0] * sa_m * sb.x; o[1] = o[1] * sa_m * sb.y;
      o[2] = o[2] * sa_m * sb.z; o[3] = o[3] * sa_m * sb.w;
    }
    if (p.bias) {
      const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
      o[0] += bf16_to_f32(bb.x & 0xffffu); o[1] += bf16_to_f32(bb.x >> 16);
      o[2] += bf16_to_f32(bb.y & 0xffffu); o[3] += bf16_to_f32(bb.y >> 16);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (n + r < p.N) {
        if (KIND == kChannelwise) o[r] = o[r] * sa_m * p.sb[n + r];
        if (p.bias) o[r] += bf16_to_f32(p.bias[n + r]);
      }
    }
  }
  return make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}

// Epilogue of the 32x32-MFMA tile kernels, staged through LDS so that the
// output leaves in whole rows. Each lane packs its 4-column groups (the out^T
// layout: row m = l % 32, columns 8q + 4h .. +3 in registers 4q .. 4q+3) into
// a [BM][BN] bf16 tile in LDS, whose 16-byte chunk c of row r sits at
// c ^ sw(r); then consecutive threads copy consecutive 16-byte chunks of a
// row to global memory. Stored straight from the MFMA layout, one store
// instruction covered 32 rows 16 bytes each and the output went out at a
// fraction of the write bandwidth. sw(r) = r % CH for rows of 256 bytes or
// more, (r / 2) % 8 for 128-byte rows, (r / 4) % 4 for 64-byte rows:
// conflict-free for both phases. The LDS
// must hold BM * BN * 2 bytes; the function begins with a barrier, so the
// caller may still be reading it.
template <int CH>
__device__ __forceinline__ int out_sw(int r) {
  static_assert(CH == 4 || CH == 8 || CH == 16 || CH == 32, "tile width");
  return CH >= 16 ? (r & (CH - 1)) : CH == 8 ? ((r >> 1) & (CH - 1)) : ((r >> 2) & (CH - 1));
}

// Second phase of the staged epilogue: consecutive threads copy consecutive
// 16-byte chunks of the [BM][BN] bf16 tile in LDS to rows < M, columns < N.
// A tile wholly inside the output takes a branch-free form: a thread's
// chunks lie NT / CH rows apart, and each batch of them is read from LDS
// before any is stored, so the LDS round trips overlap.
template <int BM, int BN, int NT>
__device__ __forceinline__ void copy_out_tile(const GemmArgs& p, const uint8_t* lds, int64_t m0,
                                              int64_t n0, int tid) {
  constexpr int CH = BN / 8;
  static_assert((BM * CH) % NT == 0 && NT % CH == 0, "copy-out split");
  if (m0 + BM <= p.M && n0 + BN <= p.N) {
    constexpr int IT = BM * CH / NT;  // chunks per thread
    constexpr int RSTEP = NT / CH;    // rows between them
    constexpr int BATCH = IT < 8 ? IT : 8;
    const int rl0 = tid / CH, c = tid % CH;
    uint16_t* dst = p.out + (m0 + rl0) * p.ldc + n0 + c * 8;
    const int64_t step = (int64_t)RSTEP * p.ldc;
#pragma unroll
    for (int i0 = 0; i0 < IT; i0 += BATCH) {
      uint4 v[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int rl = rl0 + (i0 + b) * RSTEP;
        v[b] = *reinterpret_cast<const uint4*>(lds + rl * (BN * 2) + ((c ^ out_sw<CH>(rl)) << 4));
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) *reinterpret_cast<uint4*>(dst + (i0 + b) * step) = v[b];
    }
    return;
  }
#pragma unroll 4
  for (int idx = tid; idx < BM * CH; idx += NT) {
    const int rl = idx / CH, c = idx % CH;
    const int64_t m = m0 + rl;
    const int64_t n = n0 + c * 8;
    if (m >= p.M || n >= p.N) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + rl * (BN * 2) + ((c ^ out_sw<CH>(rl)) << 4));
    uint16_t* dst = p.out + m * p.ldc + n;
    if (n + 8 <= p.N) {
      *reinterpret_cast<uint4*>(dst) = v;
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (n + r < p.N) dst[r] = (uint16_t)(w[r >> 1] >> (16 * (r & 1)));
    }
  }
}

// The same epilogue for 16x16-MFMA accumulators (lane: m = 16 i + l % 16,
// n = 16 j + 4 (l / 16) .. +3). Blockwise results are already scaled;
// channelwise ones take the tile's BM activation and BN weight scales from
// the fp32 table at byte sc_off of the LDS (staged by the caller while the
// K loop ran: scale loads issued here would wait a full memory round trip
// under the output stores of every other workgroup).
template <int BM, int BN, int WM, int WN, int KIND>
__device__ __forceinline__ void store_tile16(const GemmArgs& p,
                                             const f32x4 (&acc)[BM / WM / 16][BN / WN / 16],
                                             uint8_t* lds, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, int tid, int sc_off) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int CH = BN / 8;
  __syncthreads();
  const float* lsa = reinterpret_cast<const float*>(lds + sc_off);
  const float* lsb = lsa + BM;
#pragma unroll
  for (int i = 0; i < WTM / 16; ++i) {
    const int ml = wm * WTM + i * 16 + (lane & 15);
    const float sa_m = KIND == kChannelwise ? lsa[ml] : 1.0f;
    uint8_t* row = lds + ml * (BN * 2);
#pragma unroll
    for (int j = 0; j < WTN / 16; ++j) {
      const int nl = wn * WTN + j * 16 + 4 * (lane >> 4);
      const uint2 v = pack_out4s<KIND>(p, n0 + nl, acc[i][j], sa_m,
                                       KIND == kChannelwise ? *reinterpret_cast<const float4*>(lsb + nl)
                                                            : float4{1.f, 1.f, 1.f, 1.f});
      *reinterpret_cast<uint2*>(row + (((nl >> 3) ^ out_sw<CH>(ml)) << 4) + (((nl >> 2) & 1) << 3)) = v;
    }
  }
  __syncthreads();
  copy_out_tile<BM, BN, NT>(p, lds, m0, n0, tid);
}

// sc_off >= 0 (channelwise): the tile's scales come from the fp32 table at
// that LDS byte offset (BM activation scales, then BN weight scales), as in
// store_tile16; otherwise from global memory.
template <int BM, int BN, int WM, int WN, int KIND>
__device__ __forceinline__ void store_tile(const GemmArgs& p,
                                           const f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
                                           uint8_t* lds, int64_t m0, int64_t n0, int wm, int wn,
                                           int h, int r32, int tid, int sc_off = -1) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int CH = BN / 8;  // 16-byte chunks per tile row
  auto sw = [](int r) { return out_sw<CH>(r); };
  __syncthreads();
  const bool ls = KIND == kChannelwise && sc_off >= 0;
  const float* lsa = reinterpret_cast<const float*>(lds + (sc_off > 0 ? sc_off : 0));
  const float* lsb = lsa + BM;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int ml = wm * WTM + i * 32 + r32;
    const int64_t m = m0 + ml;
    const float sa_m = ls ? lsa[ml] : (KIND == kChannelwise && m < p.M) ? p.sa[m] : 1.0f;
    uint8_t* row = lds + ml * (BN * 2);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * WTN + j * 32 + 8 * q + 4 * h;
        const f32x4 v4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        const uint2 v = ls ? pack_out4s<KIND>(p, n0 + nl, v4, sa_m, *reinterpret_cast<const float4*>(lsb + nl))
                           : pack_out4<KIND>(p, n0 + nl, v4, sa_m);
        *reinterpret_cast<uint2*>(row + (((nl >> 3) ^ sw(ml)) << 4) + (h << 3)) = v;
      }
  }
  __syncthreads();
  copy_out_tile<BM, BN, NT>(p, lds, m0, n0, tid);
}

// ---------------------------------------------------------------------------
// Tiled kernel: BM x BN block tile, 128-byte K stages, WM x WN waves, each wave
// a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA tiles (V_MFMA_F32_32X32X64_F8F6F4,
// two per stage). A and B stages are staged through LDS, double buffered:
// global loads of stage s+1 are issued into registers before the MFMAs of
// stage s and written to the other LDS buffer after them, one barrier per
// stage. LDS rows are 128 bytes of eight 16-byte chunks placed by swz().
// MFMA operand layout: lane l holds row l % 32 and, for the 64-byte K step s
// of the stage, bytes [64s + 32h, 64s + 32h + 32) with h = l / 32 (the same
// assignment for both operands). The weight is the first operand, so the
// 32x32 result is out^T: lane l holds m = l % 32 and, in register r,
// n = 8*(r/4) + 4*(l/32) + r%4 -- four consecutive n per register quad.
// Split-K: blockIdx.y selects a K range; every split writes its fp32 partial
// tile to the workspace with agent-coherent stores, and the last split to
// arrive (arrival counter per tile) sums the partials in split order --
// deterministic -- applies the epilogue and re-arms the counter to zero.
// ---------------------------------------------------------------------------

// Physical 16-byte chunk position of logical chunk c in an LDS row r of CH
// chunks. For 128-byte rows (CH = 8) the xor key (r & 7) ^ ((r >> 3) & 1)
// gives every 8 consecutive rows distinct positions (32 banks serve 8 lanes
// of a 128-bit access per cycle) and every 16 consecutive rows distinct (row
// parity, position) pairs (64 banks serve 16 lanes per cycle). Rows of 256
// bytes or more start on the same bank, so the key is r & 15, distinct over 16
// consecutive rows. Either way fragment reads of one chunk column and
// row-wise stores are free of bank conflicts.
template <int CH>
__device__ __forceinline__ int swz(int r, int c) {
  if (CH == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
  return c ^ (r & 15);
}

// Output-tile order: workgroups are dealt round-robin to the 8 XCDs (each with
// its own L2), so consecutive workgroup ids are re-mapped to give every XCD a
// contiguous range of tiles, and tiles are walked in groups of GM tile rows,
// column by column inside a group, so the tiles resident on one XCD at a time
// share A row panels and B column panels in its L2.
__device__ __forceinline__ void tile_coords(int64_t id, int64_t tiles_m, int64_t tiles_n,
                                            int64_t* tm, int64_t* tn) {
  constexpr int64_t kXcd = 8, GM = 4;
  const int64_t total = tiles_m * tiles_n;
  int64_t t = id;
  if (total % kXcd == 0) t = (id % kXcd) * (total / kXcd) + id / kXcd;
  const int64_t per_group = GM * tiles_n;
  const int64_t group = t / per_group;
  const int64_t first = group * GM;
  const int64_t gm = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int64_t in = t - group * per_group;
  *tm = first + in % gm;
  *tn = in / gm;
}

__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& w, const i32x8& x, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, 0, 0, 0);
}

// The 32x32x64 form with E8M0 block scales applied by the matrix core (as
// mfma_fp8_e8): lane l passes the exponent of its row (l % 32) for the 32-deep
// K piece it supplies (l / 32).
__device__ __forceinline__ f32x16 mfma32_fp8_e8(const i32x8& w, const i32x8& x, const f32x16& c, int ew,
                                                int ex) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, c, 0, 0, 0, ew, 0, ex);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Fence-free deterministic split-K, shared by the tiled kernels: every split
// stores its partial tile to the workspace with device-coherent stores (the
// SC1 cache-policy bit that agent-scope atomics also use, here on dwordx4
// buffer stores, so the data reaches the device coherence point and no
// L2-wide write-back or invalidate fence is needed between XCDs), the
// workgroup drains its stores and counts itself in with one atomic; the last
// to arrive reads the partials back with device-coherent loads, sums them in
// split order into acc, re-arms the counter and returns true. The others
// return false and must exit. *flag is workgroup-shared scratch.
// Workspace layout of one tile: [split][piece][thread] 16-byte pieces, so each
// wave's store or load covers 1 KB contiguously.
namespace {
constexpr int kBufDword3 = 0x00020000;  // gfx9 raw buffer: 32-bit dwords, no format conversion
constexpr int kCacheSc1 = 16;           // cache policy: device-coherent (SC1)
}  // namespace

template <int TM, int TN, int NT, typename V>
__device__ __forceinline__ bool splitk_reduce(const GemmArgs& p, V (&acc)[TM][TN],
                                              int64_t tile, int split, int tid, int* flag) {
  constexpr int VW = sizeof(V) / sizeof(float);  // 16 (32x32 tiles) or 4 (16x16)
  static_assert(VW % 4 == 0, "whole 16-byte pieces");
  constexpr int PV = VW / 4;                     // pieces per accumulator register group
  constexpr int Q4 = TM * TN * PV;               // pieces per thread
  constexpr uint32_t SPLIT_BYTES = (uint32_t)Q4 * NT * 16;
  float* part = p.ws_part + (tile * p.split_k) * (int64_t)Q4 * 4 * NT;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(part, 0, (int)(SPLIT_BYTES * (uint32_t)p.split_k), kBufDword3);
  using v4i = int __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int c = 0; c < PV; ++c) {
        const v4i v = {__float_as_int(acc[i][j][4 * c]), __float_as_int(acc[i][j][4 * c + 1]),
                       __float_as_int(acc[i][j][4 * c + 2]), __float_as_int(acc[i][j][4 * c + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, (uint32_t)(((i * TN + j) * PV + c) * NT + tid) * 16,
                                               (uint32_t)split * SPLIT_BYTES, kCacheSc1);
      }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(p.ws_count + tile, 1);
    *flag = (old == p.split_k - 1);
  }
  __syncthreads();
  if (!*flag) return false;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int c = 0; c < PV; ++c) {
        const uint32_t off = (uint32_t)(((i * TN + j) * PV + c) * NT + tid) * 16;
        v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCacheSc1);
        float s0 = __int_as_float(v.x), s1 = __int_as_float(v.y), s2 = __int_as_float(v.z),
              s3 = __int_as_float(v.w);
        for (int sp = 1; sp < p.split_k; ++sp) {
          v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, (uint32_t)sp * SPLIT_BYTES, kCacheSc1);
          s0 += __int_as_float(v.x);
          s1 += __int_as_float(v.y);
          s2 += __int_as_float(v.z);
          s3 += __int_as_float(v.w);
        }
        acc[i][j][4 * c] = s0;
        acc[i][j][4 * c + 1] = s1;
        acc[i][j][4 * c + 2] = s2;
        acc[i][j][4 * c + 3] = s3;
      }
  if (tid == 0) __hip_atomic_store(p.ws_count + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

template <int BM, int BN, int WM, int WN, int BK, int KIND>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int CH = BK / 16;          // 16-byte chunks per LDS row
  constexpr int KS = BK / 64;          // 64-deep MFMA steps per stage
  constexpr int KB = BK / 128;         // 128-wide scale blocks per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_CH = BM * CH / NT;
  constexpr int B_CH = BN * CH / NT;
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(A_CH >= 1 && B_CH >= 1 && BM * CH % NT == 0 && BN * CH % NT == 0, "tile/threads");
  static_assert(BK == 128 || BK == 256 || BK == 512, "stage depth");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const a_lds = lds;                  // [2][BM][BK]
  uint8_t* const b_lds = lds + 2 * BM * BK;    // [2][BN][BK]
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tile = blockIdx.x;
  int64_t tile_m, tile_n;
  tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  const int64_t m0 = tile_m * BM;
  const int64_t n0 = tile_n * BN;
  const int split = blockIdx.y;
  // this split's K range, in BK-deep stages (the host plans splits in stages)
  const int64_t kt_all = (p.K + BK - 1) / BK;
  const int64_t kt_begin = (int64_t)split * p.k_tiles_per_split;
  int64_t kt_end = kt_begin + p.k_tiles_per_split;
  if (kt_end > kt_all) kt_end = kt_all;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero16();

  uint4 ra[A_CH], rb[B_CH];
  float sa_nxt[KB][TM], sb_nxt[KB][TN];

  auto gload = [&](int64_t kt) {
    const int64_t k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id / CH, c = id % CH;
      const int64_t gm = m0 + r, gk = k0 + c * 16;
      ra[i] = (gm < p.M && gk < p.K) ? load16(p.a + gm * p.lda + gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id / CH, c = id % CH;
      const int64_t gn = n0 + r, gk = k0 + c * 16;
      rb[i] = (gn < p.N && gk < p.K) ? load16(p.b + gn * p.ldb + gk) : make_uint4(0, 0, 0, 0);
    }
    if (KIND == kBlockwise) {
      const int64_t kb_all = p.K / 128;
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const int64_t kb = kt * KB + b;
        const bool kb_ok = kb < kb_all;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int64_t m = m0 + wm * WTM + i * 32 + r32;
          sa_nxt[b][i] = (kb_ok && m < p.M) ? p.sa[kb * p.sa_ld + m] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t n = n0 + wn * WTN + j * 32;
          sb_nxt[b][j] = (kb_ok && n < p.N) ? p.sb[(n / 128) * kb_all + kb] : 0.0f;
        }
      }
    }
  };
  auto swrite = [&](int buf) {
    uint8_t* ab = a_lds + buf * BM * BK;
    uint8_t* bb = b_lds + buf * BN * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id / CH, c = id % CH;
      *reinterpret_cast<uint4*>(ab + r * BK + (swz<CH>(r, c) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int id = tid + i * NT;
      const int r = id / CH, c = id % CH;
      *reinterpret_cast<uint4*>(bb + r * BK + (swz<CH>(r, c) << 4)) = rb[i];
    }
  };
  // operand fragment of row r for 64-deep step s: chunks 4s+2h and 4s+2h+1
  auto frag = [&](const uint8_t* base, int r, int s) {
    const uint8_t* row = base + r * BK;
    const int c0 = 4 * s + 2 * h;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (swz<CH>(r, c0) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (swz<CH>(r, c0 + 1) << 4));
    return join(lo, hi);
  };

  float sa_cur[KB][TM], sb_cur[KB][TN];
  if (kt_begin < kt_end) {
    gload(kt_begin);
    swrite(0);
  }
  __syncthreads();

  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (int)((kt - kt_begin) & 1);
    const bool has_next = kt + 1 < kt_end;
    if (KIND == kBlockwise) {
#pragma unroll
      for (int b = 0; b < KB; ++b) {
#pragma unroll
        for (int i = 0; i < TM; ++i) sa_cur[b][i] = sa_nxt[b][i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb_cur[b][j] = sb_nxt[b][j];
      }
    }
    if (has_next) gload(kt + 1);

    const uint8_t* ab = a_lds + buf * BM * BK;
    const uint8_t* bb = b_lds + buf * BN * BK;
    if (KIND == kChannelwise) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        i32x8 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = frag(ab, wm * WTM + i * 32 + r32, s);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = frag(bb, wn * WTN + j * 32 + r32, s);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma32_fp8(bf[j], af[i], acc[i][j]);
      }
    } else {
      // each 128-deep K block's partial product is scaled before it joins
      // the accumulator
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        i32x8 af0[TM], af1[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          af0[i] = frag(ab, wm * WTM + i * 32 + r32, 2 * b);
          af1[i] = frag(ab, wm * WTM + i * 32 + r32, 2 * b + 1);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const i32x8 bf0 = frag(bb, wn * WTN + j * 32 + r32, 2 * b);
          const i32x8 bf1 = frag(bb, wn * WTN + j * 32 + r32, 2 * b + 1);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            f32x16 t = mfma32_fp8(bf0, af0[i], zero16());
            t = mfma32_fp8(bf1, af1[i], t);
            const float sc = sa_cur[b][i] * sb_cur[b][j];
            acc[i][j] += t * sc;
          }
        }
      }
    }

    if (has_next) swrite(buf ^ 1);
    __syncthreads();
  }

  if (p.split_k > 1 && !splitk_reduce<TM, TN, NT>(p, acc, tile, split, tid, &last_flag)) return;

  static_assert(BM * BN * 2 <= 2 * (BM + BN) * BK, "output tile fits the LDS stages");
  store_tile<BM, BN, WM, WN, KIND>(p, acc, lds, m0, n0, wm, wn, h, r32, tid);
}

// ---------------------------------------------------------------------------
// Deep-pipeline tiled kernel (channelwise): BM x BN block tile, 64-byte K
// stages, WM x WN waves with 32x32 MFMA tiles as above. Global -> LDS copies
// use the LDS-DMA form of the 16-byte global load (global_load_lds_dwordx4:
// each lane's 16 bytes land at M0 + 16*lane, no registers involved), so
// NSTAGE LDS stages can be in flight at once: while stage s is multiplied,
// stages s+1 .. s+NSTAGE-1 are loading. Each wave issues exactly
// (BM + BN) / 16 / waves such loads per stage; before the barrier that
// publishes stage s a wave waits until its own outstanding loads are only
// those of the later stages (vmcnt counts in issue order), and the barrier
// then also guarantees every wave has finished multiplying stage s-1, whose
// buffer the next loads overwrite.
// The loads are written as inline assembly because the compiler, unable to
// tell which LDS stage a read depends on, would otherwise wait for every
// outstanding LDS-DMA load before each LDS read and serialize the pipeline;
// waits the compiler inserts for its own loads count these too and can only
// wait longer, never shorter.
// LDS rows are 64 bytes (four 16-byte chunks); chunk c of row r sits at
// position c ^ ((r >> 2) & 3), which gives the 16 lanes of one fragment read
// (16 consecutive rows, one chunk column) 16 distinct 16-byte bank groups.
// A DMA instruction covers 16 rows x 64 bytes, so lane i fetches the global
// chunk that belongs at LDS position i. Rows at or beyond M (or N) fetch a
// valid row instead (their outputs are never stored); K must be a multiple
// of 64 (the host falls back to the register-staged kernel otherwise).
// ---------------------------------------------------------------------------
// M0 carries the (wave-uniform) LDS destination; no other instruction of these
// kernels reads M0 (gfx9-class LDS instructions do not use it).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0v)
               : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset: one VGPR per stream instead of a 64-bit pointer.
__device__ __forceinline__ void lds_dma16_s(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
               : "memory", "m0");
}

// The 4-byte form from a per-lane 64-bit address: lane l's 4 bytes land at
// M0 + 4 l (gathers from several arrays in one instruction).
__device__ __forceinline__ void lds_dma4_v(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(m0v) : "memory", "m0");
}

// The 4-byte form: each lane's 4 bytes land at M0 + 4 * lane.
__device__ __forceinline__ void lds_dma4_s(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0v)
               : "memory", "m0");
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

// s_waitcnt with vmcnt = N and the other counters unconstrained (gfx9 layout:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same, and every LDS read of this wave complete (lgkmcnt = 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ int swz64(int r, int c) { return c ^ ((r >> 2) & 3); }

template <int BM, int BN, int WM, int WN, int NSTAGE>
__global__ __launch_bounds__(WM * WN * 64) void gemm_dma_kernel(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int NW = WM * WN;
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int A_BLK = BM / 16, B_BLK = BN / 16;        // 1 KB DMA blocks per stage
  constexpr int A_PER = A_BLK / NW, B_PER = B_BLK / NW;  // per wave
  constexpr int PER_WAVE = A_PER + B_PER;
  constexpr int STAGE_BYTES = (BM + BN) * BK;
  static_assert(A_BLK % NW == 0 && B_BLK % NW == 0, "DMA blocks per wave");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "stages");
  static_assert(PER_WAVE * NSTAGE < 64, "vmcnt range");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int last_flag;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tile = blockIdx.x;
  int64_t tile_m, tile_n;
  tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  const int64_t m0 = tile_m * BM;
  const int64_t n0 = tile_n * BN;
  const int split = blockIdx.y;
  const int64_t kt_all = p.K / BK;
  const int64_t kt_begin = (int64_t)split * p.k_tiles_per_split;
  int64_t kt_end = kt_begin + p.k_tiles_per_split;
  if (kt_end > kt_all) kt_end = kt_all;

  // per-lane byte offsets of this wave's DMA rows (clamped into the matrix;
  // the launcher guarantees they fit in 32 bits)
  const int lrow = lane >> 2, lpos = lane & 3;
  uint32_t a_off[A_PER], b_off[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int r = (wave * A_PER + i) * 16 + lrow;
    int64_t gm = m0 + r;
    if (gm >= p.M) gm = p.M - 1;
    a_off[i] = (uint32_t)(gm * p.lda + swz64(r, lpos) * 16);  // logical chunk at position lpos
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int r = (wave * B_PER + i) * 16 + lrow;
    int64_t gn = n0 + r;
    if (gn >= p.N) gn = p.N - 1;
    b_off[i] = (uint32_t)(gn * p.ldb + swz64(r, lpos) * 16);
  }
  auto slot = [&](int64_t kt) { return (int)((kt - kt_begin) % NSTAGE); };
  auto issue = [&](int64_t kt) {
    const uint32_t a_base = lds_base + slot(kt) * STAGE_BYTES;
    const uint32_t b_base = a_base + BM * BK;
    const uint8_t* ak = p.a + kt * BK;
    const uint8_t* bk = p.b + kt * BK;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) lds_dma16_s(ak, a_off[i], a_base + (wave * A_PER + i) * 1024);
#pragma unroll
    for (int i = 0; i < B_PER; ++i) lds_dma16_s(bk, b_off[i], b_base + (wave * B_PER + i) * 1024);
  };
  auto frag = [&](const uint8_t* base, int r) {
    const uint8_t* row = base + r * BK;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + (swz64(r, 2 * h) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(row + (swz64(r, 2 * h + 1) << 4));
    return join(lo, hi);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero16();

  // Pipeline: stage kt's fragments are in registers while its MFMAs run. The
  // B fragments of stage kt+1 go to a second register set; each A fragment of
  // kt+1 is read into the registers of kt's A fragment as soon as kt's MFMAs
  // on it have issued (128 accumulators plus fragments fit the 256 registers
  // of a wave at two waves per SIMD). The ring slot of stage kt is free once
  // its fragments are in registers, so stage kt+NSTAGE is issued into it,
  // keeping NSTAGE-1 stages of DMA in flight behind the one being read.
  i32x8 fa[TM], fb0[TN], fb1[TN];
  for (int q = 0; q < NSTAGE; ++q)
    if (kt_begin + q < kt_end) issue(kt_begin + q);
  if (kt_begin < kt_end) {
    const int64_t issued_after = kt_end - 1 - kt_begin;  // stages issued after the first
    if (issued_after >= NSTAGE - 1) wait_vmcnt<(NSTAGE - 1) * PER_WAVE>();
    else if (issued_after == 2) wait_vmcnt<2 * PER_WAVE>();
    else if (issued_after == 1) wait_vmcnt<PER_WAVE>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const uint8_t* ab = lds + slot(kt_begin) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = frag(ab, wm * WTM + i * 32 + r32);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb0[j] = frag(ab + BM * BK, wn * WTN + j * 32 + r32);
  }
  // One stage with a successor. Every path reaches the barrier with
  // lgkmcnt = 0, so the MFMAs never wait on the reads issued beside them.
  auto step_read = [&](int64_t kt, const i32x8 (&bc)[TN], i32x8 (&bn)[TN]) {
    const int64_t later = kt_end - 2 - kt;  // stages issued after kt+1 so far
    if (later >= NSTAGE - 2) wait_vmcnt<(NSTAGE - 2) * PER_WAVE>();
    else if (later == 1) wait_vmcnt<PER_WAVE>();
    else wait_vmcnt<0>();
    wait_vmcnt_lgkm0<63>();
    __builtin_amdgcn_s_barrier();
    if (kt + NSTAGE < kt_end) issue(kt + NSTAGE);
    const uint8_t* ab = lds + slot(kt + 1) * STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < TN; ++j) bn[j] = frag(ab + BM * BK, wn * WTN + j * 32 + r32);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32_fp8(bc[j], fa[i], acc[i][j]);
      fa[i] = frag(ab, wm * WTM + i * 32 + r32);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TN, 0);  // B reads of kt+1
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);  // MFMAs on A fragment i
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // A fragment i of kt+1
    }
  };
  auto step_last = [&](const i32x8 (&bc)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32_fp8(bc[j], fa[i], acc[i][j]);
  };
  for (int64_t kt = kt_begin; kt + 1 < kt_end; ++kt) {
    step_read(kt, fb0, fb1);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb0[j] = fb1[j];
  }
  if (kt_begin < kt_end) step_last(fb0);

  if (p.split_k > 1 && !splitk_reduce<TM, TN, NT>(p, acc, tile, split, tid, &last_flag)) return;

  static_assert(BM * BN * 2 <= NSTAGE * STAGE_BYTES, "output tile fits the LDS ring");
  store_tile<BM, BN, WM, WN, kChannelwise>(p, acc, lds, m0, n0, wm, wn, h, r32, tid);
}

// ---------------------------------------------------------------------------
// Panel-ring kernel (K % 128 == 0): BM x BN block tile, 128-byte K stages,
// WM x WN waves of 32x32 MFMA tiles as above. A stage is two panels -- its
// B (weight) rows, then its A rows, 128 bytes each, in the 128-byte row
// layout of the tiled kernel (swz<8>) -- and panel q (stage q/2, A if q is
// odd) lives in slot q % NP of an NP-slot LDS ring. The weight panel goes
// first because it comes from HBM while the activation panel is mostly an L2
// hit: with the order the refill below implies, the first panel of a stage
// is issued two stages before it is needed and the second one stage before,
// and this order measured up to 1.45x faster for the small tiles. One
// LDS-DMA instruction moves 8 whole 128-byte row pieces, one cache line per
// row: measured on MI355X with every CU streaming, that feeds a CU about
// 1.45x faster from L2 than the 16 half-line pieces of the 64-byte-stage
// kernel, which bounds that kernel at large M. The MFMAs walk a stage in two
// 64-deep halves with the fragment pipeline of that kernel (next fragments
// read while the current ones are multiplied). One barrier per stage, between
// its halves: it makes the next stage's panels visible and frees the two
// slots of the finished stage s, which at once take panels 2s+NP and
// 2s+NP+1, so NP-2 panels stay in flight. Large tiles fill the LDS with five
// 32 KB slots. For small tiles, five slots let several workgroups share a
// compute unit; deeper rings (more weight bytes in flight per workgroup, fewer
// workgroups) measured faster only at small M, so both are variants.
// Blockwise: the stage is one 128-deep scale block. Its two MFMA halves
// accumulate into a separate partial tile that is scaled by
// a_scale[m][kb] * b_scale[nb][kb] before it joins the accumulator. The
// stage's scales ride with its B panel: the DMA also copies the BM activation
// scales of block kb (the waves split them) and, per wave, the tile's weight
// block scales into the spare end of the B slot.
// ---------------------------------------------------------------------------
// SC_IN_A: the blockwise scales travel with the A panel instead of the B panel.
template <int BM, int BN, int WM, int WN, int KIND, int NP, bool SC_IN_A = false>
struct PanelGeom {
  static constexpr int NW = WM * WN;
  static constexpr int NBLK = (BN + 127) / 128;                // weight scale blocks per tile
  static constexpr int SA_BYTES = KIND != kChannelwise ? BM * 4 : 0;
  static constexpr int SB_BYTES = KIND != kChannelwise ? NW * 16 : 0;
  static constexpr int A_BYTES = BM * 128 + (SC_IN_A ? SA_BYTES + SB_BYTES : 0);
  static constexpr int B_BYTES = BN * 128 + (SC_IN_A ? 0 : SA_BYTES + SB_BYTES);
  static constexpr int SLOT = ((A_BYTES > B_BYTES ? A_BYTES : B_BYTES) + 1023) / 1024 * 1024;
  static constexpr int LDS = NP * SLOT;
  static constexpr int SC_OFF = SC_IN_A ? BM * 128 : BN * 128;  // scales inside their slot
};

// Channelwise panel tiles whose ring leaves room keep the tile's scales in a
// table past it for the epilogue (store_tile, sc_off); LDS bytes of a tile.
template <int BM, int BN, int WM, int WN, int KIND, int NP>
constexpr bool panel_epi_scales() {
  return KIND == kChannelwise && PanelGeom<BM, BN, WM, WN, KIND, NP>::LDS + (BM + BN) * 4 <= 163840;
}
template <int BM, int BN, int WM, int WN, int KIND, int NP>
constexpr int panel_lds_bytes() {
  return PanelGeom<BM, BN, WM, WN, KIND, NP>::LDS + (panel_epi_scales<BM, BN, WM, WN, KIND, NP>() ? (BM + BN) * 4 : 0);
}

// Wait until at most the c newest DMA panels of this wave are outstanding,
// c <= C, those panels alternating P0 instructions, P1, P0, ... from the
// oldest of them.
template <int C, int P0, int P1>
__device__ __forceinline__ void wait_panels(int64_t c) {
  if constexpr (C <= 0) {
    wait_vmcnt<0>();
  } else {
    if (c >= C) wait_vmcnt<((C + 1) / 2) * P0 + (C / 2) * P1>();
    else wait_panels<C - 1, P0, P1>(c);
  }
}

template <int BM, int BN, int WM, int WN, int KIND, int NP>
__global__ __launch_bounds__(WM * WN * 64) void gemm_panel_kernel(GemmArgs p) {
  using G = PanelGeom<BM, BN, WM, WN, KIND, NP>;
  constexpr bool BW = KIND != kChannelwise;
  // blockwise fp32 scales: per-stage partial tiles promoted in fp32; E8M0
  // scales: exponents handed to the block-scaled MFMA, no partial tile
  constexpr bool PROMOTE = KIND == kBlockwise;
  constexpr bool E8 = KIND == kBlockwiseE8;
  constexpr int NT = WM * WN * 64;
  constexpr int NW = WM * WN;
  constexpr int BK = 128;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int SLOT = G::SLOT;
  constexpr int PPA = BM / 8 / NW;     // DMA instructions per wave per A panel
  constexpr int PPB = BN / 8 / NW;     // ... per B panel (rows only)
  // blockwise: the per-stage scale copies ride with the B panel
  constexpr int PPB_ALL = PPB + (BW ? 2 : 0);
  constexpr int PPA_ALL = PPA;
  constexpr int SA_OFF = G::SC_OFF;    // scale area inside its slot
  constexpr int SB_OFF = SA_OFF + G::SA_BYTES;
  constexpr int SA_LANES = BM / 4 / NW;  // lanes of a wave's 16-byte activation-scale DMA
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(PPA >= 1 && PPB >= 1 && (BM / 8) % NW == 0 && (BN / 8) % NW == 0, "panel rows per wave");
  static_assert(G::LDS <= 163840, "ring fits the LDS");
  static_assert(NP >= 4, "ring depth");
  static_assert(((NP - 1) / 2) * PPB_ALL + ((NP - 2) / 2) * PPA_ALL < 64 &&
                ((NP - 1) / 2) * PPA_ALL + ((NP - 2) / 2) * PPB_ALL < 64, "vmcnt range");
  static_assert(BM * BN * 2 <= G::LDS, "output tile fits the ring");
  static_assert(!BW || (SA_LANES >= 1 && SA_LANES * 4 <= 64 && BM % (4 * NW) == 0 && G::NBLK <= 4 &&
                        WTN <= 128 && 128 % WTN == 0),
                "blockwise scale layout");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int h = lane >> 5;
  const int r32 = lane & 31;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tile = blockIdx.x;
  int64_t tile_m, tile_n;
  tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  const int64_t m0 = tile_m * BM;
  const int64_t n0 = tile_n * BN;
  // grouped (MoE experts): expert blockIdx.z has masked_m[e] valid rows of
  // its own M-row slab; the tile order covers all M rows, and tiles wholly
  // past the valid rows leave here, before any barrier or LDS use
  if (p.masked_m) {
    const int64_t e = blockIdx.z;
    int64_t rows = p.masked_m[e];
    rows = rows < 0 ? 0 : (rows > p.M ? p.M : rows);
    if (m0 >= rows) return;
    p.M = rows;
    p.a += e * p.a_es;
    p.sa += e * p.sa_es;
    p.b += e * p.b_es;
    p.sb += e * p.sb_es;
    p.out += e * p.out_es;
  }
  const int split = blockIdx.y;
  const int64_t kt_all = p.K / BK;
  const int64_t kt_begin = (int64_t)split * p.k_tiles_per_split;
  int64_t kt_end = kt_begin + p.k_tiles_per_split;
  if (kt_end > kt_all) kt_end = kt_all;
  const int64_t nst = kt_end - kt_begin;  // stages of this split (may be <= 0)

  // DMA addressing. Instruction i of a wave covers panel rows
  // rb_i = (wave * PP + i) * 8 .. +7, lane l row rb_i + l / 8, and fetches
  // logical chunk swz<8>(row, l % 8), which lands at position l % 8 of the
  // row in LDS; the swizzle depends on the row through l / 8 and the parity
  // of rb_i / 8 only. Rows past the matrix read its last row (never stored).
  const int lrow = lane >> 3;
  uint32_t lchunk[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) lchunk[par] = (uint32_t)(swz<8>(par * 8 + lrow, lane & 7) << 4);
  auto issue_rows = [&](const uint8_t* src, uint32_t r0, uint32_t last, uint32_t ld, uint32_t dst,
                        auto pp) {
    constexpr int PP = decltype(pp)::value;
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      uint32_t row = r0 + (wave * PP + i) * 8 + lrow;
      row = row < last ? row : last;
      lds_dma16_s(src, row * ld + lchunk[(wave * PP + i) & 1], dst + i * 1024);
    }
  };
  // blockwise scales of block kt into the scale area of the slot at sbase
  // activation-scale columns that start on 16 bytes (ld a multiple of 4)
  // travel in 16-byte pieces, others one scale per lane; either way one DMA
  // instruction per wave with the same LDS image
  const bool sa_vec = (p.sa_ld & 3) == 0 && (reinterpret_cast<uintptr_t>(p.sa) & 15) == 0;
  auto issue_scales = [&](int64_t kt, uint32_t sbase) {
    // activation scales of block kt, rows m0 .. m0+BM-1 (column-major, ld
    // sa_ld; pieces clamped into the column): wave w copies rows
    // [w * BM / NW, (w + 1) * BM / NW), SA_LANES lanes of 4 rows or BM / NW
    // lanes of one row
    {
      const uint8_t* col = reinterpret_cast<const uint8_t*>(p.sa + kt * p.sa_ld);
      const uint32_t dst = sbase + SA_OFF + wave * SA_LANES * 16;
      // lane 0 is always active, so the instruction always issues and
      // counts once in this wave's vmcnt
      if (sa_vec) {
        int64_t r = m0 + (int64_t)(wave * SA_LANES + (lane < SA_LANES ? lane : 0)) * 4;
        if (r > p.sa_ld - 4) r = p.sa_ld - 4;
        if (lane < SA_LANES) lds_dma16_s(col, (uint32_t)(r * 4), dst);
      } else {
        int64_t r = m0 + (int64_t)wave * (SA_LANES * 4) + (lane < SA_LANES * 4 ? lane : 0);
        if (r > p.sa_ld - 1) r = p.sa_ld - 1;
        if (lane < SA_LANES * 4) lds_dma4_s(col, (uint32_t)(r * 4), dst);
      }
    }
    // weight block scales b_scale[n0 / 128 + l][kt], lanes l < NBLK, one
    // 16-byte copy per wave (lane 0 always active, as above); a block past
    // the last one (a tile overhanging N) reads the last block instead, its
    // columns are never stored
    {
      const int64_t kb_all = p.K / 128;
      const int64_t nb_last = (p.N + 127) / 128 - 1;
      int64_t nb = (n0 >> 7) + lane;
      nb = nb < nb_last ? nb : nb_last;
      if (lane < G::NBLK)
        lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sb + kt), (uint32_t)(nb * kb_all * 4),
                   sbase + SB_OFF + wave * 16);
    }
  };
  auto issue_a = [&](int64_t kt, int slot) {
    const uint32_t sbase = lds_base + (uint32_t)slot * SLOT;
    issue_rows(p.a + kt * BK, (uint32_t)m0, (uint32_t)(p.M - 1), (uint32_t)p.lda,
               sbase + wave * PPA * 1024, IntC<PPA>());
  };
  auto issue_b = [&](int64_t kt, int slot) {
    const uint32_t sbase = lds_base + (uint32_t)slot * SLOT;
    issue_rows(p.b + kt * BK, (uint32_t)n0, (uint32_t)(p.N - 1), (uint32_t)p.ldb,
               sbase + wave * PPB * 1024, IntC<PPB>());
    if constexpr (BW) issue_scales(kt, sbase);
  };
  // Per-lane byte offsets, within a panel, of the two 16-byte chunks of this
  // lane's A fragment row for each 64-deep half kh (chunks 4kh + 2h, +1). The
  // swizzle depends on the row only through row % 16, the same for every
  // 32-row fragment of every wave, so A fragment i adds i * 32 * BK and B
  // fragment j adds (wn * WTN - wm * WTM + j * 32) * BK.
  uint32_t fo[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      fo[kh][t] = (uint32_t)((wm * WTM + r32) * BK + (swz<8>(r32, 4 * kh + 2 * h + t) << 4));
  const int b_shift = (wn * WTN - wm * WTM) * BK;
  auto frag_at = [&](const uint8_t* base, int kh) {
    return join(*reinterpret_cast<const uint4*>(base + fo[kh][0]),
                *reinterpret_cast<const uint4*>(base + fo[kh][1]));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero16();
  // blockwise: the current stage's partial tile and scales (E8M0: the
  // scales' exponents only)
  f32x16 part[PROMOTE ? TM : 1][PROMOTE ? TN : 1];
  float sc_a[PROMOTE ? TM : 1], sc_b[PROMOTE ? TN : 1];
  int ex_a[E8 ? TM : 1], ex_b[E8 ? TN : 1];

  i32x8 fa[TM], fb0[TN], fb1[TN];
  // MFMAs on (fa, fb0) while the next half's fragments are read from the
  // slots (sa, sb): B into fb1 first, each A fragment into fa right after its
  // MFMAs; then fb1 becomes the current B. kh is the half being read: when it
  // is 1 the MFMAs are the first half of their stage (whose second half is
  // being read), when 0 the second half (the next stage is being read).
  auto half = [&](int sa, int sb, int kh) {
    const uint8_t* pa = lds + sa * SLOT;
    const uint8_t* pb = lds + sb * SLOT + b_shift;
    if constexpr (PROMOTE) {
      if (kh == 1) {  // this stage's scales, while its B slot is still ours
        const uint8_t* sc = lds + sb * SLOT;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          sc_a[i] = *reinterpret_cast<const float*>(sc + SA_OFF + (wm * WTM + i * 32 + r32) * 4);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          sc_b[j] = *reinterpret_cast<const float*>(sc + SB_OFF + wave * 16 +
                                                     ((wn * WTN + j * 32) >> 7) * 4);
      }
    }
    if constexpr (E8) {
      if (kh == 1) {  // the same reads, keeping the biased exponents
        const uint8_t* sc = lds + sb * SLOT;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          ex_a[i] = (int)(*reinterpret_cast<const uint32_t*>(sc + SA_OFF + (wm * WTM + i * 32 + r32) * 4) >> 23);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          ex_b[j] = (int)(*reinterpret_cast<const uint32_t*>(sc + SB_OFF + wave * 16 +
                                                            ((wn * WTN + j * 32) >> 7) * 4) >> 23);
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) fb1[j] = frag_at(pb + j * 32 * BK, kh);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (PROMOTE) {
          part[i][j] = mfma32_fp8(fb0[j], fa[i], kh == 1 ? zero16() : part[i][j]);
        } else if constexpr (E8) {
          acc[i][j] = mfma32_fp8_e8(fb0[j], fa[i], acc[i][j], ex_b[j], ex_a[i]);
        } else {
          acc[i][j] = mfma32_fp8(fb0[j], fa[i], acc[i][j]);
        }
      }
      fa[i] = frag_at(pa + i * 32 * BK, kh);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TN, 0);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) fb0[j] = fb1[j];
  };
  // blockwise: the finished stage's partial tile joins the accumulator
  auto promote = [&]() {
    if constexpr (PROMOTE) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] += part[i][j] * (sc_a[i] * sc_b[j]);
    }
  };
  auto wrap = [](int x) { return x >= NP ? x - NP : x; };

  const int64_t np_all = 2 * nst;  // panels of this split
  auto issue_panel = [&](int64_t q, int slot) {
    if (q & 1) issue_a(kt_begin + (q >> 1), slot);
    else issue_b(kt_begin + (q >> 1), slot);
  };
  // the epilogue's scale table (entries e < BM: activation scale of row
  // m0 + e, then weight scale of column n0 + e - BM; indices past the matrix
  // read its last one), before any panel so that every wait covers it; every
  // instruction has lane 0 active
  constexpr bool EPI_SC = panel_epi_scales<BM, BN, WM, WN, KIND, NP>();
  if constexpr (EPI_SC) {
    for (int c = wave * 64; c < BM + BN; c += NW * 64) {
      const int e = c + lane;
      if (e < BM + BN) {
        if (e < BM) {
          int64_t r = m0 + e;
          r = r < p.M - 1 ? r : p.M - 1;
          lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sa), (uint32_t)(r * 4), lds_base + G::LDS + c * 4);
        } else {
          int64_t n = n0 + (e - BM);
          n = n < p.N - 1 ? n : p.N - 1;
          lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sb), (uint32_t)(n * 4), lds_base + G::LDS + c * 4);
        }
      }
    }
    if (nst <= 0) wait_vmcnt<0>();
  }
  if (nst > 0) {
    // prologue: panels 0 .. min(NP, 2 nst) - 1 into slots 0 .. NP-1, then
    // stage 0 (panels 0 and 1) complete; the outstanding ones start with a
    // B panel
    const int64_t first = np_all < NP ? np_all : NP;
    for (int64_t q = 0; q < first; ++q) issue_panel(q, (int)q);
    wait_panels<NP - 2, PPB_ALL, PPA_ALL>(first - 2);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = frag_at(lds + SLOT + i * 32 * BK, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb0[j] = frag_at(lds + b_shift + j * 32 * BK, 0);
  }
  int cs = 0;  // slot of the current stage's B panel (2s % NP); its A panel is in wrap(cs + 1)
  for (int64_t s = 0; s + 1 < nst; ++s) {
    const int cs1 = wrap(cs + 1);
    // first half of stage s; its second half's fragments come from the same slots
    half(cs1, cs, 1);
    // stage s+1 (panels 2s+2, 2s+3) complete: panels up to 2s+NP-1 are
    // issued, so panels 2s+4 .. (from a B panel on) may still be outstanding
    {
      const int64_t later = np_all - 2 * s - 4;
      wait_panels<NP - 4, PPB_ALL, PPA_ALL>(later < NP - 4 ? later : NP - 4);
    }
    wait_vmcnt_lgkm0<63>();
    __builtin_amdgcn_s_barrier();
    // every wave is done with stage s: its slots take panels 2s+NP, 2s+NP+1
    if (2 * s + NP < np_all) issue_panel(2 * s + NP, cs);
    if (2 * s + NP + 1 < np_all) issue_panel(2 * s + NP + 1, cs1);
    cs = wrap(cs + 2);
    half(wrap(cs + 1), cs, 0);
    promote();
  }
  if (nst > 0) {  // last stage: both halves from the slots already in LDS
    half(wrap(cs + 1), cs, 1);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (PROMOTE) part[i][j] = mfma32_fp8(fb0[j], fa[i], part[i][j]);
        else if constexpr (E8) acc[i][j] = mfma32_fp8_e8(fb0[j], fa[i], acc[i][j], ex_b[j], ex_a[i]);
        else acc[i][j] = mfma32_fp8(fb0[j], fa[i], acc[i][j]);
      }
    promote();
  }

  // the ring is idle from here on: its first word serves as the split flag
  if (p.split_k > 1 && !splitk_reduce<TM, TN, NT>(p, acc, tile, split, tid, reinterpret_cast<int*>(lds)))
    return;
  store_tile<BM, BN, WM, WN, KIND>(p, acc, lds, m0, n0, wm, wn, h, r32, tid, EPI_SC ? G::LDS : -1);
}


// ---------------------------------------------------------------------------
// Ping-pong 256x256 tile (K % 128 == 0) on 16x16x128 MFMAs, for channelwise
// scales, blockwise fp32 scales (each MFMA covers one 128-deep block, and its
// result joins the accumulator times a_scale[m][kb] * b_scale[nb][kb]) and
// blockwise E8M0 scales (applied by the block-scaled MFMA).
// Eight waves, two per SIMD: waves 0-3 (group 0) own output rows 0-127 of the
// tile, waves 4-7 (group 1) rows 128-255, each wave a 128x64 piece (8 x 4
// accumulators of 16x16). Both groups run the same sequence of phases, each
// ending at a workgroup barrier, group 1 one phase behind group 0 (it starts
// with one barrier more; group 0 ends with one more). A wave alternates
// memory phases (its share of the ring refills, the LDS fragment and scale
// reads for its next 16 MFMAs, the waits) and compute phases (those 16 MFMAs
// and, for fp32 block scales, their promotion), so on every SIMD one wave
// multiplies while the other loads. The phases are kept apart for the
// compiler too: no instruction is scheduled across a phase barrier, and the
// accumulators a compute phase wrote are pinned before it ends.
// Stage s (one 128-deep K block) is read in two halves h: (s,0) takes the B
// fragments and A fragments 0-3 (rows 0-63 of the wave's 128), (s,1) A
// fragments 4-7; group 0 reads half (s,h) in global phase 4s + 2h, group 1 in
// 4s + 2h + 1. Ring: four slots, B(s) in slot 2s % 4, A(s) in (2s + 1) % 4
// together with the stage's scales. A wave issues its share of A(s+1) in its
// memory phase (s,0) -- A(s-1), in that slot, was last read in phase 4s - 1
// -- and of B(s+2) in (s,1) -- B(s) was last read in phase 4s + 1. Stage s+1
// is read from phase 4s + 4 on, so both groups wait for their share of it at
// the end of phase 4s + 3 (group 0 after its compute phase (s,1), group 1
// after its memory phase (s,1)), when only their B(s+2) share is younger.
// Grouped calls (masked_m, one expert per blockIdx.z) as in the panel tiles.
// ---------------------------------------------------------------------------
// LDS of the ping-pong tile: the ring, then a 2 KB table: channelwise the
// epilogue's 256 activation and 256 weight scales, blockwise the tile's two
// weight block scales of up to 256 K blocks.
template <int KIND>
constexpr int pingpong_lds_bytes() {
  return PanelGeom<256, 256, 2, 4, KIND, 4, true>::LDS + 2 * 256 * 4;
}

__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int KIND>
__global__ __launch_bounds__(512) void gemm_pingpong_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NP = 4, BK = 128;
  using G = PanelGeom<BM, BN, WM, WN, KIND, NP, true>;
  constexpr bool SC = KIND != kChannelwise;  // scales travel with the A panels
  constexpr bool PROMOTE = KIND == kBlockwise;
  constexpr bool E8 = KIND == kBlockwiseE8;
  constexpr int NT = 512, NW = 8;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FI = WTM / 16, FJ = WTN / 16;  // 8 x 4 accumulators per wave
  constexpr int SLOT = G::SLOT;
  constexpr int PPA = BM / 8 / NW, PPB = BN / 8 / NW;  // DMA instructions per wave per panel
  constexpr int SA_OFF = G::SC_OFF;
  constexpr int SB_OFF = SA_OFF + G::SA_BYTES;
  constexpr int SA_LANES = BM / 4 / NW;
  static_assert(pingpong_lds_bytes<KIND>() <= 163840 && BM * BN * 2 <= G::LDS, "ring and output tile fit the LDS");
  static_assert(2 * PPA + 2 < 64, "vmcnt range");

  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / WN;  // the group is the wave's row half
  const int wm = grp, wn = wave % WN;
  const int g16 = lane >> 4, r16 = lane & 15;

  const int64_t tiles_n = (p.N + BN - 1) / BN;
  const int64_t tiles_m = (p.M + BM - 1) / BM;
  const int64_t tile = blockIdx.x;
  int64_t tile_m, tile_n;
  tile_coords(tile, tiles_m, tiles_n, &tile_m, &tile_n);
  const int64_t m0 = tile_m * BM;
  const int64_t n0 = tile_n * BN;
  if (p.masked_m) {  // tiles wholly past the expert's rows leave before any barrier
    const int64_t e = blockIdx.z;
    int64_t rows = p.masked_m[e];
    rows = rows < 0 ? 0 : (rows > p.M ? p.M : rows);
    if (m0 >= rows) return;
    p.M = rows;
    p.a += e * p.a_es;
    p.sa += e * p.sa_es;
    p.b += e * p.b_es;
    p.sb += e * p.sb_es;
    p.out += e * p.out_es;
  }
  const int split = blockIdx.y;
  const int64_t kt_all = p.K / BK;
  const int64_t kt_begin = (int64_t)split * p.k_tiles_per_split;
  int64_t kt_end = kt_begin + p.k_tiles_per_split;
  if (kt_end > kt_all) kt_end = kt_all;
  const int64_t nst = kt_end - kt_begin;

  // DMA of panel rows, as in the panel tiles (instruction i of a wave: rows
  // (wave * PP + i) * 8 .. +7, lane l row + l / 8, logical chunk swz<8> landing
  // at position l % 8). The per-lane offsets are recomputed at every refill:
  // kept live across the loop they would take eight registers.
  const int lrow = lane >> 3;
  auto issue_rows = [&](const uint8_t* src, uint32_t r0, uint32_t last, uint32_t ld, uint32_t dst, auto pp) {
    constexpr int PP = decltype(pp)::value;
    int lr = lrow;
    __asm__ volatile("" : "+v"(lr));
#pragma unroll
    for (int i = 0; i < PP; ++i) {
      uint32_t row = r0 + (wave * PP + i) * 8 + lr;
      row = row < last ? row : last;
      const uint32_t chunk = (uint32_t)(swz<8>(((wave * PP + i) & 1) * 8 + lr, lane & 7) << 4);
      lds_dma16_s(src, row * ld + chunk, dst + i * 1024);
    }
  };
  // the stage's scales into the scale area of its A slot: activation scales
  // of rows m0 .. m0+255, one per lane, placed so that the four a wave needs
  // for one half of a stage are adjacent (position 128 g + 8 r + f holds
  // row 128 g + 16 f + r: group g, fragment f, fragment row r), and, per
  // wave, the tile's two weight block scales; one DMA instruction each per
  // wave (lane 0 always active)
  // blockwise, K <= 256 blocks: the tile's weight block scales of every K
  // block are copied once, before the first panel, into a table past the
  // ring ([block][kb], 256 apart), not with every stage
  const bool sb_table = SC && p.K / 128 <= 256;
  auto issue_scales = [&](int64_t kt, uint32_t sbase) {
    const uint8_t* col = reinterpret_cast<const uint8_t*>(p.sa + kt * p.sa_ld);
    const uint32_t dst = sbase + SA_OFF + wave * SA_LANES * 16;
    {
      const int pos = wave * (SA_LANES * 4) + (lane < SA_LANES * 4 ? lane : 0);
      int64_t r = m0 + (pos & ~127) + (pos & 7) * 16 + ((pos & 127) >> 3);
      if (r > p.sa_ld - 1) r = p.sa_ld - 1;
      if (lane < SA_LANES * 4) lds_dma4_s(col, (uint32_t)(r * 4), dst);
    }
    if (sb_table) return;
    const int64_t kb_all = p.K / 128;
    const int64_t nb_last = (p.N + 127) / 128 - 1;
    int64_t nb = (n0 >> 7) + lane;
    nb = nb < nb_last ? nb : nb_last;
    if (lane < G::NBLK)
      lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sb + kt), (uint32_t)(nb * kb_all * 4),
                 sbase + SB_OFF + wave * 16);
  };
  auto issue_a = [&](int64_t s) {
    const uint32_t sbase = lds_base + (uint32_t)((2 * s + 1) & 3) * SLOT;
    issue_rows(p.a + (kt_begin + s) * BK, (uint32_t)m0, (uint32_t)(p.M - 1), (uint32_t)p.lda,
               sbase + wave * PPA * 1024, IntC<PPA>());
    if constexpr (SC) issue_scales(kt_begin + s, sbase);
  };
  auto issue_b = [&](int64_t s) {
    const uint32_t sbase = lds_base + (uint32_t)((2 * s) & 3) * SLOT;
    issue_rows(p.b + (kt_begin + s) * BK, (uint32_t)n0, (uint32_t)(p.N - 1), (uint32_t)p.ldb,
               sbase + wave * PPB * 1024, IntC<PPB>());
  };

  // lane's chunks of a 16-row fragment: row r16, K bytes [32 g16, 32 g16 + 32)
  uint32_t fo16[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) fo16[t] = (uint32_t)(r16 * BK + (swz<8>(r16, 2 * g16 + t) << 4));
  auto frag16 = [&](const uint8_t* base) {
    return join(*reinterpret_cast<const uint4*>(base + fo16[0]), *reinterpret_cast<const uint4*>(base + fo16[1]));
  };

  f32x4 acc16[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc16[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  i32x8 fb[FJ], fa[4];
  float sc[4] = {1.f, 1.f, 1.f, 1.f}, sbv = 1.f;  // fp32 block scales
  int ea[4] = {0, 0, 0, 0}, eb = 0;                // E8M0 exponents

  // memory phase of half H of stage s. Blockwise, the phase runs at raised
  // wave priority: the other group's compute phase issues the promotion's
  // VALU work at the same time, and the memory phases set the stage period
  // (measured 2-3% faster at M = 4096 and 8192; channelwise unchanged, so
  // left at the default there)
  auto mem = [&](int64_t s, auto hc) {
    constexpr int H = decltype(hc)::value;
    if constexpr (PROMOTE) __builtin_amdgcn_s_setprio(1);
    if (H == 0) {
      if (s + 1 < nst) issue_a(s + 1);
    } else {
      if (s + 2 < nst) issue_b(s + 2);
    }
    const uint8_t* pa = lds + ((2 * s + 1) & 3) * SLOT;
    if (H == 0) {
      const uint8_t* pb = lds + ((2 * s) & 3) * SLOT + (wn * WTN) * BK;
#pragma unroll
      for (int j = 0; j < FJ; ++j) fb[j] = frag16(pb + j * 16 * BK);
      const uint32_t sbw =
          !SC ? 0u
          : sb_table ? *reinterpret_cast<const uint32_t*>(lds + G::LDS + (((wn * WTN) >> 7) * 256 + kt_begin + s) * 4)
                     : *reinterpret_cast<const uint32_t*>(pa + SB_OFF + wave * 16 + ((wn * WTN) >> 7) * 4);
      if constexpr (PROMOTE) sbv = __uint_as_float(sbw);
      if constexpr (E8) eb = (int)(sbw >> 23);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag16(pa + (wm * WTM + (4 * H + i) * 16) * BK);
    if constexpr (SC) {
      // this lane's four row scales of the half, adjacent (see issue_scales)
      const uint4 w4 = *reinterpret_cast<const uint4*>(pa + SA_OFF + (wm * WTM + r16 * 8 + 4 * H) * 4);
      const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (PROMOTE) sc[i] = __uint_as_float(w[i]) * sbv;
        if constexpr (E8) ea[i] = (int)(w[i] >> 23);
      }
    }
    if constexpr (PROMOTE) __builtin_amdgcn_s_setprio(0);
    if (H == 1 && grp == 1) {  // stage s+1 complete; B(s+2) may be younger
      if (s + 2 < nst) wait_vmcnt_lgkm0<PPB>();
      else wait_vmcnt_lgkm0<0>();
    } else {
      wait_vmcnt_lgkm0<63>();
    }
  };
  // compute phase of half H of stage s
  auto comp = [&](int64_t s, auto hc) {
    constexpr int H = decltype(hc)::value;
    if constexpr (PROMOTE) {
      // three-deep pipeline: the promotion of MFMA q follows the issue of
      // MFMA q+2, so it never waits for a result still in the matrix core
      constexpr int NQ = 4 * FJ;
      f32x4 tq[3];
      tq[0] = mfma_fp8(fb[0], fa[0], f32x4{0.f, 0.f, 0.f, 0.f});
      tq[1] = mfma_fp8(fb[1 % FJ], fa[1 / FJ], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 2; q < NQ + 2; ++q) {
        if (q < NQ) tq[q % 3] = mfma_fp8(fb[q % FJ], fa[q / FJ], f32x4{0.f, 0.f, 0.f, 0.f});
        const int d = q - 2;
        acc16[4 * H + d / FJ][d % FJ] += tq[d % 3] * sc[d / FJ];
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
#pragma unroll
      for (int q = 2; q < NQ; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          if constexpr (E8) acc16[4 * H + i][j] = mfma_fp8_e8(fb[j], fa[i], acc16[4 * H + i][j], eb, ea[i]);
          else acc16[4 * H + i][j] = mfma_fp8(fb[j], fa[i], acc16[4 * H + i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __asm__ volatile("" : "+v"(acc16[4 * H + i][0]), "+v"(acc16[4 * H + i][1]), "+v"(acc16[4 * H + i][2]),
                       "+v"(acc16[4 * H + i][3]));
    if (H == 1 && grp == 0) {  // stage s+1 complete; B(s+2) may be younger
      if (s + 2 < nst) wait_vmcnt<PPB>();
      else wait_vmcnt<0>();
    }
  };

  if (SC && sb_table) {
    // wave w: weight block (n0 >> 7) + (w & 1), K blocks 64 (w >> 1) + lane
    const int64_t kb_all = p.K / 128;
    const int64_t nb_last = (p.N + 127) / 128 - 1;
    int64_t nb = (n0 >> 7) + (wave & 1);
    nb = nb < nb_last ? nb : nb_last;
    const int64_t kb0 = (int64_t)(wave >> 1) * 64;
    if (kb0 < kb_all) {
      int64_t kb = kb0 + lane;
      kb = kb < kb_all - 1 ? kb : kb_all - 1;
      lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sb), (uint32_t)((nb * kb_all + kb) * 4),
                 lds_base + (uint32_t)G::LDS + (uint32_t)((wave & 1) * 256 + kb0) * 4);
    }
  }
  // channelwise: the tile's scales into the table past the ring for the
  // epilogue, before any panel, so every wait below covers them; waves 0-3
  // copy activation scales of rows m0 + 64w .., waves 4-7 weight scales of
  // columns n0 + 64(w - 4) .. (indices past the matrix read its last one)
  if constexpr (KIND == kChannelwise) {
    const uint32_t dst = lds_base + (uint32_t)G::LDS + (uint32_t)wave * 256;
    if (grp == 0) {
      int64_t r = m0 + wave * 64 + lane;
      r = r < p.M - 1 ? r : p.M - 1;
      lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sa), (uint32_t)(r * 4), dst);
    } else {
      int64_t c = n0 + (wave - 4) * 64 + lane;
      c = c < p.N - 1 ? c : p.N - 1;
      lds_dma4_s(reinterpret_cast<const uint8_t*>(p.sb), (uint32_t)(c * 4), dst);
    }
  }
  if (nst > 0) {
    issue_b(0);
    issue_a(0);
    if (nst > 1) {
      issue_b(1);
      wait_vmcnt<PPB>();
    } else {
      wait_vmcnt<0>();
    }
    phase_barrier();
    if (grp == 1) phase_barrier();
    for (int64_t s = 0; s < nst; ++s) {
      mem(s, IntC<0>());
      phase_barrier();
      comp(s, IntC<0>());
      phase_barrier();
      mem(s, IntC<1>());
      phase_barrier();
      comp(s, IntC<1>());
      phase_barrier();
    }
    if (grp == 0) phase_barrier();
  } else {
    wait_vmcnt<0>();
  }
  // the ring is idle from here on: its first word serves as the split flag
  if (p.split_k > 1 && !splitk_reduce<FI, FJ, NT>(p, acc16, tile, split, tid, reinterpret_cast<int*>(lds)))
    return;
  store_tile16<BM, BN, WM, WN, KIND>(p, acc16, lds, m0, n0, wm, wn, lane, tid, G::LDS);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [LO, HI] (a branch tree over
// the immediate forms); n above HI waits for HI, which only waits longer.
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (LO == HI) {
    wait_vmcnt<LO>();
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vmcnt_upto<LO, MID>(n);
    else wait_vmcnt_upto<MID + 1, HI>(n);
  }
}

// ---------------------------------------------------------------------------
// Decode-size weight stream (M <= 16, K % 128 == 0). One workgroup of 8 waves
// per 16 weight rows (16 output columns). Every wave streams its own 128-deep
// K blocks through its own LDS ring and multiplies each with one
// V_MFMA_F32_16X16X128_F8F6F4: no barrier until the final reduction, so no
// wave waits for another while it has copies in flight. A block is the 16
// weight rows' 128-byte pieces (two LDS-DMA instructions, one cache line per
// row) and the activation rows' pieces (one instruction per 8 rows, rows at
// or past M read as row M - 1, whose outputs are never stored); in LDS chunk
// c of row r sits at position c ^ (r % 8), so the 16 rows of a fragment read
// hit distinct banks. Wave w takes blocks 4w .. 4w + 3 of every 32 (4 KB of
// K), in that order, as the register-staged weight-streaming kernel does, so
// the fp32 sums and the outputs are bit-identical to its (and to the
// single-launch linear's). Each wave counts its own copies and waits for the
// block it multiplies next; a slot is refilled by the wave that read it, one
// block after its fragments went to registers. Ring depth (slots per wave)
// is a launch parameter: with one round of workgroups over the compute units
// as many as fit 160 KB (at most 6), beyond that as many as fit 80 KB (two
// workgroups per compute unit). The blockwise scales of the whole K range
// go to an LDS table by LDS-DMA ahead of the first blocks. The eight waves'
// partial tiles are summed through LDS in wave order (deterministic).
// ---------------------------------------------------------------------------
namespace {
constexpr int kDecWaves = 8;
constexpr int kDecMaxWaveSlots = 6;
}  // namespace

// Activation tiles of 16 rows (1, 2 or 4 for M <= 16, 32, 64); LDS bytes of
// the decode kernel's scale table (blockwise: 16 x tiles + 1 floats per K
// block, in whole 64-float pieces, one LDS-DMA instruction each) and of one
// wave's ring slot (16 weight rows, then the activation rows in groups of
// 8, 128 bytes each).
__host__ __device__ inline int decode_tiles(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }
__host__ __device__ inline size_t decode_scale_bytes(int64_t K, int kind, int64_t M) {
  const int64_t st = 16 * decode_tiles(M) + 1;
  return kind != kChannelwise ? (size_t)(((K / 128) * st + 63) / 64) * 256 : 0;
}
__host__ __device__ inline size_t decode_slot_bytes(int64_t M) { return 2048 + (size_t)((M + 7) / 8) * 1024; }

// Blocks of wave w: i -> K block 32 (i / 4) + 4 w + i % 4, for i < the count.
__device__ __forceinline__ int decode_wave_blocks(int64_t kb_all, int wave) {
  int tail = (int)(kb_all % 32) - 4 * wave;
  tail = tail < 0 ? 0 : (tail > 4 ? 4 : tail);
  return (int)(kb_all / 32) * 4 + tail;
}
__device__ __forceinline__ int64_t decode_wave_kb(int i, int wave) {
  return (int64_t)(i >> 2) * 32 + 4 * wave + (i & 3);
}

template <int KIND, int MT>
__global__ __launch_bounds__(kDecWaves * 64) void gemm_decode_kernel(GemmArgs p) {
  static_assert(KIND == kChannelwise || KIND == kBlockwise, "fp32 scales");
  static_assert(MT == 1 || MT == 2 || MT == 4, "16-row activation tiles");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int M = (int)p.M;  // <= 16 MT
  const int R = p.ring_slots;  // slots per wave, 2 .. kDecMaxWaveSlots
  const uint32_t sbytes = (uint32_t)decode_slot_bytes(M);
  const int arows = (M + 7) / 8;  // activation DMA instructions per block (8 rows each)
  const int cnt = 2 + arows;      // this wave's copies per block
  const int64_t kb_all = p.K / 128;
  // split-K: split s takes this wave's blocks [s per, (s + 1) per)
  const int split = blockIdx.y;
  const int nb_all = decode_wave_blocks(kb_all, wave);
  const int i0 = split * p.k_tiles_per_split < nb_all ? split * p.k_tiles_per_split : nb_all;
  const int i1 = i0 + p.k_tiles_per_split < nb_all ? i0 + p.k_tiles_per_split : nb_all;
  const int nb = i1 - i0;
  const uint32_t ring = (uint32_t)kDecWaves * R * sbytes;
  const uint32_t wbase = lds_base + (uint32_t)wave * R * sbytes;
  // blockwise: scale of (row r, block kb) at sc[ST kb + r] (r < 16 MT), the
  // weight block scale of block kb at sc[ST kb + 16 MT]
  constexpr int ST = 16 * MT + 1;
  const float* sc = reinterpret_cast<const float*>(lds + ring);

  if constexpr (KIND == kBlockwise) {
    // 64 entries per instruction; rows at or past M take row M - 1's scale,
    // entries past the table fill its padding from a valid address
    const int64_t nbk = n0 >> 7, total = kb_all * ST, pieces = (total + 63) / 64;
    for (int64_t i = wave; i < pieces; i += kDecWaves) {
      const int64_t e = i * 64 + lane;
      const int64_t kb = e / ST;
      const int r = (int)(e - kb * ST);
      const float* src = e >= total   ? p.sb + nbk * kb_all
                         : r == ST - 1 ? p.sb + nbk * kb_all + kb
                                       : p.sa + kb * p.sa_ld + (r < M ? r : M - 1);
      lds_dma4_v(src, lds_base + ring + (uint32_t)(i * 256));
    }
  }
  // lane l of a DMA instruction fills LDS row 8 t + l / 8 (t the instruction)
  // at chunk position l % 8 with logical chunk (l % 8) ^ (row % 8)
  const int lr = lane >> 3;
  const uint32_t chunk = (uint32_t)(((lane & 7) ^ lr) << 4);  // row % 8 == lr for every instruction
  auto issue = [&](int i) {  // i counts this split's blocks from 0
    const int64_t kb = decode_wave_kb(i0 + i, wave);
    const uint32_t slot = wbase + (uint32_t)(i % R) * sbytes;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int64_t n = n0 + 8 * t + lr;
      n = n < p.N ? n : p.N - 1;
      lds_dma16_s(p.b, (uint32_t)(n * p.ldb + kb * 128) + chunk, slot + (uint32_t)t * 1024);
    }
    for (int t = 0; t < arows; ++t) {
      int r = 8 * t + lr;
      r = r < M ? r : M - 1;
      lds_dma16_s(p.a, (uint32_t)(r * p.lda + kb * 128) + chunk, slot + 2048 + (uint32_t)t * 1024);
    }
  };
  // this lane's fragment chunks: weight row r16 and, per activation tile t,
  // LDS row am_t = min(16 t + r16, M - 1); 16-byte chunks 2g and 2g + 1
  const uint32_t fb0 = (uint32_t)r16 * 128 + (uint32_t)(((2 * g) ^ (r16 & 7)) << 4);
  const uint32_t fb1 = (uint32_t)r16 * 128 + (uint32_t)(((2 * g + 1) ^ (r16 & 7)) << 4);
  uint32_t fa0[MT], fa1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int am = 16 * t + r16 < M ? 16 * t + r16 : M - 1;
    fa0[t] = 2048 + (uint32_t)am * 128 + (uint32_t)(((2 * g) ^ (am & 7)) << 4);
    fa1[t] = 2048 + (uint32_t)am * 128 + (uint32_t)(((2 * g + 1) ^ (am & 7)) << 4);
  }

  const int pro = R - 1 < nb ? R - 1 : nb;
  for (int i = 0; i < pro; ++i) issue(i);
  if constexpr (KIND == kBlockwise) {
    // the table's copies are this wave's oldest: wait for them, then for
    // every wave's
    wait_vmcnt_upto<0, 63>(pro * cnt);
    __syncthreads();
  }
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* wl = lds + (size_t)wave * R * sbytes;
  for (int i = 0; i < nb; ++i) {
    const int last = i + R - 2 < nb - 1 ? i + R - 2 : nb - 1;
    wait_vmcnt_upto<0, 63>((last - i) * cnt);  // block i has landed
    // the slot of block i - 1, whose fragments are in registers, takes block i + R - 1
    if (i + R - 1 < nb) issue(i + R - 1);
    const uint8_t* slot = wl + (size_t)(i % R) * sbytes;
    const i32x8 bf = join(*reinterpret_cast<const uint4*>(slot + fb0), *reinterpret_cast<const uint4*>(slot + fb1));
    const int64_t kb = decode_wave_kb(i0 + i, wave);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const i32x8 af =
          join(*reinterpret_cast<const uint4*>(slot + fa0[t]), *reinterpret_cast<const uint4*>(slot + fa1[t]));
      if constexpr (KIND == kChannelwise) {
        acc[t] = mfma_fp8(bf, af, acc[t]);
      } else {
        const f32x4 part = mfma_fp8(bf, af, f32x4{0.f, 0.f, 0.f, 0.f});
        acc[t] += part * (sc[kb * ST + 16 * t + r16] * sc[kb * ST + ST - 1]);
      }
    }
  }

  // split-K: every thread's partials go to the workspace; the last split
  // to arrive sums them in split order (per thread, so per wave) and goes on
  __syncthreads();  // the ring is idle: its first word serves as the flag
  if (p.split_k > 1) {
    f32x4 part[MT][1];
#pragma unroll
    for (int t = 0; t < MT; ++t) part[t][0] = acc[t];
    if (!splitk_reduce<MT, 1, kDecWaves * 64>(p, part, blockIdx.x, split, tid, reinterpret_cast<int*>(lds)))
      return;
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = part[t][0];
    __syncthreads();
  }
  // the eight partial tiles summed through LDS in wave order; wave t stores
  // activation tile t
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [wave][tile][64]
#pragma unroll
  for (int t = 0; t < MT; ++t) red[(wave * MT + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (wave >= MT) return;
  f32x4 sum = red[wave * 64 + lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += red[(w * MT + wave) * 64 + lane];
  const int64_t m = 16 * wave + r16;
  const float sa_m = (KIND == kChannelwise && m < p.M) ? p.sa[m] : 1.0f;
  store_out4<KIND>(p, m, n0 + 4 * g, sum, sa_m);
}

// ---------------------------------------------------------------------------
// Skinny kernel for M <= 16*MT: the weight is streamed from HBM exactly once.
// A workgroup of 8 waves owns one 16-row weight tile (16 output columns) and
// walks K in 4 KB chunks. For each chunk, wave w reads weight rows 2w and 2w+1
// with contiguous 1 KB load instructions (lane i takes bytes 16i..16i+15 of
// each 1 KB segment) -- reading 16 rows per instruction instead, as the MFMA
// operand layout would, measured markedly slower on HBM -- and the chunk is
// re-laid out through LDS ([16 rows][4096 B], 16-byte chunk c of row r at
// position c ^ r, so the 16 rows of one fragment read hit distinct banks).
// Wave w then runs the four 128-deep MFMAs of K bytes [512w, 512w+512) of the
// chunk, with the activation fragments loaded straight from global memory
// (cache-resident, rows >= M not loaded). The next chunk's loads are issued
// before the current chunk's MFMAs. The eight partial 16x16 tiles are summed
// through LDS in wave order (deterministic) and wave t stores row tile t.
// MFMA K assignment: lane group g = l/16 holds bytes [32g, 32g + 32) of each
// 128-byte K block for both operands.
// ---------------------------------------------------------------------------
namespace {
constexpr int kStreamWaves = 8;
constexpr int kStreamChunk = 4096;
}  // namespace

// v where ok, else zero (component-wise: a select on the whole struct goes
// through scratch memory)
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4& v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <int MT, int KIND>
struct StreamRegs {
  uint4 b[2][4];          // rows 2w, 2w+1; four 1 KB segments
  uint4 a[MT][4][2];      // activation fragments: 4 K blocks x 32 bytes
  // blockwise: this wave's four K blocks' weight scales and this lane's
  // activation scales (0 for rows >= M)
  float sb[KIND == kBlockwise ? 4 : 1];
  float sa[KIND == kBlockwise ? MT : 1][4];
};

// Loads of one chunk: the weight rows and (blockwise) the scales of the K
// blocks this wave multiplies, and, unless the quantization is fused (FQ),
// the activation code fragments. Every load is issued unconditionally from a
// clamped in-bounds address and the value selected afterwards: with no
// branches around loads the compiler's waits count exactly the loads still
// needed, so the next chunk's loads stay in flight across the MFMAs.
template <int MT, int KIND, bool FQ>
__device__ __forceinline__ void stream_load(const GemmArgs& p, StreamRegs<MT, KIND>& r, int64_t k0,
                                            int64_t n0, int wave, int lane) {
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int64_t n = n0 + 2 * wave + rr;
    const uint8_t* row = p.b + (n < p.N ? n : p.N - 1) * p.ldb;
#pragma unroll
    for (int sgm = 0; sgm < 4; ++sgm) {
      const int64_t off = k0 + sgm * 1024 + lane * 16;
      const bool ok = n < p.N && off < p.K;
      r.b[rr][sgm] = keep_if(ok, load16_nt(row + (ok ? off : 0)));
    }
  }
  const int g = lane >> 4;
  if constexpr (KIND == kBlockwise) {
    const int64_t kb_all = p.K / 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t kb = (k0 + wave * 512 + j * 128) / 128;
      kb = kb < kb_all ? kb : kb_all - 1;  // blocks past K are never used
      r.sb[j] = p.sb[(n0 / 128) * kb_all + kb];
      if constexpr (!FQ) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int64_t m = t * 16 + (lane & 15);
          const float v = p.sa[kb * p.sa_ld + (m < p.M ? m : p.M - 1)];
          r.sa[t][j] = m < p.M ? v : 0.0f;
        }
      }
    }
  }
  if constexpr (FQ) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = t * 16 + (lane & 15);
    const uint8_t* arow = p.a + (m < p.M ? m : p.M - 1) * p.lda;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t off = k0 + wave * 512 + j * 128 + g * 32;
      const bool ok0 = m < p.M && off < p.K;        // K is a multiple of 16 only
      const bool ok1 = m < p.M && off + 16 < p.K;
      r.a[t][j][0] = keep_if(ok0, load16(arow + (ok0 ? off : 0)));
      r.a[t][j][1] = keep_if(ok1, load16(arow + (ok1 ? off + 16 : 0)));
    }
  }
}

// Fused quantization (M <= FR): thread tid owns the 8-element unit tid of
// every row of a chunk (K elements [k0 + 8 tid, k0 + 8 tid + 8)), so the
// quantizing work grows with M, not with the 16-row MFMA tile. Its bf16 loads
// are issued before the chunk's weight loads: loads complete in issue order,
// so the quantization waits only for the (cache-resident) activation while
// the weight chunk is still arriving from HBM. QF holds the quantizer flags:
// with SiLU-and-mul the rows are [gate | up] (2K wide) and the up half of the
// unit is loaded into xu beside the gate; the SiLU itself runs when the unit
// is quantized, so these loads stay ahead of the weight loads.
template <int QF>
constexpr int fused_up_regs(int fr) { return (QF & kQuantSiluMul) != 0 ? fr : 1; }

template <int FR, int QF>
__device__ __forceinline__ void fused_load_x(const GemmArgs& p, const QuantArgs& qa, uint4 (&xr)[FR],
                                             uint4 (&xu)[fused_up_regs<QF>(FR)], int64_t k0, int tid) {
  const int64_t k = k0 + 8 * tid;
  const bool kin = k < p.K;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const bool ok = i < p.M && kin;
    const uint16_t* row = qa.x + (i < p.M ? i : p.M - 1) * qa.ldx;
    xr[i] = keep_if(ok, load16(row + (kin ? k : 0)));
    if constexpr ((QF & kQuantSiluMul) != 0) xu[i] = keep_if(ok, load16(row + p.K + (kin ? k : 0)));
  }
}

// The 8 bf16 values of a fused unit that are quantized: the loaded values, or
// silu(gate) * up correctly rounded to bf16 (zero where nothing was loaded).
template <int QF>
__device__ __forceinline__ uint4 fused_values(const uint4& g, const uint4& u) {
  if constexpr ((QF & kQuantSiluMul) != 0) return silu_mul8(g, u);
  else return g;
}

// Scale of a fused row or group from its |x| maximum, as the quantizers form it.
template <int QF>
__device__ __forceinline__ float fused_scale(float amax, float eps) {
  const float s = fmaxf(amax, eps) / kE4M3Max;
  return (QF & kQuantUe8m0) != 0 ? pow2_ceil(s) : s;
}

// Max over each aligned group of 16 lanes, with DPP lane moves (no LDS
// crossbar): xor 1 and xor 2 inside quads, then the 8-lane and 16-lane
// mirrors, each pairing the two halves whose maxima are already uniform.
__device__ __forceinline__ float max16_dpp(float v) {
  auto mv = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  v = fmaxf(v, mv(v, IntC<0xB1>()));   // quad_perm [1,0,3,2]
  v = fmaxf(v, mv(v, IntC<0x4E>()));   // quad_perm [2,3,0,1]
  v = fmaxf(v, mv(v, IntC<0x141>()));  // row_half_mirror
  v = fmaxf(v, mv(v, IntC<0x140>()));  // row_mirror
  return v;
}

// FR > 0: the activation quantization is fused, for M <= FR rows (FR a power
// of two, a compile-time row count so that the per-row work is straight-line
// code the compiler can interleave), with the quantizer flags QF.
template <int MT, int KIND, int FR, int QF = 0>
__global__ __launch_bounds__(kStreamWaves * 64) void gemm_skinny_kernel(GemmArgs p, QuantArgs qa) {
  constexpr bool FQ = FR > 0;
  constexpr bool SILU = (QF & kQuantSiluMul) != 0;
  static_assert(!FQ || (MT == 1 && FR <= 16), "the fused quantization serves one 16-row tile");
  static_assert(FQ || QF == 0, "quantizer flags belong to the fused quantization");
  constexpr int CPR = kStreamChunk / 16;  // 16-byte LDS chunks per chunk row
  constexpr int BPC = kStreamChunk / 128; // K blocks per chunk
  __shared__ uint4 wt[16 * CPR];          // 64 KB: one weight chunk
  // FQ: the activation codes of the chunk in the weight chunk's layout, their
  // group scales (blockwise) and the row scales (per token)
  __shared__ uint4 codes[FQ ? 16 * CPR : 1];
  __shared__ float blk_scale[FQ ? 16 * BPC : 1];
  __shared__ float row_scale[FQ ? 16 : 1], row_inv[FQ ? 16 : 1];
  __shared__ float row_part[FQ ? kStreamWaves * 16 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  // with FQ, workgroup 0 also stores the codes and scales it computes
  const bool writer = FQ && blockIdx.x == 0;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 xr[FQ ? FR : 1];
  uint4 xu[FQ ? fused_up_regs<QF>(FR) : 1];
  if constexpr (FQ) fused_load_x<FR, QF>(p, qa, xr, xu, 0, tid);
  StreamRegs<MT, KIND> cur;
  stream_load<MT, KIND, FQ>(p, cur, 0, n0, wave, lane);

  // FQ: quantize the chunk whose activation is in xr into `codes` (16-byte
  // chunk c of row i at position c ^ i, as the weights; unit tid is bytes
  // 8 tid .. +7 of the row) and, blockwise, its group scales into blk_scale.
  // Rows M..FR-1 quantize zeros; K past the end gives zero codes, as in the
  // unfused path.
  auto quantize_chunk = [&](int64_t k0) {
    if constexpr (FQ) {
      const int64_t k = k0 + 8 * tid;
      const int pos = ((tid >> 1) << 4) + ((tid & 1) << 3);
      const bool kin = k < p.K;
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const uint4 v = fused_values<QF>(xr[i], xu[SILU ? i : 0]);
        float sc, y;
        if constexpr (KIND == kChannelwise) {
          sc = row_scale[i];
          y = row_inv[i];
        } else {  // group of 128 = 16 consecutive threads
          sc = fused_scale<QF>(max16_dpp(absmax8_bf16(v)), qa.eps);
          y = 1.0f / sc;
        }
        const uint2 c = kin ? quant8_bf16(v, sc, y) : make_uint2(0, 0);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(codes) + i * (CPR * 16) +
                                  (pos ^ (i << 4))) = c;
        if (KIND == kBlockwise && (tid & 15) == 0) blk_scale[i * BPC + (tid >> 4)] = sc;
        if (writer && kin && i < p.M) {
          *reinterpret_cast<uint2*>(qa.q + i * qa.ldq + k) = c;
          if (KIND == kBlockwise && (tid & 15) == 0) qa.scale[(k / 128) * qa.scale_ld + i] = sc;
        }
      }
    }
  };

  if constexpr (FQ) {
    // code rows FR..15 and their scales stay zero; no output of theirs is stored
    for (int idx = tid + FR * CPR; idx < 16 * CPR; idx += kStreamWaves * 64)
      codes[idx] = make_uint4(0, 0, 0, 0);
    for (int idx = tid + FR * BPC; idx < 16 * BPC; idx += kStreamWaves * 64) blk_scale[idx] = 0.0f;
    if constexpr (KIND == kChannelwise) {
      // per-token scales: absmax over the whole row (chunks after the first
      // are read here once more), reduced over the workgroup through LDS
      float am[FR];
#pragma unroll
      for (int i = 0; i < FR; ++i)  // zero where not loaded
        am[i] = absmax8_bf16(fused_values<QF>(xr[i], xu[SILU ? i : 0]));
      for (int64_t k1 = kStreamChunk; k1 < p.K; k1 += kStreamChunk) {
        uint4 xn[FR], xnu[fused_up_regs<QF>(FR)];
        fused_load_x<FR, QF>(p, qa, xn, xnu, k1, tid);
#pragma unroll
        for (int i = 0; i < FR; ++i)
          am[i] = fmaxf(am[i], absmax8_bf16(fused_values<QF>(xn[i], xnu[SILU ? i : 0])));
      }
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const float w = wave_max(am[i]);
        if (lane == 0) row_part[wave * 16 + i] = w;
      }
      __syncthreads();
      if (tid < FR) {
        float mx = row_part[tid];
        for (int w = 1; w < kStreamWaves; ++w) mx = fmaxf(mx, row_part[w * 16 + tid]);
        const float sc = fused_scale<QF>(mx, qa.eps);
        row_scale[tid] = sc;
        row_inv[tid] = 1.0f / sc;
        if (writer && tid < p.M) qa.scale[tid] = sc;
      }
      __syncthreads();
    }
    quantize_chunk(0);
  }

  for (int64_t k0 = 0; k0 < p.K; k0 += kStreamChunk) {
    __syncthreads();  // the previous chunk's fragment reads are done; (FQ) codes are in
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = 2 * wave + rr;
#pragma unroll
      for (int sgm = 0; sgm < 4; ++sgm) {
        const int c = sgm * 64 + lane;
        wt[r * CPR + (c ^ r)] = cur.b[rr][sgm];
      }
    }
    __syncthreads();
    StreamRegs<MT, KIND> use = cur;
    const bool more = k0 + kStreamChunk < p.K;
    if (more) {
      if constexpr (FQ) fused_load_x<FR, QF>(p, qa, xr, xu, k0 + kStreamChunk, tid);
      stream_load<MT, KIND, FQ>(p, cur, k0 + kStreamChunk, n0, wave, lane);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kbase = k0 + wave * 512 + j * 128;
      if (kbase >= p.K) break;
      const int c0 = (wave * 512 + j * 128 + g * 32) / 16;
      const uint4 lo = wt[r16 * CPR + (c0 ^ r16)];
      const uint4 hi = wt[r16 * CPR + ((c0 + 1) ^ r16)];
      const i32x8 bf = join(lo, hi);
      // activation codes of this K block and (blockwise) their group scales
      i32x8 af[MT];
      float sa_blk[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if constexpr (FQ) {
          af[t] = join(codes[r16 * CPR + (c0 ^ r16)], codes[r16 * CPR + ((c0 + 1) ^ r16)]);
          if (KIND == kBlockwise) sa_blk[t] = blk_scale[r16 * BPC + wave * 4 + j];
        } else {
          af[t] = join(use.a[t][j][0], use.a[t][j][1]);
          if (KIND == kBlockwise) sa_blk[t] = use.sa[t][j];
        }
      }
      if constexpr (KIND == kChannelwise) {
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = mfma_fp8(bf, af[t], acc[t]);
      } else {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const f32x4 part = mfma_fp8(bf, af[t], f32x4{0.f, 0.f, 0.f, 0.f});
          acc[t] += part * (sa_blk[t] * use.sb[j]);
        }
      }
    }
    if constexpr (FQ) {
      if (more) {
        __syncthreads();  // every wave is done with this chunk's codes
        quantize_chunk(k0 + kStreamChunk);
      }
    }
  }

  // cross-wave reduction through the (now idle) weight buffer
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(wt);  // [W][MT][64]
#pragma unroll
  for (int t = 0; t < MT; ++t) red[(wave * MT + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (wave >= MT) return;
  const int t = wave;
  f32x4 sum = red[t * 64 + lane];
#pragma unroll
  for (int w = 1; w < kStreamWaves; ++w) sum += red[(w * MT + t) * 64 + lane];
  const int64_t m = t * 16 + r16;
  float sa_m = 1.0f;
  if (KIND == kChannelwise && m < p.M) sa_m = FQ ? row_scale[r16] : p.sa[m];
  store_out4<KIND>(p, m, n0 + 4 * g, sum, sa_m);
}

// ---------------------------------------------------------------------------
// The decode stream with the activation quantization fused, for the single-
// launch linear (M <= FR rows, FR in {1, 2, 4}; quantizer flags QF). Every
// workgroup quantizes the whole activation and then streams the weight as
// gemm_decode_kernel does (per-wave rings), with slots of weight rows only and
// the activation fragments read from an LDS copy of the codes ([FR][K], 16-byte
// chunk c of row i at position c ^ i). Codes, scales and MFMAs, and their
// order, are those of the quantization kernels followed by
// gemm_decode_kernel, so the outputs are the same bits; workgroup 0 also
// stores the codes (rows < M) and scales. The bf16 rows travel by LDS-DMA
// into a staging area (which the codes then overwrite), issued before the
// weight's first blocks: each wave waits for its own activation copies
// only, so the quantization runs while those blocks are in flight and no
// compiler wait for an ordinary load ever holds back the stream. Thread t
// owns the 8-value units t + 512 u of every row (K positions 8 (t + 512 u)
// .. +7), held in registers from the row maximum to the quantization: at
// most kDecFusedUnits units over the FR rows (FR ceil(K / 4096) <= 8).
// ---------------------------------------------------------------------------
namespace {
constexpr int kDecFusedUnits = 8;
}  // namespace

__host__ __device__ inline int64_t decode_fused_rows(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// Bytes of LDS past the ring: the staging area of the bf16 rows ([FR][2K],
// with SiLU-and-mul [FR][4K]; the codes [FR][K] overwrite its start), the
// scale tables (blockwise: weight block scales in 64-float pieces, activation
// group scales [K/128][FR]; per token: row scales and their inverses) and the
// row-maximum partials.
__host__ __device__ inline size_t decode_fused_fixed_bytes(int64_t K, int kind, int64_t fr, bool silu) {
  const int64_t kb = K / 128;
  size_t b = (size_t)(fr * K * (silu ? 4 : 2));
  if (kind != kChannelwise) b += (size_t)((kb + 63) / 64) * 256 + (size_t)(kb * fr) * 4;
  b += (size_t)(2 * fr + kDecWaves * fr) * 4;
  return b;
}

// The 16-byte LDS-DMA from a per-lane 64-bit address (lane l's 16 bytes land
// at M0 + 16 l).
__device__ __forceinline__ void lds_dma16_v(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0v) : "memory", "m0");
}

template <int KIND, int FR, int QF>
__global__ __launch_bounds__(kDecWaves * 64) void gemm_decode_fused_kernel(GemmArgs p, QuantArgs qa) {
  static_assert(KIND == kChannelwise || KIND == kBlockwise, "fp32 scales");
  static_assert(FR == 1 || FR == 2 || FR == 4, "row buckets");
  constexpr bool SILU = (QF & kQuantSiluMul) != 0;
  constexpr int UM = kDecFusedUnits / FR;  // units per thread and row, at most
  constexpr int NT = kDecWaves * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int M = (int)p.M;
  const int64_t K = p.K, kb_all = K / 128;
  const int R = p.ring_slots;  // slots per wave (2 KB of weight rows each), 2 .. kDecMaxWaveSlots
  const int nb = decode_wave_blocks(kb_all, wave);
  const int nu = (int)((K / 8 + NT - 1) / NT);  // <= UM (checked on the host)
  const bool writer = blockIdx.x == 0;
  const int64_t RB = K * (SILU ? 4 : 2);  // staged bytes per row
  const uint32_t ring = (uint32_t)kDecWaves * R * 2048;
  uint8_t* stage = lds + ring;
  uint8_t* codes = stage;  // after the staged rows are read
  float* tail = reinterpret_cast<float*>(stage + (size_t)FR * RB);
  const int64_t sb_pieces = KIND == kBlockwise ? (kb_all + 63) / 64 : 0;
  float* sbt = tail;                      // blockwise: weight block scales [kb_all]
  float* sat = tail + sb_pieces * 64;     // blockwise: group scales [kb_all][FR]
  float* row_scale = sat + (KIND == kBlockwise ? kb_all * FR : 0);
  float* row_inv = row_scale + FR;
  float* row_part = row_inv + FR;         // [wave][FR]

  // 1. the bf16 rows < M ([M][RB] bytes, 1 KB per copy), the weight block
  // scales (blockwise) and this wave's first weight blocks, in that order
  const int64_t xbytes = (int64_t)M * RB, xpieces = (xbytes + 1023) / 1024;
  const uint32_t stage_lds = lds_base + ring;
  for (int64_t pc = wave; pc < xpieces; pc += kDecWaves) {
    const int64_t b = pc * 1024 + lane * 16;
    if (b < xbytes) {
      const int64_t row = b / RB;
      lds_dma16_v(reinterpret_cast<const uint8_t*>(qa.x) + row * qa.ldx * 2 + (b - row * RB),
                  stage_lds + (uint32_t)(pc * 1024));
    }
  }
  int younger = 0;  // this wave's copies issued after its activation copies
  if constexpr (KIND == kBlockwise) {
    const int64_t nb = n0 >> 7;
    for (int64_t i = wave; i < sb_pieces; i += kDecWaves) {
      const int64_t kb = i * 64 + lane;
      lds_dma4_v(p.sb + nb * kb_all + (kb < kb_all ? kb : 0),
                 (uint32_t)(uintptr_t)sbt + (uint32_t)(i * 256));
      ++younger;
    }
  }
  // this wave's blocks as in gemm_decode_kernel, weight rows only (lane l
  // of instruction t: row 8 t + l / 8, chunk position l % 8 holding logical
  // chunk (l % 8) ^ (l / 8))
  const int lr = lane >> 3;
  const uint32_t chunk = (uint32_t)(((lane & 7) ^ lr) << 4);
  const uint32_t wbase = lds_base + (uint32_t)wave * R * 2048;
  auto issue = [&](int i) {
    const int64_t kb = decode_wave_kb(i, wave);
    const uint32_t slot = wbase + (uint32_t)(i % R) * 2048;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int64_t n = n0 + 8 * t + lr;
      n = n < p.N ? n : p.N - 1;
      lds_dma16_s(p.b, (uint32_t)(n * p.ldb + kb * 128) + chunk, slot + (uint32_t)t * 1024);
    }
  };
  const int pro = R - 1 < nb ? R - 1 : nb;
  for (int i = 0; i < pro; ++i) {
    issue(i);
    younger += 2;
  }
  wait_vmcnt_upto<0, 63>(younger);  // this wave's activation copies have landed
  wait_vmcnt_lgkm0<63>();
  __syncthreads();

  // 2. this thread's units (zero outside rows < M and K)
  uint4 xv[FR][UM];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int u = 0; u < UM; ++u) {
      if (u < nu) {
        const int64_t j = (int64_t)tid + (int64_t)NT * u;
        const bool ok = i < M && 8 * j < K;
        const uint8_t* src = stage + (size_t)(i < M ? i : 0) * RB + (size_t)(8 * j < K ? j : 0) * 16;
        const uint4 gv = *reinterpret_cast<const uint4*>(src);
        if constexpr (SILU) {
          const uint4 uv = *reinterpret_cast<const uint4*>(src + 2 * K);
          xv[i][u] = keep_if(ok, fused_values<QF>(gv, uv));
        } else {
          xv[i][u] = keep_if(ok, gv);
        }
      }
    }

  // 3. quantize into `codes` (over the staging area: every thread has read
  // its units before the first code is written; rows M..FR-1 and K past the
  // end give zero codes)
  auto put = [&](int i, int64_t k, uint2 c) {
    const int64_t cc = k >> 4;  // 16-byte chunk
    *reinterpret_cast<uint2*>(codes + (size_t)i * K + (size_t)((cc ^ i) << 4) + ((k >> 3) & 1) * 8) = c;
    if (writer && i < M) *reinterpret_cast<uint2*>(qa.q + (int64_t)i * qa.ldq + k) = c;
  };
  if constexpr (KIND == kChannelwise) {
    float am[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      am[i] = 0.0f;
#pragma unroll
      for (int u = 0; u < UM; ++u)
        if (u < nu) am[i] = fmaxf(am[i], absmax8_bf16(xv[i][u]));
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const float w = wave_max(am[i]);
      if (lane == 0) row_part[wave * FR + i] = w;
    }
    __syncthreads();
    if (tid < FR) {
      float mx = row_part[tid];
      for (int w = 1; w < kDecWaves; ++w) mx = fmaxf(mx, row_part[w * FR + tid]);
      const float sc = fused_scale<QF>(mx, qa.eps);
      row_scale[tid] = sc;
      row_inv[tid] = 1.0f / sc;
      if (writer && tid < M) qa.scale[tid] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const float sc = row_scale[i], y = row_inv[i];
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        if (u < nu) {
          const int64_t k = 8 * ((int64_t)tid + (int64_t)NT * u);
          if (k < K) put(i, k, quant8_bf16(xv[i][u], sc, y));
        }
      }
    }
  } else {
    __syncthreads();  // the staged rows are read
#pragma unroll
    for (int i = 0; i < FR; ++i) {
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        if (u < nu) {
          // a group of 128 values is 16 consecutive threads' units
          const int64_t k = 8 * ((int64_t)tid + (int64_t)NT * u);
          const float sc = fused_scale<QF>(max16_dpp(absmax8_bf16(xv[i][u])), qa.eps);
          const float y = 1.0f / sc;
          if (k < K) {
            put(i, k, quant8_bf16(xv[i][u], sc, y));
            if ((tid & 15) == 0) {
              sat[(k >> 7) * FR + i] = sc;
              if (writer && i < M) qa.scale[(k >> 7) * qa.scale_ld + i] = sc;
            }
          }
        }
      }
    }
  }
  // workgroup 0's stores of codes and scales count with its copies; they
  // are waited for here, so that the stream's waits count copies only
  if (writer) wait_vmcnt<0>();
  __syncthreads();

  // 5. the weight stream (as gemm_decode_kernel: the same K blocks per wave
  // in the same order)
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int am = r16 < M ? r16 : M - 1;
  const uint32_t fb0 = (uint32_t)r16 * 128 + (uint32_t)(((2 * g) ^ (r16 & 7)) << 4);
  const uint32_t fb1 = (uint32_t)r16 * 128 + (uint32_t)(((2 * g + 1) ^ (r16 & 7)) << 4);
  const uint8_t* arow = codes + (size_t)am * K;
  const uint8_t* wl = lds + (size_t)wave * R * 2048;
  for (int i = 0; i < nb; ++i) {
    const int last = i + R - 2 < nb - 1 ? i + R - 2 : nb - 1;
    wait_vmcnt_upto<0, 63>((last - i) * 2);
    if (i + R - 1 < nb) issue(i + R - 1);
    const int64_t kb = decode_wave_kb(i, wave);
    const uint8_t* slot = wl + (size_t)(i % R) * 2048;
    const i32x8 bf = join(*reinterpret_cast<const uint4*>(slot + fb0), *reinterpret_cast<const uint4*>(slot + fb1));
    const int64_t c0 = kb * 8 + 2 * g;
    const i32x8 af = join(*reinterpret_cast<const uint4*>(arow + ((c0 ^ am) << 4)),
                          *reinterpret_cast<const uint4*>(arow + (((c0 + 1) ^ am) << 4)));
    if constexpr (KIND == kChannelwise) {
      acc = mfma_fp8(bf, af, acc);
    } else {
      const f32x4 part = mfma_fp8(bf, af, f32x4{0.f, 0.f, 0.f, 0.f});
      acc += part * (sat[kb * FR + am] * sbt[kb]);
    }
  }

  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [wave][64]
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = red[lane];
#pragma unroll
  for (int w = 1; w < kDecWaves; ++w) sum += red[w * 64 + lane];
  const int64_t m = r16;
  const float sa_m = (KIND == kChannelwise && m < p.M) ? row_scale[r16] : 1.0f;
  store_out4<KIND>(p, m, n0 + 4 * g, sum, sa_m);
}

// ---------------------------------------------------------------------------
// Variant table and launch.
// ---------------------------------------------------------------------------
namespace {

template <int BM, int BN, int WM, int WN, int BK, int KIND>
hipError_t launch_tile(const GemmArgs& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const size_t lds = (size_t)2 * (BM + BN) * BK;
  auto kern = gemm_tile_kernel<BM, BN, WM, WN, BK, KIND>;
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

template <int BM, int BN, int WM, int WN, int KIND, int NP>
hipError_t launch_panel(const GemmArgs& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const size_t lds = (size_t)panel_lds_bytes<BM, BN, WM, WN, KIND, NP>();
  auto kern = gemm_panel_kernel<BM, BN, WM, WN, KIND, NP>;
  static bool lds_attr_set = false;
  if (lds > 65536 && !lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  const unsigned experts = p.masked_m ? (unsigned)p.experts : 1u;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)p.split_k, experts), dim3(WM * WN * 64),
                     lds, stream, p);
  return hipGetLastError();
}


template <int KIND>
hipError_t launch_pingpong(const GemmArgs& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const size_t lds = (size_t)pingpong_lds_bytes<KIND>();
  auto kern = gemm_pingpong_kernel<KIND>;
  static bool lds_attr_set = false;
  if (!lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  const unsigned experts = p.masked_m ? (unsigned)p.experts : 1u;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)p.split_k, experts), dim3(512), lds, stream, p);
  return hipGetLastError();
}

// The decode stream takes whole 128-deep K blocks, 32-bit DMA offsets (the
// last byte of the last row of either operand within 2^32 - 1) and two ring
// slots per wave beside its scale table in the LDS.
template <int KIND>
bool decode_eligible(const GemmArgs& p) {
  const uint64_t lim = 0xFFFFFFFFull;
  return p.K % 128 == 0 && (uint64_t)(p.N - 1) * (uint64_t)p.ldb + (uint64_t)p.K <= lim &&
         (uint64_t)(p.M - 1) * (uint64_t)p.lda + (uint64_t)p.K <= lim &&
         2 * kDecWaves * decode_slot_bytes(p.M) + decode_scale_bytes(p.K, KIND, p.M) <= 163840;
}

template <int KIND, int MT>
hipError_t launch_decode_t(const GemmArgs& p, hipStream_t stream) {
  auto kern = gemm_decode_kernel<KIND, MT>;
  static bool lds_attr_set = false;
  if (!lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  // slots per wave: one round of workgroups over the compute units, as many
  // as fit 160 KB (at most kDecMaxWaveSlots); more workgroups, as many as fit
  // 80 KB (two per compute unit); never more than a wave has blocks, plus one
  const int64_t tiles = (p.N + 15) / 16;
  const size_t fixed = decode_scale_bytes(p.K, KIND, p.M), slot = decode_slot_bytes(p.M) * kDecWaves;
  const size_t budget = (tiles <= 256 ? (size_t)163840 : (size_t)81920);
  int64_t ns = budget > fixed ? (int64_t)((budget - fixed) / slot) : 0;
  int64_t per_wave = ((p.K / 128) + kDecWaves - 1) / kDecWaves;
  if (p.split_k > 1 && p.k_tiles_per_split < per_wave) per_wave = p.k_tiles_per_split;
  if (ns > per_wave + 1) ns = per_wave + 1;
  if (ns > kDecMaxWaveSlots) ns = kDecMaxWaveSlots;
  if (ns < 2) ns = 2;
  const size_t lds = (size_t)ns * slot + fixed;
  if (lds > 163840) return hipErrorInvalidValue;
  GemmArgs q = p;
  q.ring_slots = (int)ns;
  if (q.split_k < 1) q.split_k = 1;
  if (q.split_k == 1) q.k_tiles_per_split = (int)(4 * ((p.K / 128 + 31) / 32));  // every block
  if (q.split_k > 1 && tiles > kMaxSplitTiles) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles, (unsigned)q.split_k), dim3(kDecWaves * 64), lds, stream, q);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_decode(const GemmArgs& p, hipStream_t stream) {
  switch (decode_tiles(p.M)) {
    case 1: return launch_decode_t<KIND, 1>(p, stream);
    case 2: return launch_decode_t<KIND, 2>(p, stream);
    default: return launch_decode_t<KIND, 4>(p, stream);
  }
}

template <int BM, int BN, int WM, int WN, int NSTAGE>
hipError_t launch_dma(const GemmArgs& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  const size_t lds = (size_t)NSTAGE * (BM + BN) * 64;
  auto kern = gemm_dma_kernel<BM, BN, WM, WN, NSTAGE>;
  static bool lds_attr_set = false;
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

// The LDS-DMA tiles take whole 64-byte K stages, channelwise scales only, and
// per-lane row offsets that fit the 32-bit offset of the DMA instruction.
template <int KIND>
bool dma_eligible(const GemmArgs& p) {
  const uint64_t lim = 0xFFFFFFFFull - 64;
  return KIND == kChannelwise && p.K % 64 == 0 && (uint64_t)(p.M - 1) * (uint64_t)p.lda <= lim &&
         (uint64_t)(p.N - 1) * (uint64_t)p.ldb <= lim;
}

// The panel tiles take whole 128-byte K stages and 32-bit DMA row offsets
// (blockwise: also within each activation-scale column).
template <int KIND>
bool panel_eligible(const GemmArgs& p) {
  const uint64_t lim = 0xFFFFFFFFull - 128;
  if (p.K % 128 != 0 || (uint64_t)(p.M - 1) * (uint64_t)p.lda > lim ||
      (uint64_t)(p.N - 1) * (uint64_t)p.ldb > lim)
    return false;
  if (KIND == kBlockwise) return (uint64_t)p.sa_ld * 4 <= lim;
  return true;
}

// The 256x256 tile where nothing else is asked for by name: channelwise the
// 8-wave register-staged kernel; blockwise the ping-pong tile, or, past the
// panel tiles' 32-bit DMA offsets, the 8-wave 128x128
// register-staged kernel (the register-staged 256x256 blockwise kernels do
// not fit their registers). Its split-K partials of 128x128 tiles fill the
// workspace planned for 256x256 ones exactly or less.
template <int KIND>
hipError_t launch_256(const GemmArgs& p, hipStream_t stream);


template <int KIND>
hipError_t launch_kind(int variant, const GemmArgs& p, hipStream_t stream) {
  switch (variant) {
    case 0: {  // FP8_VARIANT_SKINNY
      const dim3 grid((unsigned)((p.N + 15) / 16)), block(kStreamWaves * 64);
      const QuantArgs none{};
      if (p.M <= 16)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, KIND, 0>), grid, block, 0, stream, p, none);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<2, KIND, 0>), grid, block, 0, stream, p, none);
      return hipGetLastError();
    }
    case 1: return launch_tile<64, 64, 2, 2, 512, KIND>(p, stream);
    case 2: return launch_tile<128, 128, 2, 2, 128, KIND>(p, stream);
    case 3: return launch_tile<256, 128, 2, 2, 128, KIND>(p, stream);
    // the 4-wave 256x256 tile spilled its accumulators: both names take the
    // 8-wave one
    case 4:
    case 5: return launch_256<KIND>(p, stream);
    case 6: return launch_tile<256, 128, 4, 2, 128, KIND>(p, stream);
    case 7: return launch_tile<128, 128, 2, 4, 128, KIND>(p, stream);
    case 8: return launch_tile<128, 64, 2, 2, 256, KIND>(p, stream);
    case 9: return launch_tile<64, 128, 2, 2, 256, KIND>(p, stream);
    case 10: return launch_tile<128, 128, 2, 2, 256, KIND>(p, stream);
    case 11:
      if (!dma_eligible<KIND>(p)) return launch_256<KIND>(p, stream);
      return launch_dma<256, 256, 2, 4, 4>(p, stream);
    case 12:
      if (!dma_eligible<KIND>(p)) return launch_tile<256, 128, 4, 2, 128, KIND>(p, stream);
      return launch_dma<256, 128, 4, 2, 4>(p, stream);
    case 13:
      if (!dma_eligible<KIND>(p)) return launch_tile<128, 128, 2, 2, 256, KIND>(p, stream);
      return launch_dma<128, 128, 2, 2, 4>(p, stream);
    // panel variants: the fallbacks keep the tile shape and the 128-deep
    // stages the split plan counts in
    case 14:
      if (KIND != kChannelwise || !panel_eligible<KIND>(p)) return launch_256<KIND>(p, stream);
      return launch_pingpong<kChannelwise>(p, stream);
    case 15:
      if (!panel_eligible<KIND>(p)) return launch_tile<256, 128, 4, 2, 128, KIND>(p, stream);
      return launch_panel<256, 128, 4, 2, KIND, 5>(p, stream);
    case 16:
      if (!panel_eligible<KIND>(p)) return launch_tile<128, 128, 2, 2, 128, KIND>(p, stream);
      return launch_panel<128, 128, 2, 2, KIND, 5>(p, stream);
    case 17:
      if (!panel_eligible<KIND>(p)) return launch_tile<128, 64, 2, 2, 128, KIND>(p, stream);
      return launch_panel<128, 64, 2, 2, KIND, 5>(p, stream);
    case 18:
      if (!panel_eligible<KIND>(p)) return launch_tile<64, 64, 2, 2, 128, KIND>(p, stream);
      return launch_panel<64, 64, 2, 2, KIND, 5>(p, stream);
    case 19:
      if (!panel_eligible<KIND>(p)) return launch_tile<64, 64, 2, 2, 128, KIND>(p, stream);
      return launch_panel<64, 64, 2, 2, KIND, 9>(p, stream);
    case 20:
      if (!panel_eligible<KIND>(p)) return launch_tile<128, 64, 2, 2, 128, KIND>(p, stream);
      return launch_panel<128, 64, 2, 2, KIND, 7>(p, stream);
    case 21:
      if (!panel_eligible<KIND>(p)) return launch_tile<128, 128, 2, 4, 128, KIND>(p, stream);
      return launch_panel<128, 128, 2, 4, KIND, 5>(p, stream);
    case 22:
      if (!panel_eligible<KIND>(p)) return launch_tile<128, 64, 4, 2, 128, KIND>(p, stream);
      return launch_panel<128, 64, 4, 2, KIND, 5>(p, stream);
    // narrow deep-ring tiles for small M: more workgroups at the same bytes per CU
    case 23:
      if (!panel_eligible<KIND>(p)) return launch_tile<32, 32, 1, 1, 128, KIND>(p, stream);
      return launch_panel<32, 32, 1, 1, KIND, 9>(p, stream);
    case 24:
      if (!panel_eligible<KIND>(p)) return launch_tile<64, 32, 2, 1, 128, KIND>(p, stream);
      return launch_panel<64, 32, 2, 1, KIND, 7>(p, stream);
    // the ping-pong 256x256 tile on 16x16x128 MFMAs, either kind (blockwise
    // through launch_256, which keeps its fallbacks)
    case 25:
      if (KIND == kBlockwise || !panel_eligible<KIND>(p)) return launch_256<KIND>(p, stream);
      return launch_pingpong<kChannelwise>(p, stream);
    case 26: {  // FP8_VARIANT_DECODE
      if (p.M > 64) return hipErrorInvalidValue;
      if (decode_eligible<KIND>(p)) return launch_decode<KIND>(p, stream);
      // past its DMA offsets or its LDS: the skinny kernel (M <= 32; the same
      // sums when unsplit), else the 64x64 tile, unsplit
      GemmArgs q = p;
      q.split_k = 1;
      q.k_tiles_per_split = (int)(p.K / 128);
      if (p.M <= 32) {
        if (p.M <= 16)
          hipLaunchKernelGGL((gemm_skinny_kernel<1, KIND, 0>), dim3((unsigned)((p.N + 15) / 16)),
                             dim3(kStreamWaves * 64), 0, stream, q, QuantArgs{});
        else
          hipLaunchKernelGGL((gemm_skinny_kernel<2, KIND, 0>), dim3((unsigned)((p.N + 15) / 16)),
                             dim3(kStreamWaves * 64), 0, stream, q, QuantArgs{});
        return hipGetLastError();
      }
      q.k_tiles_per_split = (int)((p.K + 511) / 512);
      return launch_tile<64, 64, 2, 2, 512, KIND>(q, stream);
    }
    default: return hipErrorInvalidValue;
  }
}

template <int KIND>
hipError_t launch_256(const GemmArgs& p, hipStream_t stream) {
  if constexpr (KIND == kChannelwise) {
    return launch_tile<256, 256, 2, 4, 128, KIND>(p, stream);
  } else {
    if (panel_eligible<KIND>(p)) return launch_pingpong<kBlockwise>(p, stream);
    if (p.split_k > 1 && ((p.M + 127) / 128) * ((p.N + 127) / 128) > kMaxSplitTiles) return hipErrorInvalidValue;
    return launch_tile<128, 128, 2, 4, 128, KIND>(p, stream);
  }
}
}  // namespace

VariantInfo variant_info(int variant) {
  switch (variant) {
    case 0: return {32, 16, 4096, 8, true};
    case 1: return {64, 64, 512, 4, true};
    case 2: return {128, 128, 128, 4, true};
    case 3: return {256, 128, 128, 4, true};
    case 4: return {256, 256, 128, 8, true};
    case 5: return {256, 256, 128, 8, true};
    case 6: return {256, 128, 128, 8, true};
    case 7: return {128, 128, 128, 8, true};
    case 8: return {128, 64, 256, 4, true};
    case 9: return {64, 128, 256, 4, true};
    case 10: return {128, 128, 256, 4, true};
    // deep-pipeline (LDS-DMA) variants, channelwise with K % 64 == 0; other
    // requests run the register-staged kernel of the same tile shape
    case 11: return {256, 256, 64, 8, true};
    case 12: return {256, 128, 64, 8, true};
    case 13: return {128, 128, 64, 4, true};
    // panel-ring LDS-DMA variant, channelwise with K % 128 == 0
    case 14: return {256, 256, 128, 8, true};
    case 15: return {256, 128, 128, 8, true};
    case 16: return {128, 128, 128, 4, true};
    case 17: return {128, 64, 128, 4, true};
    case 18: return {64, 64, 128, 4, true};
    case 19: return {64, 64, 128, 4, true};
    case 20: return {128, 64, 128, 4, true};
    case 21: return {128, 128, 128, 8, true};
    case 22: return {128, 64, 128, 8, true};
    case 23: return {32, 32, 128, 1, true};
    case 24: return {64, 32, 128, 2, true};
    case 25: return {256, 256, 128, 8, true};
    case 26: return {64, 16, 1024, 8, true};
    default: return {0, 0, 0, 0, false};
  }
}

int64_t variant_tiles(int variant, int64_t M, int64_t N) {
  const VariantInfo v = variant_info(variant);
  if (!v.exists) return 0;
  if (variant == 0 || variant == 26) return (N + 15) / 16;
  return ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
}

// Blocks per wave of the decode stream (wave 0 has the most) and the split
// plan over them: `per` blocks per split, `splits` splits (<= split_k).
void decode_split_plan(int64_t K, int split_k, int* splits, int* per) {
  const int64_t kb_all = K / 128;
  const int64_t nbw = 4 * (kb_all / 32) + (kb_all % 32 < 4 ? kb_all % 32 : 4);
  int64_t s = split_k < 1 ? 1 : split_k;
  if (s > nbw) s = nbw > 0 ? nbw : 1;
  const int64_t pr = nbw > 0 ? (nbw + s - 1) / s : 1;
  *per = (int)pr;
  *splits = (int)(nbw > 0 ? (nbw + pr - 1) / pr : 1);
}

size_t variant_workspace_bytes(int variant, int split_k, int64_t M, int64_t N) {
  if (split_k <= 1 || variant == 0) return 0;
  if (variant == 26)  // one 16-byte partial per thread of the 512 and activation tile, per tile and split
    return kCounterBytes + (size_t)((N + 15) / 16) * split_k * decode_tiles(M) * kDecWaves * 64 * 16;
  const VariantInfo v = variant_info(variant);
  const int64_t tiles = variant_tiles(variant, M, N);
  return kCounterBytes + (size_t)tiles * split_k * v.bm * v.bn * sizeof(float);
}

namespace {
template <int KIND, int FR, int QF>
hipError_t launch_fused_rows(const GemmArgs& p, const QuantArgs& qa, hipStream_t stream) {
  const dim3 grid((unsigned)((p.N + 15) / 16)), block(kStreamWaves * 64);
  hipLaunchKernelGGL((gemm_skinny_kernel<1, KIND, FR, QF>), grid, block, 0, stream, p, qa);
  return hipGetLastError();
}

template <int KIND, int FR, int QF>
hipError_t launch_decode_fused_rows(const GemmArgs& p, const QuantArgs& qa, hipStream_t stream) {
  auto kern = gemm_decode_fused_kernel<KIND, FR, QF>;
  static bool lds_attr_set = false;
  if (!lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    if (e != hipSuccess) return e;
    lds_attr_set = true;
  }
  // ring depth as for the unfused stream (slots of 2 KB per wave: weight rows only)
  const int64_t tiles = (p.N + 15) / 16;
  const size_t fixed = decode_fused_fixed_bytes(p.K, KIND, FR, (QF & kQuantSiluMul) != 0);
  const size_t budget = tiles <= 256 ? (size_t)163840 : (size_t)81920;
  int64_t ns = budget > fixed ? (int64_t)((budget - fixed) / (kDecWaves * 2048)) : 0;
  const int64_t per_wave = ((p.K / 128) + kDecWaves - 1) / kDecWaves;
  if (ns > per_wave + 1) ns = per_wave + 1;
  if (ns > kDecMaxWaveSlots) ns = kDecMaxWaveSlots;
  if (ns < 2) ns = 2;
  const size_t lds = (size_t)ns * kDecWaves * 2048 + fixed;
  if (lds > 163840) return hipErrorInvalidValue;
  GemmArgs q = p;
  q.ring_slots = (int)ns;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kDecWaves * 64), lds, stream, q, qa);
  return hipGetLastError();
}

template <int KIND, int QF>
hipError_t launch_decode_fused_kind(const GemmArgs& p, const QuantArgs& qa, hipStream_t stream) {
  if (p.M <= 1) return launch_decode_fused_rows<KIND, 1, QF>(p, qa, stream);
  if (p.M <= 2) return launch_decode_fused_rows<KIND, 2, QF>(p, qa, stream);
  if (p.M <= 4) return launch_decode_fused_rows<KIND, 4, QF>(p, qa, stream);
  return hipErrorInvalidValue;
}

template <int KIND, int QF>
hipError_t launch_fused_kind(const GemmArgs& p, const QuantArgs& qa, hipStream_t stream) {
  if (p.M <= 1) return launch_fused_rows<KIND, 1, QF>(p, qa, stream);
  if (p.M <= 2) return launch_fused_rows<KIND, 2, QF>(p, qa, stream);
  if (p.M <= 4) return launch_fused_rows<KIND, 4, QF>(p, qa, stream);
  static_assert(kFusedRows == 4, "fused row buckets");
  return hipErrorInvalidValue;
}

template <int KIND>
hipError_t launch_fused_flags(const GemmArgs& p, const QuantArgs& qa, int flags, bool decode,
                              hipStream_t stream) {
  if (decode) {
    switch (flags & (kQuantSiluMul | kQuantUe8m0)) {
      case 0: return launch_decode_fused_kind<KIND, 0>(p, qa, stream);
      case kQuantSiluMul: return launch_decode_fused_kind<KIND, kQuantSiluMul>(p, qa, stream);
      case kQuantUe8m0: return launch_decode_fused_kind<KIND, kQuantUe8m0>(p, qa, stream);
      default: return launch_decode_fused_kind<KIND, kQuantSiluMul | kQuantUe8m0>(p, qa, stream);
    }
  }
  switch (flags & (kQuantSiluMul | kQuantUe8m0)) {
    case 0: return launch_fused_kind<KIND, 0>(p, qa, stream);
    case kQuantSiluMul: return launch_fused_kind<KIND, kQuantSiluMul>(p, qa, stream);
    case kQuantUe8m0: return launch_fused_kind<KIND, kQuantUe8m0>(p, qa, stream);
    default: return launch_fused_kind<KIND, kQuantSiluMul | kQuantUe8m0>(p, qa, stream);
  }
}
}  // namespace

// The fused form fits its registers (FR ceil(K / 4096) <= 8) and its LDS:
// with more workgroups than compute units it must leave room for two per
// compute unit (80 KB with two slots per wave; measured: blockwise 7168^2 at
// M = 4 with one workgroup per compute unit ran 29 us, the two launches 17).
bool decode_fused_launchable(const GemmArgs& p, bool silu) {
  const int64_t fr = decode_fused_rows(p.M);
  const size_t budget = (p.N + 15) / 16 <= 256 ? 163840 : 81920;
  return p.M >= 1 && p.M <= kFusedRows && p.K % 128 == 0 && fr * ((p.K + 4095) / 4096) <= kDecFusedUnits &&
         (uint64_t)(p.N - 1) * (uint64_t)p.ldb + (uint64_t)p.K <= 0xFFFFFFFFull &&
         decode_fused_fixed_bytes(p.K, kBlockwise, fr, silu) + 2 * kDecWaves * 2048 <= budget;
}

hipError_t launch_linear_fused(int kind, const GemmArgs& p, const QuantArgs& qa, int flags, bool decode,
                               hipStream_t stream) {
  if (decode && !decode_fused_launchable(p, (flags & kQuantSiluMul) != 0)) return hipErrorInvalidValue;
  return kind == kChannelwise ? launch_fused_flags<kChannelwise>(p, qa, flags, decode, stream)
                              : launch_fused_flags<kBlockwise>(p, qa, flags, decode, stream);
}

namespace {
// UE8M0 blockwise on the block-scaled MFMA: the tiles where that measured
// faster than promoting each 128-deep block in fp32 on the same inputs (HBM-
// resident weights): 256x128 panel 1.16-1.20x (4096x4096 M = 2048,
// 7168x7168 M = 1024), 128x64 8-wave panel 1.11x (3072x4096 M = 512), 16x16
// 256x256 tile 1.13x. The 128x128 8-wave panel measured 0.94-1.04x and the
// other tiles were not measured: they keep the fp32 promotion, which is
// exact for power-of-two scales. Shapes and ring depths as in launch_kind's
// panel cases; panel-eligible arguments only.
bool e8_tile(int variant) { return variant == 15 || variant == 22 || variant == 25; }

hipError_t launch_e8(int variant, const GemmArgs& p, hipStream_t stream) {
  switch (variant) {
    case 15: return launch_panel<256, 128, 4, 2, kBlockwiseE8, 5>(p, stream);
    case 22: return launch_panel<128, 64, 4, 2, kBlockwiseE8, 5>(p, stream);
    case 25: return launch_pingpong<kBlockwiseE8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// Static split-K scratch (see static_scratch in kernels.h). In host code the
// array's name stands for a host-side shadow, not a device address: only the
// address hipGetSymbolAddress returns for the current device is passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the arrival counters must start at zero (each call leaves them so)
    constexpr int64_t words = (int64_t)(kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(words / 256)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool grouped_launchable(int variant, const GemmArgs& p) {
  return variant >= 15 && variant <= 25 && p.split_k == 1 && panel_eligible<kBlockwise>(p);
}

hipError_t launch_gemm(int kind, int variant, const GemmArgs& p, hipStream_t stream) {
  // grouped calls may reach only the panel tiles (the kernels that read masked_m)
  if (p.masked_m && (kind == kChannelwise || !grouped_launchable(variant, p))) return hipErrorInvalidValue;
  if (kind == kBlockwiseE8) {
    // the block-scaled MFMA serves the tiles of e8_tile; every other tile
    // (and arguments the panel tiles cannot take) promotes in fp32, which is
    // exact for power-of-two scales
    if (e8_tile(variant) && panel_eligible<kBlockwise>(p)) return launch_e8(variant, p, stream);
    return launch_kind<kBlockwise>(variant, p, stream);
  }
  return kind == kChannelwise ? launch_kind<kChannelwise>(variant, p, stream)
                              : launch_kind<kBlockwise>(variant, p, stream);
}

}  // namespace fp8w8a8
