// Host-side launchers of the gfx950 kernels (arguments validated by the caller).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w8a8 {

// Quantizer flags (the values of FP8_QUANT_* in the C header). With
// kQuantSiluMul the input rows hold 2K values [gate | up] and K is the width
// of the quantized row.
enum QuantFlag { kQuantSiluMul = 1, kQuantUe8m0 = 2 };

// Masked per-expert quantization: expert e (grid y) has masked_m[e] valid
// rows (clamped to [0, M]) of an M-row slab; slabs are x_es, q_es and s_es
// elements apart. Null masked_m: one plain batch.
struct MaskArgs {
  const int* masked_m;
  int64_t x_es, q_es, s_es;
};

hipError_t launch_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* scale, float eps, int flags,
                                  hipStream_t stream);

hipError_t launch_quant_per_token_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                        int group_size, int64_t m_pad, uint8_t* q, int64_t ldq,
                                        float* scale, float eps, int flags, hipStream_t stream);

// The same over `experts` slabs with per-expert valid row counts (M = M_max).
hipError_t launch_quant_per_token_group_masked(const uint16_t* x, int64_t experts, int64_t M,
                                               int64_t K, int64_t ldx, int group_size,
                                               int64_t m_pad, uint8_t* q, int64_t ldq, float* scale,
                                               float eps, int flags, const MaskArgs& mask,
                                               hipStream_t stream);

hipError_t launch_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* scale, uint8_t* q, int64_t ldq, hipStream_t stream);

// kBlockwiseE8: blockwise with power-of-two (UE8M0) scales, held as fp32
// powers of two; the 16x16 256x256 tile hands their exponents to the
// block-scaled MFMA, every other tile runs the kBlockwise kernels (their fp32
// promotion is exact for powers of two).
enum GemmKind { kChannelwise = 0, kBlockwise = 1, kBlockwiseE8 = 2 };

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;     // channelwise: [M]; blockwise: column-major, (m, kb) at kb*sa_ld + m
  int64_t sa_ld;
  const float* sb;     // channelwise: [N]; blockwise: [N/128][K/128]
  const uint16_t* bias;  // [N] or null
  uint16_t* out;
  int64_t M, N, K, lda, ldb, ldc;
  float* ws_part;      // split-K partial tiles (null when split_k == 1)
  int* ws_count;       // split-K arrival counters, one per output tile
  int split_k;
  int k_tiles_per_split;  // 128-deep K steps handled by one split
  // Grouped (MoE experts, panel tiles only, split_k == 1): `experts` GEMMs,
  // expert e (blockIdx.z) on slabs offset by e times the strides below
  // (elements), with masked_m[e] valid rows of M (= M_max); null: one GEMM.
  const int* masked_m;
  int experts;
  int64_t a_es, sa_es, b_es, sb_es, out_es;
  // decode weight stream (M <= 16): LDS ring slots, set by its launcher
  int ring_slots;
};


// Activation quantization fused into the skinny GEMM (M <= kFusedRows): the
// kernel reads bf16 x instead of codes and scales, quantizes it as the
// quantization kernels do, and workgroup 0 also stores the codes (rows < M of
// q) and the scales (per token: scale[m]; per group of 128: scale[kb *
// scale_ld + m]). Every workgroup quantizes the whole activation, so the
// fused launch beats the two launches only while M is small: measured on the
// N = K = 4096 linear, ahead by 2-4.5 us at M <= 4, even at M = 8, behind at
// M = 16.
struct QuantArgs {
  const uint16_t* x;
  int64_t ldx;
  uint8_t* q;
  int64_t ldq;
  float* scale;
  int64_t scale_ld;
  float eps;
};
constexpr int64_t kFusedRows = 4;

// flags: the quantizer flags (kQuantSiluMul: x rows are [gate | up], 2K wide,
// and silu(gate) * up is quantized; kQuantUe8m0: power-of-two scales).
// decode: the decode weight stream with the quantization fused (when
// decode_fused_launchable), else the skinny kernel with it fused.
hipError_t launch_linear_fused(int kind, const GemmArgs& args, const QuantArgs& qa, int flags, bool decode,
                               hipStream_t stream);
bool decode_fused_launchable(const GemmArgs& args, bool silu);

// Geometry of a compiled kernel variant.
struct VariantInfo {
  int bm, bn, bk, waves;
  bool exists;
};
VariantInfo variant_info(int variant);

// Number of output tiles the variant launches for (M, N).
int64_t variant_tiles(int variant, int64_t M, int64_t N);

// Split-K workspace layout: a fixed region of arrival counters (one int per
// output tile, at most kMaxSplitTiles tiles) at the start, then the fp32
// partial tiles. The counter region sits at the same place for every shape,
// so the all-zero state each call leaves behind holds for the next call
// whatever its shape.
constexpr int64_t kMaxSplitTiles = 65536;
constexpr size_t kCounterBytes = (size_t)kMaxSplitTiles * sizeof(int);

// The decode stream's split plan: its splits cut every wave's block list
// into `per` blocks each; `splits` (<= split_k) of them.
void decode_split_plan(int64_t K, int split_k, int* splits, int* per);

// Bytes of split-K workspace for (variant, split_k, M, N); 0 when split_k == 1.
size_t variant_workspace_bytes(int variant, int split_k, int64_t M, int64_t N);

// The library's own split-K workspace, for callers that cannot allocate: a
// static device array of kStaticScratchBytes (arrival counters, then 64 MiB
// of partial tiles), one per device, held until the process ends. The first
// call on a device looks up that device's copy and clears its counters (a
// fill kernel on `stream`); *ptr receives the device address to pass to the
// kernels. Calls that overlap on one device share the array and race.
constexpr size_t kStaticScratchBytes = kCounterBytes + ((size_t)64 << 20);
hipError_t static_scratch(hipStream_t stream, void** ptr);

hipError_t launch_gemm(int kind, int variant, const GemmArgs& args, hipStream_t stream);

// Grouped blockwise GEMMs run only on the blockwise panel tiles (variants
// 15-25) with split_k == 1; true when `variant` and the arguments allow it.
bool grouped_launchable(int variant, const GemmArgs& args);

// Measurement probes (probes.hip): sink holds workgroups * 256 words.
hipError_t launch_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups,
                                    hipStream_t stream);
hipError_t launch_probe_strided_read(const void* src, int64_t rows, int64_t row_bytes, int rows_per_wg,
                                     int piece, uint32_t* sink, hipStream_t stream);
hipError_t launch_probe_l2_feed(const void* src, size_t window, int reps, int dma, uint32_t* sink,
                                int workgroups, hipStream_t stream);
hipError_t launch_probe_panel_feed(const void* src, uint32_t row_bytes, int panels, int stages, int mode,
                                   uint32_t* sink, int workgroups, hipStream_t stream);
hipError_t launch_probe_mfma(int iters, float* sink, int workgroups, hipStream_t stream);
hipError_t launch_probe_wave_read(const void* src, size_t bytes, int threads, int depth, int dma, uint32_t* sink,
                                  int workgroups, hipStream_t stream);
hipError_t launch_probe_mfma_dot(const void* w, const void* x, const float* c, float* d, int count, int form,
                                 hipStream_t stream);
hipError_t launch_probe_lds(int iters, int threads, uint32_t* sink, int workgroups, hipStream_t stream);

}  // namespace fp8w8a8
