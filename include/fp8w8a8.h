/*
 * fp8w8a8.h -- C ABI of the MI355X (gfx950) FP8 W8A8 quantized-linear library.
 *
 * The library implements the FP8 W8A8 linear hot path described by three
 * prhub.com.cn digests of sglang pull requests:
 *   [PR34331] "Tune FP8 GEMM Triton tiles on L40S and enable them by default"
 *             -- channelwise scaled GEMM and its per-(N, K, device) tile table
 *             with nearest-M lookup, null entries and a kill switch.
 *   [PR31340] "Fix FP8 Triton dtype selection on A100"
 *             -- the FP8 format is torch's float8_e4m3fn (OCP E4M3).
 *   [PR27896] "Remove the per-call padding overhead of the FP8 blockwise GEMM"
 *             -- row-padded per-token-group quantization with column-major
 *             scales feeding a blockwise (1x128 activation, 128x128 weight)
 *             scaled GEMM.
 *
 * Conventions for every function below
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates device memory and never frees caller memory.
 *   - bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *   - FP8 values are raw OCP E4M3 codes (uint8_t): sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits; no infinities; 0x7F/0xFF are NaN; max 448.
 *   - Matrices are row-major with an explicit leading dimension (elements).
 *     Base pointers and leading dimensions must keep every row 16-byte aligned.
 *   - Every compute call is asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns a status code; it never throws or aborts.
 *     Argument validation happens on the host before anything is launched.
 *   - M == 0 is a successful no-op.
 *
 * Status codes: FP8_OK (0); FP8_ERR_INVALID (-1) bad argument (null pointer,
 * negative size, misalignment, K not a multiple of the group size, leading
 * dimension too small); FP8_ERR_UNSUPPORTED (-2) a valid request this build
 * has no kernel for (group size outside {16,32,64,128}, blockwise N or K not a
 * multiple of 128, block size other than 128x128); FP8_ERR_WORKSPACE (-3)
 * workspace too small; FP8_ERR_HIP (-4) a HIP runtime error. fp8_last_error()
 * returns a message for the last failure on the calling thread.
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP8_OK = 0,
  FP8_ERR_INVALID = -1,
  FP8_ERR_UNSUPPORTED = -2,
  FP8_ERR_WORKSPACE = -3,
  FP8_ERR_HIP = -4,
};

/* FP8_KIND_BLOCKWISE_UE8M0: blockwise with power-of-two scales (see
 * fp8_scaled_mm_blockwise_ue8m0); it shares the blockwise tiles and tables. */
enum { FP8_KIND_CHANNELWISE = 0, FP8_KIND_BLOCKWISE = 1, FP8_KIND_BLOCKWISE_UE8M0 = 2 };

/* Kernel variants a tile config can name. */
enum {
  FP8_VARIANT_DEFAULT = -1, /* let the library choose */
  FP8_VARIANT_SKINNY = 0,      /* M <= 32 rows: weight streamed once, K split over waves */
  FP8_VARIANT_T64x64 = 1,      /* 64x64 block tile, 512-deep K stages, 4 waves */
  FP8_VARIANT_T128x128 = 2,    /* 128x128 block tile, 4 waves */
  FP8_VARIANT_T256x128 = 3,    /* 256x128 block tile, 4 waves */
  FP8_VARIANT_T256x256 = 4,    /* 256x256 block tile, 4 waves */
  FP8_VARIANT_T256x256W8 = 5,  /* 256x256 block tile, 8 waves */
  FP8_VARIANT_T256x128W8 = 6,  /* 256x128 block tile, 8 waves */
  FP8_VARIANT_T128x128W8 = 7,  /* 128x128 block tile, 8 waves */
  FP8_VARIANT_T128x64K256 = 8, /* 128x64 block tile, 256-deep K stages, 4 waves */
  FP8_VARIANT_T64x128K256 = 9, /* 64x128 block tile, 256-deep K stages, 4 waves */
  FP8_VARIANT_T128x128K256 = 10, /* 128x128 block tile, 256-deep K stages, 4 waves */
  /* deep pipeline: 4 LDS stages of 64-deep K filled by LDS-DMA loads; used for
     channelwise GEMMs with K % 64 == 0, other requests run the register-staged
     kernel of the same tile shape */
  FP8_VARIANT_T256x256DMA = 11, /* 256x256 block tile, 8 waves */
  FP8_VARIANT_T256x128DMA = 12, /* 256x128 block tile, 8 waves */
  FP8_VARIANT_T128x128DMA = 13, /* 128x128 block tile, 4 waves */
  /* LDS-DMA ring of 128-byte-deep panels (whole cache-line row pieces), five
   * 32 KB slots: channelwise only, K % 128 == 0; other requests run the
   * register-staged 256x256 8-wave kernel. */
  FP8_VARIANT_T256x256PANEL = 14, /* 256x256 block tile, 8 waves */
  /* The same ring with a 256x128 tile, both kinds (blockwise: K-block scales
   * staged with the B panels); other requests run the register-staged
   * 256x128 8-wave kernel. */
  FP8_VARIANT_T256x128PANEL = 15, /* 256x128 block tile, 8 waves */
  /* Smaller panel-ring tiles (4 waves; five-slot rings of 40-85 KB, so
   * several workgroups share a compute unit); fallbacks as above, same tile
   * shape. */
  FP8_VARIANT_T128x128PANEL = 16, /* 128x128 block tile, 4 waves */
  FP8_VARIANT_T128x64PANEL = 17,  /* 128x64 block tile, 4 waves */
  FP8_VARIANT_T64x64PANEL = 18,   /* 64x64 block tile, 4 waves */
  /* The same with deeper rings (9 and 7 slots): more weight bytes in flight
   * per workgroup, fewer workgroups per compute unit; faster at small M. */
  FP8_VARIANT_T64x64DEEP = 19,    /* 64x64 block tile, 4 waves */
  FP8_VARIANT_T128x64DEEP = 20,   /* 128x64 block tile, 4 waves */
  /* 8-wave forms of the small panel tiles (two waves per SIMD) */
  FP8_VARIANT_T128x128PANEL8 = 21, /* 128x128 block tile, 8 waves */
  FP8_VARIANT_T128x64PANEL8 = 22,  /* 128x64 block tile, 8 waves */
  /* Narrow deep-ring tiles for small M (more workgroups for the same bytes
   * per compute unit); fallbacks: register-staged tiles of the same shape. */
  FP8_VARIANT_T32x32DEEP = 23,     /* 32x32 block tile, 1 wave, 9-slot ring */
  FP8_VARIANT_T64x32DEEP = 24,     /* 64x32 block tile, 2 waves, 7-slot ring */
  FP8_VARIANT_T256x256BW16 = 25,   /* blockwise 256x256, 8 waves, 16x16x128 MFMAs, 4-slot ring */
  /* M <= 16, K % 128 == 0: the weight stream of the skinny variant (same K
   * order and sums, so the same bits) with 1 KB row segments copied by
   * LDS-DMA into a ring of 2-8 slots; split_k 1. Requests past its 32-bit
   * DMA offsets run the skinny kernel. */
  FP8_VARIANT_DECODE = 26,         /* 16 output columns per workgroup, 8 waves */
  FP8_VARIANT_COUNT = 27,
};

/* One tile configuration of the scaled GEMM. The PR34331 digest ("Key source
 * excerpts") keys a tile by block sizes M/N/K plus launch parameters; here
 * `variant` names a compiled gfx950 kernel (its block sizes are fixed and are
 * reported in bm/bn/bk/waves) and `split_k` divides the K loop over that many
 * workgroups whose fp32 partial sums are reduced inside the same launch. */
typedef struct fp8_tile_config {
  int32_t variant;
  int32_t bm, bn, bk; /* block tile (filled in by the library) */
  int32_t split_k;    /* >= 1 */
  int32_t waves;      /* waves per workgroup (filled in by the library) */
} fp8_tile_config;

/* ------------------------------------------------------------------------ */
/* Quantization                                                              */
/* ------------------------------------------------------------------------ */

/* Rows of the row-padded buffers: ceil(M / row_alignment) * row_alignment.
 * [PR27896, "Key source excerpts": the row-padded quant aligns the row count
 * up to row_alignment, 4 by default.] Returns -1 if M < 0 or row_alignment < 1. */
int64_t fp8_padded_rows(int64_t M, int32_t row_alignment);

/* Dynamic per-token FP8 quantization (one scale per row).
 * For each row m < M:  s[m] = fp32(max(max_k |x[m,k]|, eps) / 448),
 *                      q[m,k] = E4M3_RNE(clamp(fp32(x[m,k] / s[m]), -448, 448)).
 * This is the activation quantization that feeds the channelwise GEMM of
 * [PR34331, "Key source excerpts", apply_fp8_linear], where the quantized
 * input and its per-token scale arrive already made; it is the per-token-group
 * quantization below with one group spanning the row.
 *   x      bf16 [M][ldx], ldx >= K         (input, read only)
 *   q      E4M3 [M][ldq], ldq >= K         (output codes)
 *   scale  fp32 [M]                         (output scales)
 *   eps    clamp of the row absmax (1e-10 in the pages' quantizer)
 * K must be a positive multiple of 16. */
int fp8_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* scale, float eps,
                        hipStream_t stream);

/* Dynamic per-token-group FP8 quantization into row-padded buffers.
 * [PR27896, "Implementation" step 1 and "Key source excerpts",
 * the row-padded per-token-group quant function; "Risks and impact" for the
 * untouched tail rows.] For each row m < M and group g < K/G:
 *   s = fp32(max(max_{k in g} |x[m,k]|, eps) / 448),  scale[g*M_pad + m] = s,
 *   q[m,k] = E4M3_RNE(clamp(fp32(x[m,k] / s), -448, 448))  for k in group g,
 * with M_pad = fp8_padded_rows(M, row_alignment). The scales are therefore
 * column-major: logically (M_pad, K/G) with unit stride along rows.
 * Rows M..M_pad-1 of q and of every scale column are NOT written.
 *   x            bf16 [M][ldx], ldx >= K
 *   group_size   G in {16, 32, 64, 128}  (others: FP8_ERR_UNSUPPORTED)
 *   row_alignment >= 1 (the pages use 4)
 *   q            E4M3 [M_pad][ldq], ldq >= K (only rows < M written)
 *   scale        fp32 [K/G][M_pad]
 * K must be a positive multiple of G. */
int fp8_quant_per_token_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              int32_t group_size, int32_t row_alignment,
                              uint8_t* q, int64_t ldq, float* scale, float eps,
                              hipStream_t stream);

/* Flags of the _ex quantizers. [PR27896, "Key source excerpts": the row-padded
 * quant function's kernel call passes scale_ue8m0 and fuse_silu_and_mul flags
 * (both off there); the digest shows no body for either. The readings below
 * are this library's.]
 *   FP8_QUANT_FUSE_SILU_MUL  x rows hold 2K values [gate | up]; the row that is
 *     quantized is y[k] = bf16_RNE(silu(x[m,k]) * x[m,K+k]), silu(g) = g/(1+e^-g),
 *     correctly rounded to bf16 (the value a separate SiLU-and-mul writing bf16
 *     would pass on), so codes and scales equal those of the unfused pair.
 *   FP8_QUANT_SCALE_UE8M0    every scale s is rounded up to a power of two
 *     (the smallest 2^e >= s) before the codes are formed; the scale buffer
 *     still holds fp32 values (exact powers of two). */
enum { FP8_QUANT_FUSE_SILU_MUL = 1, FP8_QUANT_SCALE_UE8M0 = 2 };

/* fp8_quant_per_token with flags (FP8_QUANT_*; unknown bits: FP8_ERR_INVALID).
 * With FP8_QUANT_FUSE_SILU_MUL, x is bf16 [M][ldx] with ldx >= 2K; q, scale and
 * K describe the quantized K-wide rows as before. */
int fp8_quant_per_token_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                           uint8_t* q, int64_t ldq, float* scale, float eps,
                           int32_t flags, hipStream_t stream);

/* fp8_quant_per_token_group with flags, as fp8_quant_per_token_ex. The SiLU-
 * and-mul form is the step between the gate/up projection (N = 2K) and the
 * down projection (K). */
int fp8_quant_per_token_group_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                 int32_t group_size, int32_t row_alignment,
                                 uint8_t* q, int64_t ldq, float* scale, float eps,
                                 int32_t flags, hipStream_t stream);

/* Masked per-expert group quantization (MoE experts).
 * [PR27896, "Key source excerpts": the group quantizer's kernel call takes a
 * masked_m argument (None there; no body shown). Reading: an [E, M_max, K]
 * batch of expert slabs whose first masked_m[e] rows are valid.] For every
 * expert e and row m < masked_m[e], exactly fp8_quant_per_token_group_ex on
 * that row (flags as there); all other rows of q and scale are NOT written.
 *   x         bf16 [E][M_max][ldx] (ldx >= K, or >= 2K with SiLU-and-mul)
 *   masked_m  int32 [E], DEVICE memory, read by the kernel; each value is
 *             clamped to [0, M_max] (so a bad count cannot write out of bounds)
 *   q         E4M3 [E][M_pad][ldq], M_pad = fp8_padded_rows(M_max, row_alignment)
 *   scale     fp32 [E][K/G][M_pad]  (column-major per expert)
 * E <= 65535; other arguments and errors as fp8_quant_per_token_group_ex. */
int fp8_quant_per_token_group_masked(const uint16_t* x, int64_t E, int64_t M_max, int64_t K,
                                     int64_t ldx, const int32_t* masked_m, int32_t group_size,
                                     int32_t row_alignment, uint8_t* q, int64_t ldq, float* scale,
                                     float eps, int32_t flags, hipStream_t stream);

/* Grouped blockwise FP8 GEMM over E experts with per-expert valid rows.
 * [PR27896: the masked_m argument above; each expert is the blockwise GEMM
 * of that digest on its own weight.] For every expert e and row m <
 * masked_m[e] (clamped to [0, M_max]):
 *   out[e][m][n] = bf16_RNE(sum_kb a_scale[e][kb][m] b_scale[e][n/128][kb]
 *                          sum_{k in kb} dec(a[e][m][k]) dec(b[e][n][k])),
 * no bias; other rows of out are NOT written.
 *   a         E4M3 [E][a_scale_ld][lda] (the masked quantizer's q, M_pad rows)
 *   a_scale   fp32 [E][K/128][a_scale_ld], a_scale_ld >= M_max, a multiple of 4
 *   b         E4M3 [E][N][ldb];  b_scale fp32 [E][N/128][K/128]
 *   out       bf16 [E][M_max][ldc]
 *   masked_m  int32 [E], device memory
 *   scale_ue8m0  non-zero: every scale is a power of two (as
 *             fp8_scaled_mm_blockwise_ue8m0)
 *   cfg       NULL or FP8_VARIANT_DEFAULT: a tile chosen by rows per expert
 *             (64x64 panel up to M_max 64, 128x128 8-wave panel up to 128,
 *             256x128 panel up to 256, the 16x16 256x256 tile above), unsplit;
 *             else one of the blockwise panel tiles
 *             (FP8_VARIANT_T256x128PANEL .. FP8_VARIANT_T256x256BW16), split_k 1.
 * Errors as fp8_scaled_mm_blockwise; FP8_ERR_UNSUPPORTED for a tile without
 * the grouped path. E <= 65535. */
int fp8_scaled_mm_blockwise_masked(const uint8_t* a, const uint8_t* b, const float* a_scale,
                                   int64_t a_scale_ld, const float* b_scale, uint16_t* out,
                                   const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N,
                                   int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                   int32_t scale_ue8m0, const fp8_tile_config* cfg,
                                   hipStream_t stream);

/* Static per-tensor FP8 quantization with a given scale.
 * [PR31340, "Implementation" step 2 and "Key files": a static FP8
 * quantization kernel; the ModelOpt FP8 linear carries a precomputed
 * input_scale. The digest shows no body; reading: the dynamic quantizer's
 * element step with the scale supplied.]
 *   q[m,k] = E4M3_RNE(clamp(fp32(x[m,k] / s), -448, 448)),  s = scale[0],
 * IEEE fp32 division; no scale is written.
 *   x      bf16 [M][ldx], ldx >= K
 *   scale  fp32 [1], device memory, read by the kernel: a positive finite
 *          value (others give unspecified codes; it cannot be checked on
 *          the host without a device read)
 *   q      E4M3 [M][ldq], ldq >= K
 * K must be a positive multiple of 16. */
int fp8_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     const float* scale, uint8_t* q, int64_t ldq, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Scaled GEMMs                                                              */
/* ------------------------------------------------------------------------ */

/* Channelwise FP8 scaled GEMM with fused epilogue.
 * [PR34331, "Key source excerpts", apply_fp8_linear: the scaled matmul takes
 * the quantized input, the FP8 weight, the per-token input scale, the
 * per-channel weight scale, the output dtype and a fused bias.]
 *   out[m,n] = bf16_RNE( a_scale[m] * b_scale[n] * sum_k dec(a[m,k]) dec(b[n,k])
 *                        + bias[n] ),   m < M, n < N,
 * accumulated in fp32 on the FP8 matrix cores.
 *   a        E4M3 [M][lda], lda >= K            (activations)
 *   b        E4M3 [N][ldb], ldb >= K            (weight, K-contiguous; the
 *            pages view it as [K, N]: N = its second dim, K its first)
 *   a_scale  fp32 [M];  b_scale fp32 [N]
 *   bias     bf16 [N] or NULL
 *   out      bf16 [M][ldc], ldc >= N            (only rows < M written)
 *   ws, ws_bytes  split-K workspace (see fp8_scaled_mm_workspace_size), 256-byte
 *            aligned; may be NULL/0 when the chosen config needs none. Its
 *            first 256 KiB hold per-tile arrival counters and must be
 *            zero-filled before the first use; every call leaves them zero
 *            again, so one workspace serves calls of any shape. The rest holds
 *            fp32 partial tiles and needs no initialisation. Calls that run
 *            concurrently must not share one workspace.
 * K must be a positive multiple of 16. */
int fp8_scaled_mm_channelwise(const uint8_t* a, const uint8_t* b,
                              const float* a_scale, const float* b_scale,
                              const uint16_t* bias, uint16_t* out,
                              int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* As fp8_scaled_mm_channelwise with an explicit tile config (NULL or variant
 * FP8_VARIANT_DEFAULT = table lookup / default heuristic). Used by the sweep. */
int fp8_scaled_mm_channelwise_ex(const uint8_t* a, const uint8_t* b,
                                 const float* a_scale, const float* b_scale,
                                 const uint16_t* bias, uint16_t* out,
                                 int64_t M, int64_t N, int64_t K,
                                 int64_t lda, int64_t ldb, int64_t ldc,
                                 void* ws, size_t ws_bytes,
                                 const fp8_tile_config* cfg, hipStream_t stream);

/* Blockwise FP8 scaled GEMM (1x128 activation groups, 128x128 weight blocks).
 * [PR27896, "Key source excerpts", the blockwise linear: group-128
 * activation quant into row-padded buffers, a blockwise scaled matmul of the
 * [N, K] weight with block_size [128, 128], rows beyond M dropped, bias added.]
 *   out[m,n] = bf16_RNE( sum_kb a_scale[kb*a_scale_ld + m] * b_scale[(n/128)*KB + kb]
 *                        * sum_{k in block kb} dec(a[m,k]) dec(b[n,k]) + bias[n] ),
 *   KB = K/128, m < M, n < N. The per-block partial sum is promoted to fp32
 *   and scaled before it joins the accumulator.
 *   a            E4M3 [>=M][lda]   (rows >= M are never read)
 *   a_scale      fp32 column-major, (m, kb) at kb*a_scale_ld + m;
 *                a_scale_ld >= M (the row-padded M_pad of the quantizer)
 *   b            E4M3 [N][ldb];  b_scale fp32 [N/128][K/128] row-major
 *   bias, out, ws as for the channelwise GEMM.
 * N and K must be multiples of 128 (else FP8_ERR_UNSUPPORTED). */
int fp8_scaled_mm_blockwise(const uint8_t* a, const uint8_t* b,
                            const float* a_scale, int64_t a_scale_ld,
                            const float* b_scale,
                            const uint16_t* bias, uint16_t* out,
                            int64_t M, int64_t N, int64_t K,
                            int64_t lda, int64_t ldb, int64_t ldc,
                            void* ws, size_t ws_bytes, hipStream_t stream);

int fp8_scaled_mm_blockwise_ex(const uint8_t* a, const uint8_t* b,
                               const float* a_scale, int64_t a_scale_ld,
                               const float* b_scale,
                               const uint16_t* bias, uint16_t* out,
                               int64_t M, int64_t N, int64_t K,
                               int64_t lda, int64_t ldb, int64_t ldc,
                               void* ws, size_t ws_bytes,
                               const fp8_tile_config* cfg, hipStream_t stream);

/* Blockwise FP8 scaled GEMM with UE8M0 (power-of-two) scales.
 * [PR27896, "Key source excerpts": the group quantizer's scale_ue8m0 flag;
 * the scales it makes (FP8_QUANT_SCALE_UE8M0) and 128x128 weight block scales
 * rounded up the same way feed this GEMM.] Same operation, arguments, layouts
 * and errors as fp8_scaled_mm_blockwise, and the same tile configs; every
 * a_scale and b_scale value must be a positive power of two held as fp32
 * (only its exponent field is used: other values give wrong results). On
 * gfx950 the large-M tile (FP8_VARIANT_T256x256BW16) hands the exponents to
 * the block-scaled MFMA, which applies them to the products itself instead of
 * promoting every 128-deep block's partial sum in fp32; other tiles run the
 * blockwise kernels, exact for powers of two. fp8_scaled_mm_workspace_size
 * takes FP8_KIND_BLOCKWISE_UE8M0 or FP8_KIND_BLOCKWISE alike. */
int fp8_scaled_mm_blockwise_ue8m0(const uint8_t* a, const uint8_t* b,
                                  const float* a_scale, int64_t a_scale_ld,
                                  const float* b_scale, const uint16_t* bias, uint16_t* out,
                                  int64_t M, int64_t N, int64_t K,
                                  int64_t lda, int64_t ldb, int64_t ldc,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

int fp8_scaled_mm_blockwise_ue8m0_ex(const uint8_t* a, const uint8_t* b,
                                     const float* a_scale, int64_t a_scale_ld,
                                     const float* b_scale, const uint16_t* bias, uint16_t* out,
                                     int64_t M, int64_t N, int64_t K,
                                     int64_t lda, int64_t ldb, int64_t ldc,
                                     void* ws, size_t ws_bytes, const fp8_tile_config* cfg,
                                     hipStream_t stream);

/* The scaled GEMMs without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same operation, arguments, layouts, tile
 * configs and errors as fp8_scaled_mm_channelwise_ex (kind
 * FP8_KIND_CHANNELWISE; a_scale_ld is ignored), fp8_scaled_mm_blockwise_ex
 * (FP8_KIND_BLOCKWISE) and fp8_scaled_mm_blockwise_ue8m0_ex
 * (FP8_KIND_BLOCKWISE_UE8M0), and bit-identical outputs, but the split-K
 * partial tiles and arrival counters live in a library-owned static device
 * array of FP8_NOALLOC_SCRATCH_BYTES per device (held until the process
 * ends). No device memory is allocated. A call whose split-K plan needs more
 * than that returns FP8_ERR_WORKSPACE (checked on the host before any device
 * work); plans without split-K need none. The first call on a device looks up
 * that device's copy and clears its counters with a small kernel on `stream`.
 * Every call on one device shares the array and leaves the counters at zero;
 * calls that overlap in time on one device (different streams) race and give
 * undefined results. */
#define FP8_NOALLOC_SCRATCH_BYTES ((size_t)(256u << 10) + ((size_t)64 << 20))
int fp8_scaled_mm_noalloc(int32_t kind, const uint8_t* a, const uint8_t* b,
                          const float* a_scale, int64_t a_scale_ld,
                          const float* b_scale, const uint16_t* bias, uint16_t* out,
                          int64_t M, int64_t N, int64_t K,
                          int64_t lda, int64_t ldb, int64_t ldc,
                          const fp8_tile_config* cfg, hipStream_t stream);

/* Workspace bytes the GEMM of `kind` needs for (M, N, K) with `cfg` (NULL =
 * the config the library would pick). 0 when no workspace is needed.
 * Returns (size_t)-1 on invalid arguments. */
size_t fp8_scaled_mm_workspace_size(int32_t kind, int64_t M, int64_t N, int64_t K,
                                    const fp8_tile_config* cfg);

/* ------------------------------------------------------------------------ */
/* Linears: activation quantization and scaled GEMM in one call              */
/* ------------------------------------------------------------------------ */

/* Channelwise FP8 linear. [PR34331, "Key source excerpts", apply_fp8_linear:
 * the input is quantized per token with a dynamic scale, and the codes and
 * that scale go to the scaled matmul with the per-channel weight scale and
 * the bias.] On success q rows < M and a_scale[0..M) hold exactly what
 * fp8_quant_per_token writes for x, and out exactly what
 * fp8_scaled_mm_channelwise computes from them (the same bits).
 * For M <= 4 with the skinny or the decode variant selected (the defaults
 * at small M) both happen in ONE launch: every workgroup quantizes the
 * activation rows it multiplies (x is read from cache by each of them) and
 * workgroup 0 also stores q and a_scale (the decode variant: while
 * 4 ceil(K / 4096) <= 8 at M = 3..4, 2 ceil(K / 4096) <= 8 at M = 2,
 * ceil(K / 4096) <= 8 at M = 1, K % 128 == 0). Otherwise the quantizer and
 * the GEMM run as two launches on `stream`. FP8W8A8_FUSED_LINEAR=0 in the
 * environment turns the single launch off; =all also takes it on the skinny
 * kernel with SiLU-and-mul at every M <= 4 (see the _ex forms; for
 * measurement).
 *   x        bf16 [M][ldx], ldx >= K (input)
 *   q        E4M3 [M][ldq], ldq >= K (output codes; the GEMM's input)
 *   a_scale  fp32 [M] (output per-token scales)
 *   b, b_scale, bias, out, ws, ws_bytes  as for fp8_scaled_mm_channelwise
 *   cfg      tile config or NULL (table lookup / default heuristic)
 * Errors as for the quantizer and the GEMM; nothing is launched on error. */
int fp8_linear_channelwise(const uint16_t* x, const uint8_t* b, const float* b_scale,
                           const uint16_t* bias, uint16_t* out,
                           int64_t M, int64_t N, int64_t K,
                           int64_t ldx, int64_t ldb, int64_t ldc, float eps,
                           uint8_t* q, int64_t ldq, float* a_scale,
                           void* ws, size_t ws_bytes,
                           const fp8_tile_config* cfg, hipStream_t stream);

/* Blockwise FP8 linear. [PR27896, "Key source excerpts", the blockwise
 * linear: group-128 activation quant into row-padded buffers, then the
 * blockwise scaled matmul with 128x128 weight blocks over the first M rows,
 * bias added.] On success q rows < M and the scale entries of rows < M hold
 * exactly what fp8_quant_per_token_group(x, group 128, row_alignment) writes,
 * and out exactly what fp8_scaled_mm_blockwise computes from them; pad rows
 * M..M_pad-1 are not written. One launch for M <= 4 with the skinny or the
 * decode variant selected, as above; two otherwise.
 *   x        bf16 [M][ldx], ldx >= K
 *   q        E4M3 [M_pad][ldq], M_pad = fp8_padded_rows(M, row_alignment)
 *   a_scale  fp32 [K/128][M_pad] (column-major scales, (m, kb) at kb*M_pad + m)
 *   b, b_scale, bias, out, ws, ws_bytes  as for fp8_scaled_mm_blockwise
 * N and K must be multiples of 128 (else FP8_ERR_UNSUPPORTED). */
int fp8_linear_blockwise(const uint16_t* x, const uint8_t* b, const float* b_scale,
                         const uint16_t* bias, uint16_t* out,
                         int64_t M, int64_t N, int64_t K,
                         int64_t ldx, int64_t ldb, int64_t ldc,
                         int32_t row_alignment, float eps,
                         uint8_t* q, int64_t ldq, float* a_scale,
                         void* ws, size_t ws_bytes,
                         const fp8_tile_config* cfg, hipStream_t stream);

/* The linears with quantizer flags (FP8_QUANT_*, as for fp8_quant_per_token_ex;
 * unknown bits: FP8_ERR_INVALID). With FP8_QUANT_FUSE_SILU_MUL, x is bf16
 * [M][ldx] with ldx >= 2K holding [gate | up] rows, so the down projection
 * runs straight from the gate/up projection's output; K is the width of the
 * quantized rows (the GEMM's depth) as before. With FP8_QUANT_SCALE_UE8M0 the
 * activation scales are powers of two, and the blockwise linear then runs the
 * GEMM as fp8_scaled_mm_blockwise_ue8m0 (its weight block scales must be powers
 * of two as well). q, a_scale and out hold exactly what the flagged quantizer
 * and that GEMM write. With the skinny kernel selected the flags apply inside
 * the single fused launch (SiLU-and-mul evaluated there, correctly rounded as
 * in the quantizer) for M <= 4 with UE8M0 alone, and with SiLU-and-mul for
 * M = 1 channelwise and M <= 2 blockwise (every workgroup of that launch
 * evaluates SiLU over the whole input, which pays only for so few rows); with
 * the decode variant selected, for every flag at M <= 4 (it evaluates SiLU
 * once per value); the other calls run the flagged quantizer and the GEMM as
 * two launches.
 * fp8_linear_launches_ex tells which. flags == 0 is exactly
 * fp8_linear_channelwise / fp8_linear_blockwise. */
int fp8_linear_channelwise_ex(const uint16_t* x, const uint8_t* b, const float* b_scale,
                              const uint16_t* bias, uint16_t* out,
                              int64_t M, int64_t N, int64_t K,
                              int64_t ldx, int64_t ldb, int64_t ldc, float eps,
                              uint8_t* q, int64_t ldq, float* a_scale,
                              void* ws, size_t ws_bytes,
                              const fp8_tile_config* cfg, int32_t flags, hipStream_t stream);

int fp8_linear_blockwise_ex(const uint16_t* x, const uint8_t* b, const float* b_scale,
                            const uint16_t* bias, uint16_t* out,
                            int64_t M, int64_t N, int64_t K,
                            int64_t ldx, int64_t ldb, int64_t ldc,
                            int32_t row_alignment, float eps,
                            uint8_t* q, int64_t ldq, float* a_scale,
                            void* ws, size_t ws_bytes,
                            const fp8_tile_config* cfg, int32_t flags, hipStream_t stream);

/* Kernel launches an fp8_linear_* call of `kind` makes for (M, N, K, cfg):
 * 1 (fused), 2 (quantizer, then GEMM) or 0 (M == 0); FP8_ERR_INVALID on bad
 * arguments. Host only. */
int fp8_linear_launches(int32_t kind, int64_t M, int64_t N, int64_t K,
                        const fp8_tile_config* cfg);

/* The same for an fp8_linear_*_ex call with quantizer `flags` (unknown bits:
 * FP8_ERR_INVALID). Host only. */
int fp8_linear_launches_ex(int32_t kind, int64_t M, int64_t N, int64_t K,
                           const fp8_tile_config* cfg, int32_t flags);

/* ------------------------------------------------------------------------ */
/* Tile-config table                                                         */
/* ------------------------------------------------------------------------ */

/* Resolve the tile config for (kind, N, K, M). [PR34331, "Implementation"
 * steps 1 and 5 and "Key source excerpts": one JSON table per (N, K, device,
 * dtype), keys are M values, the entry whose key is nearest to M wins (ties:
 * the smaller key), a null entry or a missing table means "keep the default
 * path", and an environment kill switch disables the tables.]
 * Tables are read once per (kind, N, K) from the config directory, file name
 * "N={N},K={K},device_name=gfx950,dtype=fp8_w8a8_{channelwise|blockwise}.json".
 * The kill switch is FP8W8A8_TUNED_CONFIGS=0.
 * Fills *out with the config used (table hit or default heuristic) and returns
 * 1 for a table hit, 0 for the default, FP8_ERR_INVALID on bad arguments. */
int fp8_tile_config_lookup(int32_t kind, int64_t N, int64_t K, int64_t M,
                           fp8_tile_config* out);

/* The default heuristic alone (no table). Returns 0 or FP8_ERR_INVALID. */
int fp8_tile_config_default(int32_t kind, int64_t N, int64_t K, int64_t M,
                            fp8_tile_config* out);

/* Set the directory tables are read from (NULL: back to the default, which is
 * $FP8W8A8_CONFIG_DIR or the "configs" directory next to the library) and
 * drop every cached table. Returns FP8_OK. */
int fp8_tile_config_set_dir(const char* dir);

/* ------------------------------------------------------------------------ */
/* Measurement probes (not part of the linear): the ceilings the kernels      */
/* above are compared with. Each returns FP8_OK or an error code; `sink`      */
/* (device memory, workgroups * 256 words) only receives a value if a folded  */
/* checksum happens to equal an internal key, which keeps the compiler from   */
/* dropping the work; its contents are meaningless.                            */
/* ------------------------------------------------------------------------ */

/* Reads `bytes` of device memory once (16-byte non-temporal loads, eight per
 * lane in flight, `workgroups` workgroups of 256 threads striding over the
 * buffer): the HBM read ceiling for a weight stream of that size. src 16-byte
 * aligned, bytes a positive multiple of 16. */
int fp8_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                          hipStream_t stream);

/* Reads a [rows][row_bytes] matrix once, `piece` bytes of a row at a time:
 * workgroup w (of rows / rows_per_wg) owns rows_per_wg consecutive rows and
 * walks them along the row in steps of `piece` bytes, reading all its rows'
 * pieces each step (16-byte non-temporal loads; one 64-lane instruction covers
 * 1024 / piece rows). The HBM cost of the row-piece size a GEMM tile's weight
 * stream uses. piece a power of two in [16, 1024]; rows_per_wg * piece a
 * multiple of 1024; the grid is rows / rows_per_wg workgroups (<= 65535). */
int fp8_probe_strided_read(const void* src, int64_t rows, int64_t row_bytes, int32_t rows_per_wg,
                           int32_t piece, uint32_t* sink, hipStream_t stream);

/* Every workgroup reads the same `window_bytes` (a multiple of 1 KB; small
 * enough to stay in L2) `reps` times: with dma == 0 through 16-byte register
 * loads, with dma != 0 through LDS-DMA loads (global_load_lds_dwordx4) into a
 * ring in LDS. Bytes moved = workgroups * reps * window_bytes; divided by the
 * duration and the compute units it gives the L2-to-compute-unit feed rate. */
int fp8_probe_l2_feed(const void* src, size_t window_bytes, int32_t reps, int32_t dma, uint32_t* sink,
                      int32_t workgroups, hipStream_t stream);

/* The panel tiles' feed pattern without their arithmetic: each of
 * `workgroups` workgroups (four waves) streams the 64-row block
 * (workgroup % panels) of `src` ([panels * 64][row_bytes] bytes, L2-sized)
 * in 128-byte-per-row stages by LDS-DMA, six stages in flight per wave,
 * `stages` times. mode bit 0 adds LDS reads of landed stages (4 KB per wave
 * and stage), bit 1 a workgroup barrier per stage. Bytes moved =
 * workgroups * stages * 8192. Invalid arguments (row_bytes not a positive
 * multiple of 128, mode outside 0-3, the matrix past 4 GiB) return
 * FP8_ERR_INVALID without a launch. */
int fp8_probe_panel_feed(const void* src, int32_t row_bytes, int32_t panels, int32_t stages, int32_t mode,
                         uint32_t* sink, int32_t workgroups, hipStream_t stream);

/* Back-to-back independent V_MFMA_F32_32X32X64_F8F6F4 (four accumulators per
 * wave, four waves per workgroup): FLOPs = workgroups * 4 * iters * 4 * 131072.
 * The dense FP8 matrix rate; rate / (256 CUs * 8192 FLOP per clock per CU)
 * is the clock the matrix cores ran at. */
int fp8_probe_mfma(int32_t iters, float* sink, int32_t workgroups, hipStream_t stream);

/* Reads `bytes` (a multiple of 1 KB) once in 1 KB pieces, each wave of
 * `workgroups` workgroups of `threads` threads (256, 512 or 1024) keeping
 * `depth` pieces in flight (4, 8 or 16; 4 or 8 at 1024 threads): into
 * registers (dma == 0) or, by LDS-DMA, into a depth-slot LDS ring per wave
 * (dma != 0). How the HBM read rate scales with waves per compute unit and
 * copies in flight per wave. */
int fp8_probe_wave_read(const void* src, size_t bytes, int32_t threads, int32_t depth, int32_t dma,
                        uint32_t* sink, int32_t workgroups, hipStream_t stream);

/* LDS read rate: every lane of `workgroups` workgroups of `threads` (256 or
 * 512) threads reads 16 bytes per step (ds_read_b128, a wave reading one
 * contiguous 1 KB row: no bank conflicts), iters * 8 steps. Bytes read =
 * workgroups * threads * iters * 128. */
int fp8_probe_lds(int32_t iters, int32_t threads, uint32_t* sink, int32_t workgroups, hipStream_t stream);

/* `count` independent MFMAs, one wave each: for problem i, D_i = W_i X_i^T +
 * C_i. form 0: V_MFMA_F32_16X16X128_F8F6F4, W_i and X_i [16][128] E4M3 codes,
 * C_i and D_i [16][16] fp32; form 1: V_MFMA_F32_32X32X64_F8F6F4, W_i and X_i
 * [32][64], C_i and D_i [32][32]. All row-major and consecutive over i;
 * element [n][m] of C and D pairs row n of W with row m of X. The matrix
 * core's own rounding of an FP8 dot product and of its addition to the
 * accumulator, which sets the error model of every GEMM here. w and x 16-byte
 * aligned; 1 <= count <= 65535. */
int fp8_probe_mfma_dot(const void* w, const void* x, const float* c, float* d, int32_t count, int32_t form,
                       hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* fp8_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8W8A8_H */
