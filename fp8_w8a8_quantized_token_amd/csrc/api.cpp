// C ABI of the FP8 W8A8 library: argument validation, config resolution and
// kernel dispatch. Validation runs entirely on the host before any HIP call,
// so every argument error is reported without touching the device.
#include <stdarg.h>

#include <cstdio>
#include <cstdlib>
#include <string>

#include "fp8w8a8.h"
#include "kernels.h"
#include "tile_table.h"

using namespace fp8w8a8;

static_assert(FP8_NOALLOC_SCRATCH_BYTES == kStaticScratchBytes, "the header states the static scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return FP8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Common checks of the quantizer arguments; every row of x holds xcols values
// (K, or 2K with SiLU-and-mul).
int check_quant(const char* fn, const uint16_t* x, int64_t M, int64_t K, int64_t xcols, int64_t ldx,
                const uint8_t* q, int64_t ldq, const float* scale, float eps) {
  if (M < 0 || K < 0) return fail(FP8_ERR_INVALID, "%s: negative size (M=%lld K=%lld)", fn, (long long)M, (long long)K);
  if (M == 0) return FP8_OK;
  if (!x || !q || !scale) return fail(FP8_ERR_INVALID, "%s: null pointer", fn);
  if (K == 0 || K % 16 != 0) return fail(FP8_ERR_INVALID, "%s: K=%lld must be a positive multiple of 16", fn, (long long)K);
  if (ldx < xcols || ldq < K) return fail(FP8_ERR_INVALID, "%s: leading dimension too small", fn);
  if (ldx % 8 != 0 || ldq % 16 != 0 || !aligned(x, 16) || !aligned(q, 16))
    return fail(FP8_ERR_INVALID, "%s: rows of x and q must be 16-byte aligned", fn);
  if (!aligned(scale, 4)) return fail(FP8_ERR_INVALID, "%s: scale must be 4-byte aligned", fn);
  if (!(eps >= 0.0f)) return fail(FP8_ERR_INVALID, "%s: eps must be >= 0", fn);
  return FP8_OK;
}

// Flag check of the quantizers: known bits only.
int check_quant_flags(const char* fn, int32_t flags) {
  if (flags & ~(FP8_QUANT_FUSE_SILU_MUL | FP8_QUANT_SCALE_UE8M0))
    return fail(FP8_ERR_INVALID, "%s: unknown flags 0x%x", fn, (unsigned)flags);
  return FP8_OK;
}

int check_gemm(const char* fn, const uint8_t* a, const uint8_t* b, const float* sa,
               const float* sb, const uint16_t* bias, const uint16_t* out, int64_t M, int64_t N,
               int64_t K, int64_t lda, int64_t ldb, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return fail(FP8_ERR_INVALID, "%s: negative size", fn);
  if (M == 0) return FP8_OK;
  if (!a || !b || !sa || !sb || !out) return fail(FP8_ERR_INVALID, "%s: null pointer", fn);
  if (N == 0 || K == 0 || K % 16 != 0)
    return fail(FP8_ERR_INVALID, "%s: N must be positive and K a positive multiple of 16 (N=%lld K=%lld)", fn,
                (long long)N, (long long)K);
  if (lda < K || ldb < K || ldc < N) return fail(FP8_ERR_INVALID, "%s: leading dimension too small", fn);
  if (lda % 16 || ldb % 16 || ldc % 8 || !aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16))
    return fail(FP8_ERR_INVALID, "%s: rows of a, b and out must be 16-byte aligned", fn);
  if (!aligned(sa, 4) || !aligned(sb, 16)) return fail(FP8_ERR_INVALID, "%s: misaligned scales", fn);
  if (bias && !aligned(bias, 8)) return fail(FP8_ERR_INVALID, "%s: bias must be 8-byte aligned", fn);
  return FP8_OK;
}

int resolve_config(int kind, int64_t M, int64_t N, int64_t K, const fp8_tile_config* cfg,
                   fp8_tile_config* out) {
  if (!cfg || cfg->variant == FP8_VARIANT_DEFAULT) {
    lookup_config(kind, N, K, M, out);
    // a table entry snapped from a nearby M may not fit this M
    if ((out->variant == FP8_VARIANT_SKINNY || out->variant == FP8_VARIANT_DECODE) &&
        (M > variant_info(out->variant).bm || (out->variant == FP8_VARIANT_DECODE && K % 128 != 0)))
      default_config(kind, N, K, M, out);
    return FP8_OK;
  }
  const VariantInfo vi = variant_info(cfg->variant);
  if (!vi.exists) return fail(FP8_ERR_INVALID, "unknown kernel variant %d", cfg->variant);
  if (cfg->split_k < 1) return fail(FP8_ERR_INVALID, "split_k must be >= 1");
  if (cfg->variant == FP8_VARIANT_SKINNY && (M > vi.bm || cfg->split_k != 1))
    return fail(FP8_ERR_INVALID, "the skinny variant takes M <= %d and split_k == 1", vi.bm);
  if (cfg->variant == FP8_VARIANT_DECODE && (M > vi.bm || K % 128 != 0))
    return fail(FP8_ERR_INVALID, "the decode variant takes M <= %d and K %% 128 == 0", vi.bm);
  *out = *cfg;
  out->bm = vi.bm; out->bn = vi.bn; out->bk = vi.bk; out->waves = vi.waves;
  return FP8_OK;
}

// Effective split count: never more splits than the variant's K stages;
// `per` counts stages of the variant's depth bk.
void split_plan(int64_t K, int bk, int split_k, int* splits, int* per) {
  const int64_t kt = (K + bk - 1) / bk;
  int64_t s = split_k < 1 ? 1 : split_k;
  if (s > kt) s = kt;
  const int64_t p = (kt + s - 1) / s;
  *per = (int)p;
  *splits = (int)((kt + p - 1) / p);
}

int run_gemm(const char* fn, int kind, const uint8_t* a, const uint8_t* b, const float* sa,
             int64_t sa_ld, const float* sb, const uint16_t* bias, uint16_t* out, int64_t M,
             int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, void* ws,
             size_t ws_bytes, const fp8_tile_config* cfg_in, hipStream_t stream) {
  fp8_tile_config cfg;
  // UE8M0-scaled blockwise GEMMs share the blockwise tiles and tables
  int st = resolve_config(kind == FP8_KIND_BLOCKWISE_UE8M0 ? FP8_KIND_BLOCKWISE : kind, M, N, K, cfg_in,
                          &cfg);
  if (st) return st;
  GemmArgs p{};
  p.a = a; p.b = b; p.sa = sa; p.sa_ld = sa_ld; p.sb = sb; p.bias = bias; p.out = out;
  p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.ldc = ldc;
  int splits = 1, per = (int)((K + 127) / 128);
  if (cfg.variant == FP8_VARIANT_DECODE) decode_split_plan(K, cfg.split_k, &splits, &per);
  else if (cfg.variant != FP8_VARIANT_SKINNY) split_plan(K, cfg.bk, cfg.split_k, &splits, &per);
  p.split_k = splits;
  p.k_tiles_per_split = per;
  if (splits > 1) {
    // the kernels address one tile's partials (all splits) with 32-bit offsets
    const VariantInfo vi = variant_info(cfg.variant);
    if ((int64_t)splits * vi.bm * vi.bn * (int64_t)sizeof(float) > INT32_MAX)
      return fail(FP8_ERR_UNSUPPORTED, "%s: split_k=%d keeps more than 2 GiB of partials per tile", fn,
                  splits);
    // ws layout: kCounterBytes of arrival counters (zero between calls), then partials
    const size_t need = variant_workspace_bytes(cfg.variant, splits, M, N);
    if (!ws || ws_bytes < need)
      return fail(FP8_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws ? ws_bytes : 0);
    if (!aligned(ws, 256)) return fail(FP8_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
    const int64_t tiles = variant_tiles(cfg.variant, M, N);
    if (tiles > kMaxSplitTiles)
      return fail(FP8_ERR_UNSUPPORTED, "%s: split-K over %lld output tiles (max %lld)", fn,
                  (long long)tiles, (long long)kMaxSplitTiles);
    p.ws_count = static_cast<int*>(ws);
    p.ws_part = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  return hip_status(launch_gemm(kind, cfg.variant, p, stream), fn);
}

// The linear's config: as the GEMM's, except that with none given the decode
// stream runs unsplit at M <= kFusedRows (its single-launch form does not
// split K; the two launches then compute the same bits).
int resolve_linear_config(int kind, int64_t M, int64_t N, int64_t K, const fp8_tile_config* cfg_in,
                          fp8_tile_config* out) {
  const int st = resolve_config(kind, M, N, K, cfg_in, out);
  if (st) return st;
  if ((!cfg_in || cfg_in->variant == FP8_VARIANT_DEFAULT) && out->variant == FP8_VARIANT_DECODE &&
      M <= kFusedRows)
    out->split_k = 1;
  return FP8_OK;
}

// FP8W8A8_FUSED_LINEAR=0 turns the single-launch linear off; =all takes it at
// every M <= kFusedRows whatever the quantizer flags (for measuring the
// flag-dependent limits below). Read per call.
int fused_linear_mode() {
  const char* v = std::getenv("FP8W8A8_FUSED_LINEAR");
  if (v && v[0] == '0' && v[1] == '\0') return 0;
  if (v && std::string(v) == "all") return 2;
  return 1;
}

// With SiLU-and-mul every workgroup of the fused launch evaluates SiLU over
// the whole activation (per token twice: the row maximum first), which pays
// off only for the fewest rows: measured on the down projections (4096x12288
// channelwise, 4096x1536 and 7168x2048 blockwise), one launch is 1.7 us
// faster at M = 1 channelwise and 1.4-3.8 us at M <= 2 blockwise, but 4-15 us
// slower at M = 2 and 4 channelwise and up to 2 us slower at M = 4 blockwise.
// The decode stream's fused form computes SiLU once per value (it keeps the
// activation in registers between the row maximum and the quantization) and
// fuses every flag.
bool linear_fuses(int kind, const fp8_tile_config& cfg, int64_t M, int64_t N, int64_t K, int64_t ldb,
                  int32_t flags) {
  const int mode = fused_linear_mode();
  if (M > kFusedRows || mode == 0) return false;
  if (cfg.variant == FP8_VARIANT_DECODE) {
    if (cfg.split_k > 1) return false;
    GemmArgs p{};
    p.M = M; p.N = N; p.K = K; p.ldb = ldb;
    return decode_fused_launchable(p, (flags & FP8_QUANT_FUSE_SILU_MUL) != 0);
  }
  if (cfg.variant != FP8_VARIANT_SKINNY) return false;
  if ((flags & FP8_QUANT_FUSE_SILU_MUL) && mode == 1) return M <= (kind == FP8_KIND_CHANNELWISE ? 1 : 2);
  return true;
}

// Activation quantization then scaled GEMM; one fused launch when the skinny
// kernel or the decode stream serves M <= kFusedRows, else the quantizer and
// the GEMM back to back.
int run_linear(const char* fn, int kind, const uint16_t* x, const uint8_t* b, const float* b_scale,
               const uint16_t* bias, uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t ldx,
               int64_t ldb, int64_t ldc, int32_t row_alignment, float eps, uint8_t* q, int64_t ldq,
               float* a_scale, void* ws, size_t ws_bytes, const fp8_tile_config* cfg_in,
               int32_t flags, hipStream_t stream) {
  const bool bw = kind == FP8_KIND_BLOCKWISE;
  if (bw && row_alignment < 1) return fail(FP8_ERR_INVALID, "%s: row_alignment must be >= 1", fn);
  int st = check_quant_flags(fn, flags);
  if (st) return st;
  st = check_quant(fn, x, M, K, (flags & FP8_QUANT_FUSE_SILU_MUL) ? 2 * K : K, ldx, q, ldq, a_scale, eps);
  if (st) return st;
  st = check_gemm(fn, q, b, a_scale, b_scale, bias, out, M, N, K, ldq, ldb, ldc);
  if (st) return st;
  if (M == 0) return ok();
  if (bw && (N % 128 != 0 || K % 128 != 0))
    return fail(FP8_ERR_UNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N,
                (long long)K);
  const int64_t m_pad = bw ? fp8_padded_rows(M, row_alignment) : M;
  fp8_tile_config cfg;
  st = resolve_linear_config(kind, M, N, K, cfg_in, &cfg);
  if (st) return st;
  if (linear_fuses(kind, cfg, M, N, K, ldb, flags)) {
    GemmArgs p{};
    p.a = q; p.b = b; p.sa = a_scale; p.sa_ld = m_pad; p.sb = b_scale; p.bias = bias; p.out = out;
    p.M = M; p.N = N; p.K = K; p.lda = ldq; p.ldb = ldb; p.ldc = ldc;
    p.split_k = 1;
    p.k_tiles_per_split = (int)((K + 127) / 128);
    const QuantArgs qa{x, ldx, q, ldq, a_scale, m_pad, eps};
    return hip_status(launch_linear_fused(kind, p, qa, flags, cfg.variant == FP8_VARIANT_DECODE, stream), fn);
  }
  const hipError_t e = bw ? launch_quant_per_token_group(x, M, K, ldx, 128, m_pad, q, ldq, a_scale, eps, flags, stream)
                          : launch_quant_per_token(x, M, K, ldx, q, ldq, a_scale, eps, flags, stream);
  st = hip_status(e, fn);
  if (st) return st;
  // blockwise with power-of-two scales: the block-scaled MFMA tiles
  const int gemm_kind = bw && (flags & FP8_QUANT_SCALE_UE8M0) ? FP8_KIND_BLOCKWISE_UE8M0 : kind;
  return run_gemm(fn, gemm_kind, q, b, a_scale, m_pad, b_scale, bias, out, M, N, K, ldq, ldb, ldc, ws,
                  ws_bytes, &cfg, stream);
}

}  // namespace

extern "C" {

int64_t fp8_padded_rows(int64_t M, int32_t row_alignment) {
  if (M < 0 || row_alignment < 1) return -1;
  return (M + row_alignment - 1) / row_alignment * row_alignment;
}

int fp8_quant_per_token_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                           int64_t ldq, float* scale, float eps, int32_t flags, hipStream_t stream) {
  const char* fn = "fp8_quant_per_token";
  int st = check_quant_flags(fn, flags);
  if (st) return st;
  st = check_quant(fn, x, M, K, (flags & FP8_QUANT_FUSE_SILU_MUL) ? 2 * K : K, ldx, q, ldq, scale,
                   eps);
  if (st) return st;
  if (M == 0) return ok();
  return hip_status(launch_quant_per_token(x, M, K, ldx, q, ldq, scale, eps, flags, stream), fn);
}

int fp8_quant_per_token(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                        int64_t ldq, float* scale, float eps, hipStream_t stream) {
  return fp8_quant_per_token_ex(x, M, K, ldx, q, ldq, scale, eps, 0, stream);
}

int fp8_quant_per_token_group_ex(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                 int32_t group_size, int32_t row_alignment, uint8_t* q,
                                 int64_t ldq, float* scale, float eps, int32_t flags,
                                 hipStream_t stream) {
  const char* fn = "fp8_quant_per_token_group";
  if (row_alignment < 1) return fail(FP8_ERR_INVALID, "%s: row_alignment must be >= 1", fn);
  if (group_size <= 0) return fail(FP8_ERR_INVALID, "%s: group_size must be positive", fn);
  if (K % group_size != 0)
    return fail(FP8_ERR_INVALID, "%s: K=%lld must be divisible by group_size=%d", fn, (long long)K, group_size);
  if (!(group_size == 16 || group_size == 32 || group_size == 64 || group_size == 128))
    return fail(FP8_ERR_UNSUPPORTED, "%s: group_size %d not in {16, 32, 64, 128}", fn, group_size);
  int st = check_quant_flags(fn, flags);
  if (st) return st;
  st = check_quant(fn, x, M, K, (flags & FP8_QUANT_FUSE_SILU_MUL) ? 2 * K : K, ldx, q, ldq, scale,
                   eps);
  if (st) return st;
  if (M == 0) return ok();
  const int64_t m_pad = fp8_padded_rows(M, row_alignment);
  return hip_status(launch_quant_per_token_group(x, M, K, ldx, group_size, m_pad, q, ldq, scale,
                                                 eps, flags, stream),
                    fn);
}

int fp8_quant_per_token_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              int32_t group_size, int32_t row_alignment, uint8_t* q, int64_t ldq,
                              float* scale, float eps, hipStream_t stream) {
  return fp8_quant_per_token_group_ex(x, M, K, ldx, group_size, row_alignment, q, ldq, scale, eps,
                                      0, stream);
}

int fp8_quant_per_token_group_masked(const uint16_t* x, int64_t E, int64_t M_max, int64_t K,
                                     int64_t ldx, const int32_t* masked_m, int32_t group_size,
                                     int32_t row_alignment, uint8_t* q, int64_t ldq, float* scale,
                                     float eps, int32_t flags, hipStream_t stream) {
  const char* fn = "fp8_quant_per_token_group_masked";
  if (E < 0 || E > 65535) return fail(FP8_ERR_INVALID, "%s: E=%lld outside [0, 65535]", fn, (long long)E);
  if (E == 0) return ok();
  if (row_alignment < 1) return fail(FP8_ERR_INVALID, "%s: row_alignment must be >= 1", fn);
  if (group_size <= 0) return fail(FP8_ERR_INVALID, "%s: group_size must be positive", fn);
  if (K % group_size != 0)
    return fail(FP8_ERR_INVALID, "%s: K=%lld must be divisible by group_size=%d", fn, (long long)K, group_size);
  if (!(group_size == 16 || group_size == 32 || group_size == 64 || group_size == 128))
    return fail(FP8_ERR_UNSUPPORTED, "%s: group_size %d not in {16, 32, 64, 128}", fn, group_size);
  int st = check_quant_flags(fn, flags);
  if (st) return st;
  st = check_quant(fn, x, M_max, K, (flags & FP8_QUANT_FUSE_SILU_MUL) ? 2 * K : K, ldx, q, ldq, scale,
                   eps);
  if (st) return st;
  if (M_max == 0 || E == 0) return ok();
  if (!masked_m || !aligned(masked_m, 4)) return fail(FP8_ERR_INVALID, "%s: masked_m must be a 4-byte aligned pointer", fn);
  const int64_t m_pad = fp8_padded_rows(M_max, row_alignment);
  const MaskArgs mask{masked_m, M_max * ldx, m_pad * ldq, (K / group_size) * m_pad};
  return hip_status(launch_quant_per_token_group_masked(x, E, M_max, K, ldx, group_size, m_pad, q, ldq,
                                                        scale, eps, flags, mask, stream),
                    fn);
}

int fp8_scaled_mm_blockwise_masked(const uint8_t* a, const uint8_t* b, const float* a_scale,
                                   int64_t a_scale_ld, const float* b_scale, uint16_t* out,
                                   const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N,
                                   int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                                   int32_t scale_ue8m0, const fp8_tile_config* cfg_in,
                                   hipStream_t stream) {
  const char* fn = "fp8_scaled_mm_blockwise_masked";
  if (E < 0 || E > 65535) return fail(FP8_ERR_INVALID, "%s: E=%lld outside [0, 65535]", fn, (long long)E);
  if (E == 0) return ok();
  int st = check_gemm(fn, a, b, a_scale, b_scale, nullptr, out, M_max, N, K, lda, ldb, ldc);
  if (st) return st;
  if (M_max == 0 || E == 0) return ok();
  if (!masked_m || !aligned(masked_m, 4)) return fail(FP8_ERR_INVALID, "%s: masked_m must be a 4-byte aligned pointer", fn);
  if (N % 128 != 0 || K % 128 != 0)
    return fail(FP8_ERR_UNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N,
                (long long)K);
  if (a_scale_ld < M_max || a_scale_ld % 4 != 0)
    return fail(FP8_ERR_INVALID, "%s: a_scale_ld=%lld must be >= M_max=%lld and a multiple of 4", fn,
                (long long)a_scale_ld, (long long)M_max);
  fp8_tile_config cfg;
  st = resolve_config(FP8_KIND_BLOCKWISE, M_max, N, K, cfg_in, &cfg);
  if (st) return st;
  if (!cfg_in || cfg_in->variant == FP8_VARIANT_DEFAULT) {
    // Grouped default by rows per expert, not the single-GEMM table: with E
    // expert weights the grid and the weight bytes are E times those of one
    // GEMM of M_max rows. Measured over 8 experts of the blockwise workload's
    // expert shapes (3072x4096 and 4096x1536), this rule was best or within
    // 7% at every M_max from 4 to 1024, and 20-35% faster than the table's
    // tile at M_max 64-1024. Unsplit: the split-K counters are per tile, not
    // per expert.
    cfg.variant = M_max <= 64 ? FP8_VARIANT_T64x64PANEL
                              : (M_max <= 128 ? FP8_VARIANT_T128x128PANEL8
                                              : (M_max <= 256 ? FP8_VARIANT_T256x128PANEL
                                                              : FP8_VARIANT_T256x256BW16));
    cfg.split_k = 1;
  }
  if (cfg.split_k != 1) return fail(FP8_ERR_INVALID, "%s: grouped GEMMs take split_k == 1", fn);
  GemmArgs p{};
  p.a = a; p.b = b; p.sa = a_scale; p.sa_ld = a_scale_ld; p.sb = b_scale; p.bias = nullptr; p.out = out;
  p.M = M_max; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.ldc = ldc;
  p.split_k = 1;
  p.k_tiles_per_split = (int)(K / 128);
  p.masked_m = masked_m;
  p.experts = (int)E;
  p.a_es = a_scale_ld * lda;
  p.sa_es = (K / 128) * a_scale_ld;
  p.b_es = N * ldb;
  p.sb_es = (N / 128) * (K / 128);
  p.out_es = M_max * ldc;
  if (!grouped_launchable(cfg.variant, p))
    return fail(FP8_ERR_UNSUPPORTED, "%s: variant %d is not a blockwise panel tile, or the offsets exceed "
                "its 32-bit DMA range", fn, cfg.variant);
  return hip_status(launch_gemm(scale_ue8m0 ? kBlockwiseE8 : kBlockwise, cfg.variant, p, stream), fn);
}

int fp8_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const float* scale,
                     uint8_t* q, int64_t ldq, hipStream_t stream) {
  const char* fn = "fp8_quant_static";
  int st = check_quant(fn, x, M, K, K, ldx, q, ldq, scale, 0.0f);
  if (st) return st;
  if (M == 0) return ok();
  return hip_status(launch_quant_static(x, M, K, ldx, scale, q, ldq, stream), fn);
}

int fp8_scaled_mm_channelwise_ex(const uint8_t* a, const uint8_t* b, const float* a_scale,
                                 const float* b_scale, const uint16_t* bias, uint16_t* out,
                                 int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                                 int64_t ldc, void* ws, size_t ws_bytes,
                                 const fp8_tile_config* cfg, hipStream_t stream) {
  const char* fn = "fp8_scaled_mm_channelwise";
  int st = check_gemm(fn, a, b, a_scale, b_scale, bias, out, M, N, K, lda, ldb, ldc);
  if (st) return st;
  if (M == 0) return ok();
  return run_gemm(fn, FP8_KIND_CHANNELWISE, a, b, a_scale, 0, b_scale, bias, out, M, N, K, lda,
                  ldb, ldc, ws, ws_bytes, cfg, stream);
}

int fp8_scaled_mm_channelwise(const uint8_t* a, const uint8_t* b, const float* a_scale,
                              const float* b_scale, const uint16_t* bias, uint16_t* out,
                              int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                              int64_t ldc, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fp8_scaled_mm_channelwise_ex(a, b, a_scale, b_scale, bias, out, M, N, K, lda, ldb, ldc,
                                      ws, ws_bytes, nullptr, stream);
}

int fp8_scaled_mm_blockwise_ex(const uint8_t* a, const uint8_t* b, const float* a_scale,
                               int64_t a_scale_ld, const float* b_scale, const uint16_t* bias,
                               uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t lda,
                               int64_t ldb, int64_t ldc, void* ws, size_t ws_bytes,
                               const fp8_tile_config* cfg, hipStream_t stream) {
  const char* fn = "fp8_scaled_mm_blockwise";
  int st = check_gemm(fn, a, b, a_scale, b_scale, bias, out, M, N, K, lda, ldb, ldc);
  if (st) return st;
  if (M == 0) return ok();
  if (N % 128 != 0 || K % 128 != 0)
    return fail(FP8_ERR_UNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N,
                (long long)K);
  if (a_scale_ld < M) return fail(FP8_ERR_INVALID, "%s: a_scale_ld=%lld < M=%lld", fn, (long long)a_scale_ld, (long long)M);
  return run_gemm(fn, FP8_KIND_BLOCKWISE, a, b, a_scale, a_scale_ld, b_scale, bias, out, M, N, K,
                  lda, ldb, ldc, ws, ws_bytes, cfg, stream);
}

int fp8_scaled_mm_blockwise(const uint8_t* a, const uint8_t* b, const float* a_scale,
                            int64_t a_scale_ld, const float* b_scale, const uint16_t* bias,
                            uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t lda,
                            int64_t ldb, int64_t ldc, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return fp8_scaled_mm_blockwise_ex(a, b, a_scale, a_scale_ld, b_scale, bias, out, M, N, K, lda,
                                    ldb, ldc, ws, ws_bytes, nullptr, stream);
}

int fp8_scaled_mm_blockwise_ue8m0_ex(const uint8_t* a, const uint8_t* b, const float* a_scale,
                                     int64_t a_scale_ld, const float* b_scale, const uint16_t* bias,
                                     uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t lda,
                                     int64_t ldb, int64_t ldc, void* ws, size_t ws_bytes,
                                     const fp8_tile_config* cfg, hipStream_t stream) {
  const char* fn = "fp8_scaled_mm_blockwise_ue8m0";
  int st = check_gemm(fn, a, b, a_scale, b_scale, bias, out, M, N, K, lda, ldb, ldc);
  if (st) return st;
  if (M == 0) return ok();
  if (N % 128 != 0 || K % 128 != 0)
    return fail(FP8_ERR_UNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N,
                (long long)K);
  if (a_scale_ld < M) return fail(FP8_ERR_INVALID, "%s: a_scale_ld=%lld < M=%lld", fn, (long long)a_scale_ld, (long long)M);
  return run_gemm(fn, FP8_KIND_BLOCKWISE_UE8M0, a, b, a_scale, a_scale_ld, b_scale, bias, out, M, N,
                  K, lda, ldb, ldc, ws, ws_bytes, cfg, stream);
}

int fp8_scaled_mm_blockwise_ue8m0(const uint8_t* a, const uint8_t* b, const float* a_scale,
                                  int64_t a_scale_ld, const float* b_scale, const uint16_t* bias,
                                  uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t lda,
                                  int64_t ldb, int64_t ldc, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return fp8_scaled_mm_blockwise_ue8m0_ex(a, b, a_scale, a_scale_ld, b_scale, bias, out, M, N, K,
                                          lda, ldb, ldc, ws, ws_bytes, nullptr, stream);
}

int fp8_scaled_mm_noalloc(int32_t kind, const uint8_t* a, const uint8_t* b, const float* a_scale,
                          int64_t a_scale_ld, const float* b_scale, const uint16_t* bias,
                          uint16_t* out, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                          int64_t ldc, const fp8_tile_config* cfg, hipStream_t stream) {
  const char* fn = "fp8_scaled_mm_noalloc";
  if (kind != FP8_KIND_CHANNELWISE && kind != FP8_KIND_BLOCKWISE && kind != FP8_KIND_BLOCKWISE_UE8M0)
    return fail(FP8_ERR_INVALID, "%s: unknown kind %d", fn, (int)kind);
  int st = check_gemm(fn, a, b, a_scale, b_scale, bias, out, M, N, K, lda, ldb, ldc);
  if (st) return st;
  if (M == 0) return ok();
  const bool bw = kind != FP8_KIND_CHANNELWISE;
  if (bw) {
    if (N % 128 != 0 || K % 128 != 0)
      return fail(FP8_ERR_UNSUPPORTED, "%s: N=%lld and K=%lld must be multiples of 128", fn, (long long)N,
                  (long long)K);
    if (a_scale_ld < M)
      return fail(FP8_ERR_INVALID, "%s: a_scale_ld=%lld < M=%lld", fn, (long long)a_scale_ld, (long long)M);
  }
  // the scratch this call's split-K plan needs, decided on the host before
  // any device work
  fp8_tile_config plan;
  st = resolve_config(bw ? FP8_KIND_BLOCKWISE : FP8_KIND_CHANNELWISE, M, N, K, cfg, &plan);
  if (st) return st;
  const size_t need = fp8_scaled_mm_workspace_size(kind, M, N, K, &plan);
  if (need > kStaticScratchBytes)
    return fail(FP8_ERR_WORKSPACE,
                "%s: the split-K plan of this call (variant %d, split_k %d) needs %zu bytes of scratch; "
                "the library's static scratch holds %zu (ask for fewer splits or a larger tile, or call "
                "the workspace-taking GEMM)", fn, plan.variant, plan.split_k, need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = hip_status(static_scratch(stream, &ws), fn);
    if (st) return st;
  }
  return run_gemm(fn, kind, a, b, a_scale, bw ? a_scale_ld : 0, b_scale, bias, out, M, N, K, lda, ldb, ldc,
                  ws, need > 0 ? kStaticScratchBytes : 0, &plan, stream);
}

size_t fp8_scaled_mm_workspace_size(int32_t kind, int64_t M, int64_t N, int64_t K,
                                    const fp8_tile_config* cfg_in) {
  if (kind == FP8_KIND_BLOCKWISE_UE8M0) kind = FP8_KIND_BLOCKWISE;  // same tiles
  if ((kind != FP8_KIND_CHANNELWISE && kind != FP8_KIND_BLOCKWISE) || M < 0 || N < 0 || K < 0)
    return (size_t)-1;
  if (M == 0 || N == 0 || K == 0) return 0;
  fp8_tile_config cfg;
  if (resolve_config(kind, M, N, K, cfg_in, &cfg)) return (size_t)-1;
  if (cfg.variant == FP8_VARIANT_SKINNY) return 0;
  int splits, per;
  if (cfg.variant == FP8_VARIANT_DECODE) decode_split_plan(K, cfg.split_k, &splits, &per);
  else split_plan(K, cfg.bk, cfg.split_k, &splits, &per);
  return variant_workspace_bytes(cfg.variant, splits, M, N);
}

int fp8_linear_channelwise_ex(const uint16_t* x, const uint8_t* b, const float* b_scale,
                              const uint16_t* bias, uint16_t* out, int64_t M, int64_t N, int64_t K,
                              int64_t ldx, int64_t ldb, int64_t ldc, float eps, uint8_t* q,
                              int64_t ldq, float* a_scale, void* ws, size_t ws_bytes,
                              const fp8_tile_config* cfg, int32_t flags, hipStream_t stream) {
  return run_linear("fp8_linear_channelwise", FP8_KIND_CHANNELWISE, x, b, b_scale, bias, out, M, N,
                    K, ldx, ldb, ldc, 1, eps, q, ldq, a_scale, ws, ws_bytes, cfg, flags, stream);
}

int fp8_linear_channelwise(const uint16_t* x, const uint8_t* b, const float* b_scale,
                           const uint16_t* bias, uint16_t* out, int64_t M, int64_t N, int64_t K,
                           int64_t ldx, int64_t ldb, int64_t ldc, float eps, uint8_t* q,
                           int64_t ldq, float* a_scale, void* ws, size_t ws_bytes,
                           const fp8_tile_config* cfg, hipStream_t stream) {
  return fp8_linear_channelwise_ex(x, b, b_scale, bias, out, M, N, K, ldx, ldb, ldc, eps, q, ldq,
                                   a_scale, ws, ws_bytes, cfg, 0, stream);
}

int fp8_linear_blockwise_ex(const uint16_t* x, const uint8_t* b, const float* b_scale,
                            const uint16_t* bias, uint16_t* out, int64_t M, int64_t N, int64_t K,
                            int64_t ldx, int64_t ldb, int64_t ldc, int32_t row_alignment, float eps,
                            uint8_t* q, int64_t ldq, float* a_scale, void* ws, size_t ws_bytes,
                            const fp8_tile_config* cfg, int32_t flags, hipStream_t stream) {
  return run_linear("fp8_linear_blockwise", FP8_KIND_BLOCKWISE, x, b, b_scale, bias, out, M, N, K,
                    ldx, ldb, ldc, row_alignment, eps, q, ldq, a_scale, ws, ws_bytes, cfg, flags,
                    stream);
}

int fp8_linear_blockwise(const uint16_t* x, const uint8_t* b, const float* b_scale,
                         const uint16_t* bias, uint16_t* out, int64_t M, int64_t N, int64_t K,
                         int64_t ldx, int64_t ldb, int64_t ldc, int32_t row_alignment, float eps,
                         uint8_t* q, int64_t ldq, float* a_scale, void* ws, size_t ws_bytes,
                         const fp8_tile_config* cfg, hipStream_t stream) {
  return fp8_linear_blockwise_ex(x, b, b_scale, bias, out, M, N, K, ldx, ldb, ldc, row_alignment, eps,
                                 q, ldq, a_scale, ws, ws_bytes, cfg, 0, stream);
}

int fp8_linear_launches_ex(int32_t kind, int64_t M, int64_t N, int64_t K, const fp8_tile_config* cfg_in,
                           int32_t flags) {
  if ((kind != FP8_KIND_CHANNELWISE && kind != FP8_KIND_BLOCKWISE) || M < 0 || N <= 0 || K <= 0)
    return fail(FP8_ERR_INVALID, "fp8_linear_launches: bad arguments");
  int st = check_quant_flags("fp8_linear_launches", flags);
  if (st) return st;
  if (M == 0) return 0;
  fp8_tile_config cfg;
  st = resolve_linear_config(kind, M, N, K, cfg_in, &cfg);
  if (st) return st;
  return linear_fuses(kind, cfg, M, N, K, K, flags) ? 1 : 2;  // a contiguous weight
}

int fp8_linear_launches(int32_t kind, int64_t M, int64_t N, int64_t K, const fp8_tile_config* cfg_in) {
  return fp8_linear_launches_ex(kind, M, N, K, cfg_in, 0);
}

int fp8_tile_config_lookup(int32_t kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out) {
  if ((kind != FP8_KIND_CHANNELWISE && kind != FP8_KIND_BLOCKWISE) || N <= 0 || K <= 0 || M < 0 || !out)
    return fail(FP8_ERR_INVALID, "fp8_tile_config_lookup: bad arguments");
  return lookup_config(kind, N, K, M, out);
}

int fp8_tile_config_default(int32_t kind, int64_t N, int64_t K, int64_t M, fp8_tile_config* out) {
  if ((kind != FP8_KIND_CHANNELWISE && kind != FP8_KIND_BLOCKWISE) || N <= 0 || K <= 0 || M < 0 || !out)
    return fail(FP8_ERR_INVALID, "fp8_tile_config_default: bad arguments");
  return default_config(kind, N, K, M, out);
}

int fp8_tile_config_set_dir(const char* dir) {
  set_config_dir(dir);
  return FP8_OK;
}

int fp8_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                          hipStream_t stream) {
  const char* fn = "fp8_probe_stream_read";
  if (!src || !sink || bytes < 16 || bytes % 16 != 0 || !aligned(src, 16) || workgroups < 1)
    return fail(FP8_ERR_INVALID, "%s: src 16-byte aligned, bytes a positive multiple of 16, workgroups >= 1", fn);
  return hip_status(launch_probe_stream_read(src, bytes, sink, workgroups, stream), fn);
}

int fp8_probe_strided_read(const void* src, int64_t rows, int64_t row_bytes, int32_t rows_per_wg,
                           int32_t piece, uint32_t* sink, hipStream_t stream) {
  const char* fn = "fp8_probe_strided_read";
  const bool piece_ok = piece == 16 || piece == 32 || piece == 64 || piece == 128 || piece == 256 ||
                        piece == 512 || piece == 1024;
  if (!src || !sink || !aligned(src, 16) || !piece_ok || rows_per_wg < 1 || rows < rows_per_wg ||
      rows % rows_per_wg != 0 || row_bytes % piece != 0 || row_bytes % 16 != 0 ||
      (rows_per_wg * piece) % 1024 != 0 || rows / rows_per_wg > 65535)
    return fail(FP8_ERR_INVALID, "%s: piece a power of two in [16, 1024] dividing row_bytes, rows a multiple "
                "of rows_per_wg, rows_per_wg * piece a multiple of 1024", fn);
  return hip_status(launch_probe_strided_read(src, rows, row_bytes, rows_per_wg, piece, sink, stream), fn);
}

int fp8_probe_l2_feed(const void* src, size_t window_bytes, int32_t reps, int32_t dma, uint32_t* sink,
                      int32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8_probe_l2_feed";
  if (!src || !sink || window_bytes < 4096 || window_bytes % 1024 != 0 || !aligned(src, 16) || reps < 1 ||
      workgroups < 1)
    return fail(FP8_ERR_INVALID, "%s: src 16-byte aligned, window a multiple of 1 KB (>= 4 KB), reps and "
                "workgroups >= 1", fn);
  return hip_status(launch_probe_l2_feed(src, window_bytes, reps, dma != 0, sink, workgroups, stream), fn);
}

int fp8_probe_panel_feed(const void* src, int32_t row_bytes, int32_t panels, int32_t stages, int32_t mode,
                         uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8_probe_panel_feed";
  if (!src || !sink || row_bytes < 128 || row_bytes % 128 != 0 || panels < 1 || stages < 1 || mode < 0 ||
      mode > 3 || workgroups < 1 || (uint64_t)panels * 64 * (uint64_t)row_bytes > 0xFFFFFFFFull)
    return fail(FP8_ERR_INVALID, "%s: row_bytes a positive multiple of 128, panels, stages and workgroups >= 1, "
                "mode 0-3, panels * 64 * row_bytes < 4 GiB", fn);
  return hip_status(launch_probe_panel_feed(src, (uint32_t)row_bytes, panels, stages, mode, sink, workgroups, stream),
                    fn);
}

int fp8_probe_mfma(int32_t iters, float* sink, int32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8_probe_mfma";
  if (!sink || iters < 1 || workgroups < 1)
    return fail(FP8_ERR_INVALID, "%s: iters and workgroups >= 1, sink non-null", fn);
  return hip_status(launch_probe_mfma(iters, sink, workgroups, stream), fn);
}

int fp8_probe_wave_read(const void* src, size_t bytes, int32_t threads, int32_t depth, int32_t dma,
                        uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8_probe_wave_read";
  const bool shape_ok = (threads == 256 && (depth == 4 || depth == 8 || depth == 16)) ||
                        (threads == 512 && (depth == 4 || depth == 8 || depth == 16)) ||
                        (threads == 1024 && (depth == 4 || depth == 8));
  if (!src || !sink || !aligned(src, 16) || bytes < 1024 || bytes % 1024 != 0 || workgroups < 1 || !shape_ok)
    return fail(FP8_ERR_INVALID, "%s: bytes a positive multiple of 1 KB, (threads, depth) in {256, 512} x {4, 8, "
                "16} or 1024 x {4, 8}", fn);
  return hip_status(launch_probe_wave_read(src, bytes, threads, depth, dma != 0, sink, workgroups, stream), fn);
}

int fp8_probe_lds(int32_t iters, int32_t threads, uint32_t* sink, int32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8_probe_lds";
  if (!sink || iters < 1 || workgroups < 1 || (threads != 256 && threads != 512))
    return fail(FP8_ERR_INVALID, "%s: iters and workgroups >= 1, threads 256 or 512, sink non-null", fn);
  return hip_status(launch_probe_lds(iters, threads, sink, workgroups, stream), fn);
}

int fp8_probe_mfma_dot(const void* w, const void* x, const float* c, float* d, int32_t count, int32_t form,
                       hipStream_t stream) {
  const char* fn = "fp8_probe_mfma_dot";
  if (!w || !x || !c || !d || count < 1 || count > 65535 || (form != 0 && form != 1) || !aligned(w, 16) ||
      !aligned(x, 16))
    return fail(FP8_ERR_INVALID, "%s: non-null 16-byte-aligned operands, 1 <= count <= 65535, form 0 or 1", fn);
  return hip_status(launch_probe_mfma_dot(w, x, c, d, count, form, stream), fn);
}

const char* fp8_last_error(void) { return g_last_error.c_str(); }

int32_t fp8_version(void) { return 100; }

}  // extern "C"
