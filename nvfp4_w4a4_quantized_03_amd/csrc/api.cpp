// C ABI front end: argument validation on the host, then kernel dispatch.
// Every check runs before any HIP call, so a rejected call touches no
// device state (and can be exercised on a machine without a GPU).
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/nvfp4_w4a4.h"
#include "internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// [lo, lo + len) and [lo2, lo2 + len2) intersect (byte ranges).
bool overlap(const void* a, int64_t alen, const void* b, int64_t blen) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(blen) &&
         y < x + static_cast<uintptr_t>(alen);
}

// Sizes whose byte extents stay far below 2^62.
constexpr int64_t kMaxDim = int64_t(1) << 40;

int status_of(hipError_t e) {
  return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

// Shared checks of a [rows][k] input tensor x (k % 16 == 0, ldx >= k,
// 16-byte aligned rows).  Returns NVFP4_OK or the status to report.
int check_x(const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx) {
  if (!x) return NVFP4_ERR_INVALID_VALUE;
  if (rows < 1 || k < 16 || k % 16 != 0 || ldx < k) return NVFP4_ERR_INVALID_VALUE;
  if (rows > kMaxDim || ldx > kMaxDim || rows > kMaxDim / ldx)
    return NVFP4_ERR_INVALID_VALUE;
  if (rows * (k / 16) > (int64_t(1) << 39)) return NVFP4_ERR_INVALID_VALUE;
  if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  const int64_t es = x_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0) return NVFP4_ERR_MISALIGNED;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_abi_version(void) { return 3; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_VALUE:
      return "NVFP4_ERR_INVALID_VALUE: null pointer, bad size, k not a "
             "multiple of 16, bad stride or overlapping buffers";
    case NVFP4_ERR_UNSUPPORTED:
      return "NVFP4_ERR_UNSUPPORTED: unknown dtype, global mode or epilogue, "
             "or a shape outside the call's kernels (gate pair: more than 256 "
             "columns or k not a multiple of 128; fused quantise + GEMM: more "
             "than 64 rows or k not a multiple of 128)";
    case NVFP4_ERR_MISALIGNED:
      return "NVFP4_ERR_MISALIGNED: a pointer or row stride breaks the "
             "required alignment";
    case NVFP4_ERR_LAUNCH:
      return "NVFP4_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    default: return "unknown nvfp4 status";
  }
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t k,
                   int64_t ldx, uint8_t* codes, uint8_t* scales,
                   float* global, int mode, void* stream) {
  if (!x || !codes || !scales || !global) return NVFP4_ERR_INVALID_VALUE;
  if (rows < 1 || k < 16 || k % 16 != 0 || ldx < k) return NVFP4_ERR_INVALID_VALUE;
  if (rows > kMaxDim || ldx > kMaxDim || rows > kMaxDim / ldx)
    return NVFP4_ERR_INVALID_VALUE;
  if (rows * (k / 16) > (int64_t(1) << 39)) return NVFP4_ERR_INVALID_VALUE;
  if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  if (mode != NVFP4_GLOBAL_COMPUTE && mode != NVFP4_GLOBAL_GIVEN)
    return NVFP4_ERR_UNSUPPORTED;
  const int64_t es = x_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0 || !aligned(codes, 8) ||
      !aligned(global, 4))
    return NVFP4_ERR_MISALIGNED;
  const int64_t xbytes = ((rows - 1) * ldx + k) * es;
  const int64_t cbytes = rows * (k / 2), sbytes = rows * (k / 16);
  if (overlap(x, xbytes, codes, cbytes) || overlap(x, xbytes, scales, sbytes) ||
      overlap(x, xbytes, global, 4) || overlap(codes, cbytes, scales, sbytes) ||
      overlap(codes, cbytes, global, 4) || overlap(scales, sbytes, global, 4))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_quantize(x, x_dtype, rows, k, ldx, codes,
                                          scales, global, mode,
                                          static_cast<hipStream_t>(stream)));
}

int nvfp4_harmonize_group(uint8_t* scales, int64_t k,
                          const int64_t* row_offsets, int n_modules,
                          const float* module_globals, float* shared_global,
                          void* stream) {
  if (!scales || !row_offsets || !module_globals || !shared_global)
    return NVFP4_ERR_INVALID_VALUE;
  if (k < 16 || k % 16 != 0 || k > kMaxDim) return NVFP4_ERR_INVALID_VALUE;
  if (n_modules < 1 || n_modules > nvfp4::kMaxModules)
    return NVFP4_ERR_INVALID_VALUE;
  if (row_offsets[0] != 0) return NVFP4_ERR_INVALID_VALUE;
  for (int i = 0; i < n_modules; ++i)
    if (row_offsets[i + 1] <= row_offsets[i]) return NVFP4_ERR_INVALID_VALUE;
  const int64_t total_rows = row_offsets[n_modules];
  if (total_rows > kMaxDim || total_rows > (int64_t(1) << 39) / (k / 16))
    return NVFP4_ERR_INVALID_VALUE;
  if (!aligned(scales, 16) || !aligned(module_globals, 4) || !aligned(shared_global, 4))
    return NVFP4_ERR_MISALIGNED;
  const int64_t sbytes = total_rows * (k / 16);
  if (overlap(shared_global, 4, module_globals, 4 * int64_t(n_modules)) ||
      overlap(shared_global, 4, scales, sbytes) ||
      overlap(module_globals, 4 * int64_t(n_modules), scales, sbytes))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_harmonize(scales, k, row_offsets, n_modules,
                                           module_globals, shared_global,
                                           static_cast<hipStream_t>(stream)));
}

int w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
              const float* a_global, int64_t m,
              const uint8_t* b_codes, const uint8_t* b_scales,
              const float* b_global, int64_t n, int64_t k,
              void* out, int out_dtype, int64_t ldo, int epilogue,
              void* stream) {
  if (!a_codes || !a_scales || !a_global || !b_codes || !b_scales ||
      !b_global || !out)
    return NVFP4_ERR_INVALID_VALUE;
  if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || ldo < n)
    return NVFP4_ERR_INVALID_VALUE;
  if (m > kMaxDim || n > kMaxDim || k > kMaxDim || ldo > kMaxDim ||
      m > kMaxDim / ldo || m > kMaxDim / k || n > kMaxDim / k)
    return NVFP4_ERR_INVALID_VALUE;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  if (epilogue != W4A4_EPI_NONE && epilogue != W4A4_EPI_ALPHA &&
      epilogue != W4A4_EPI_BETA)
    return NVFP4_ERR_UNSUPPORTED;
  const int64_t os = out_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 16) ||
      !aligned(b_scales, 16) || !aligned(out, 4) || !aligned(a_global, 4) ||
      !aligned(b_global, 4))
    return NVFP4_ERR_MISALIGNED;
  const int64_t obytes = ((m - 1) * ldo + n) * os;
  if (overlap(out, obytes, a_codes, m * (k / 2)) ||
      overlap(out, obytes, a_scales, m * (k / 16)) ||
      overlap(out, obytes, b_codes, n * (k / 2)) ||
      overlap(out, obytes, b_scales, n * (k / 16)) ||
      overlap(out, obytes, a_global, 4) || overlap(out, obytes, b_global, 4))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_gemm(a_codes, a_scales, a_global, m, b_codes,
                                      b_scales, b_global, n, k, out, out_dtype,
                                      ldo, epilogue,
                                      static_cast<hipStream_t>(stream)));
}

int w4a4_gemm_gdn_gates(const uint8_t* x_codes, const uint8_t* x_scales,
                        const float* x_global, int64_t m,
                        const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* w_global, int64_t n_beta, int64_t n_alpha,
                        int64_t k, const float* a_log, const float* dt_bias,
                        float* beta_out, int64_t ld_beta, float* alpha_out,
                        int64_t ld_alpha, void* stream) {
  if (!x_codes || !x_scales || !x_global || !w_codes || !w_scales || !w_global)
    return NVFP4_ERR_INVALID_VALUE;
  if (m < 1 || n_beta < 0 || n_alpha < 0 || n_beta + n_alpha < 1 || k < 16 ||
      k % 16 != 0 || m > kMaxDim || k > kMaxDim || m > kMaxDim / k)
    return NVFP4_ERR_INVALID_VALUE;
  if (n_beta > 0 && (!beta_out || ld_beta < n_beta || m > kMaxDim / ld_beta))
    return NVFP4_ERR_INVALID_VALUE;
  if (n_alpha > 0 && (!alpha_out || !a_log || !dt_bias || ld_alpha < n_alpha ||
                      m > kMaxDim / ld_alpha))
    return NVFP4_ERR_INVALID_VALUE;
  if (n_beta + n_alpha > nvfp4::kMaxGateCols || k % 128 != 0)
    return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(x_scales, 16) ||
      !aligned(w_scales, 16) || !aligned(x_global, 4) || !aligned(w_global, 4) ||
      (n_beta > 0 && !aligned(beta_out, 4)) ||
      (n_alpha > 0 && (!aligned(alpha_out, 4) || !aligned(a_log, 4) ||
                       !aligned(dt_bias, 4))))
    return NVFP4_ERR_MISALIGNED;
  const int64_t n = n_beta + n_alpha;
  struct Range { const void* p; int64_t len; };
  const Range in[] = {{x_codes, m * (k / 2)}, {x_scales, m * (k / 16)},
                      {x_global, 4}, {w_codes, n * (k / 2)},
                      {w_scales, n * (k / 16)}, {w_global, 4},
                      {a_log, 4 * n_alpha}, {dt_bias, 4 * n_alpha}};
  const Range outs[] = {{beta_out, n_beta ? ((m - 1) * ld_beta + n_beta) * 4 : 0},
                        {alpha_out, n_alpha ? ((m - 1) * ld_alpha + n_alpha) * 4 : 0}};
  for (const Range& o : outs) {
    if (o.len == 0) continue;
    for (const Range& i : in)
      if (i.len > 0 && overlap(o.p, o.len, i.p, i.len)) return NVFP4_ERR_INVALID_VALUE;
  }
  if (outs[0].len && outs[1].len && overlap(outs[0].p, outs[0].len, outs[1].p, outs[1].len))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_gdn_gates(x_codes, x_scales, x_global, m, w_codes,
                                           w_scales, w_global, n_beta, n_alpha, k,
                                           a_log, dt_bias, beta_out, ld_beta,
                                           alpha_out, ld_alpha,
                                           static_cast<hipStream_t>(stream)));
}

int w4a4_gemm_quantize_a(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                         uint8_t* x_codes, uint8_t* x_scales, float* x_global, int mode,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         const float* w_global, int64_t n, void* out, int out_dtype,
                         int64_t ldo, void* stream) {
  if (!x_codes || !x_scales || !x_global || !w_codes || !w_scales || !w_global || !out)
    return NVFP4_ERR_INVALID_VALUE;
  const int cx = check_x(x, x_dtype, m, k, ldx);
  if (cx != NVFP4_OK) return cx;
  if (n < 1 || ldo < n || n > kMaxDim || k > kMaxDim || ldo > kMaxDim ||
      m > kMaxDim / ldo || n > kMaxDim / k)
    return NVFP4_ERR_INVALID_VALUE;
  if (mode != NVFP4_GLOBAL_COMPUTE && mode != NVFP4_GLOBAL_GIVEN)
    return NVFP4_ERR_UNSUPPORTED;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  if (m > nvfp4::kMaxFusedRows || k % 128 != 0) return NVFP4_ERR_UNSUPPORTED;
  if (!aligned(x_codes, 16) || !aligned(x_scales, 16) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 16) || !aligned(x_global, 4) || !aligned(w_global, 4) ||
      !aligned(out, 4))
    return NVFP4_ERR_MISALIGNED;
  const int64_t es = x_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  const int64_t os = out_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  struct Range { const void* p; int64_t len; };
  const Range in[] = {{x, ((m - 1) * ldx + k) * es}, {w_codes, n * (k / 2)},
                      {w_scales, n * (k / 16)}, {w_global, 4}};
  const Range outs[] = {{x_codes, m * (k / 2)}, {x_scales, m * (k / 16)},
                        {x_global, 4}, {out, ((m - 1) * ldo + n) * os}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : in)
      if (overlap(outs[i].p, outs[i].len, r.p, r.len)) return NVFP4_ERR_INVALID_VALUE;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i].p, outs[i].len, outs[j].p, outs[j].len))
        return NVFP4_ERR_INVALID_VALUE;
  }
  return status_of(nvfp4::launch_quantize_gemm(x, x_dtype, m, k, ldx, mode, x_codes, x_scales,
                                               x_global, w_codes, w_scales, w_global, n, out,
                                               out_dtype, ldo,
                                               static_cast<hipStream_t>(stream)));
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                     const float* global, int64_t rows, int64_t k, void* out,
                     int out_dtype, int64_t ldo, void* stream) {
  if (!codes || !scales || !global || !out) return NVFP4_ERR_INVALID_VALUE;
  if (rows < 1 || k < 16 || k % 16 != 0 || ldo < k) return NVFP4_ERR_INVALID_VALUE;
  if (rows > kMaxDim || ldo > kMaxDim || rows > kMaxDim / ldo)
    return NVFP4_ERR_INVALID_VALUE;
  if (rows * (k / 16) > (int64_t(1) << 39)) return NVFP4_ERR_INVALID_VALUE;
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  const int64_t os = out_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  if (!aligned(codes, 8) || !aligned(out, 16) || (ldo * os) % 16 != 0 ||
      !aligned(global, 4))
    return NVFP4_ERR_MISALIGNED;
  const int64_t obytes = ((rows - 1) * ldo + k) * os;
  if (overlap(out, obytes, codes, rows * (k / 2)) ||
      overlap(out, obytes, scales, rows * (k / 16)) || overlap(out, obytes, global, 4))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_dequantize(codes, scales, global, rows, k, out,
                                            out_dtype, ldo,
                                            static_cast<hipStream_t>(stream)));
}

int nvfp4_error_stats(const void* x, int x_dtype, int64_t rows, int64_t k,
                      int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                      const float* global, double* stats, void* stream) {
  if (!x || !codes || !scales || !global || !stats) return NVFP4_ERR_INVALID_VALUE;
  if (rows < 1 || k < 16 || k % 16 != 0 || ldx < k) return NVFP4_ERR_INVALID_VALUE;
  if (rows > kMaxDim || ldx > kMaxDim || rows > kMaxDim / ldx)
    return NVFP4_ERR_INVALID_VALUE;
  if (rows * (k / 16) > (int64_t(1) << 39)) return NVFP4_ERR_INVALID_VALUE;
  if (x_dtype != NVFP4_DTYPE_F32 && x_dtype != NVFP4_DTYPE_BF16)
    return NVFP4_ERR_UNSUPPORTED;
  const int64_t es = x_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * es) % 16 != 0 || !aligned(codes, 8) ||
      !aligned(global, 4) || !aligned(stats, 8))
    return NVFP4_ERR_MISALIGNED;
  const int64_t sbytes = rows * 3 * 8;
  if (overlap(stats, sbytes, x, ((rows - 1) * ldx + k) * es) ||
      overlap(stats, sbytes, codes, rows * (k / 2)) ||
      overlap(stats, sbytes, scales, rows * (k / 16)) || overlap(stats, sbytes, global, 4))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_error_stats(x, x_dtype, rows, k, ldx, codes, scales,
                                             global, stats,
                                             static_cast<hipStream_t>(stream)));
}

int fp8_kv_amax_update(const void* x, int x_dtype, int64_t rows, int64_t k,
                       int64_t ldx, float* amax, void* stream) {
  const int st = check_x(x, x_dtype, rows, k, ldx);
  if (st != NVFP4_OK) return st;
  if (!amax) return NVFP4_ERR_INVALID_VALUE;
  if (!aligned(amax, 4)) return NVFP4_ERR_MISALIGNED;
  return status_of(nvfp4::launch_kv_amax_update(x, x_dtype, rows, k, ldx, amax,
                                                static_cast<hipStream_t>(stream)));
}

int fp8_kv_scale_from_amax(const float* amax, float* scale, void* stream) {
  if (!amax || !scale) return NVFP4_ERR_INVALID_VALUE;
  if (!aligned(amax, 4) || !aligned(scale, 4)) return NVFP4_ERR_MISALIGNED;
  return status_of(nvfp4::launch_kv_scale(amax, scale, static_cast<hipStream_t>(stream)));
}

int fp8_kv_cast(const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                const float* scale, uint8_t* out, int64_t ldo, void* stream) {
  const int st = check_x(x, x_dtype, rows, k, ldx);
  if (st != NVFP4_OK) return st;
  if (!scale || !out || ldo < k || ldo > kMaxDim || rows > kMaxDim / ldo)
    return NVFP4_ERR_INVALID_VALUE;
  if (!aligned(scale, 4) || !aligned(out, 16) || ldo % 16 != 0)
    return NVFP4_ERR_MISALIGNED;
  const int64_t es = x_dtype == NVFP4_DTYPE_F32 ? 4 : 2;
  const int64_t obytes = (rows - 1) * ldo + k;
  if (overlap(out, obytes, x, ((rows - 1) * ldx + k) * es) || overlap(out, obytes, scale, 4))
    return NVFP4_ERR_INVALID_VALUE;
  return status_of(nvfp4::launch_kv_cast(x, x_dtype, rows, k, ldx, scale, out, ldo,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
