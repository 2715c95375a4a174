// Internal declarations shared by the C-ABI front end (api.cpp) and the HIP
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace nvfp4 {

// Quantisation (quantize.hip).  Arguments are already validated.
hipError_t launch_quantize(const void* x, int x_dtype, int64_t rows,
                           int64_t k, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, float* global, int mode,
                           hipStream_t stream);

// Fused-group scale harmonisation (harmonize.hip).
constexpr int kMaxModules = 64;
hipError_t launch_harmonize(uint8_t* scales, int64_t k,
                            const int64_t* row_offsets, int n_modules,
                            const float* module_globals,
                            float* shared_global, hipStream_t stream);

// W4A4 GEMM (gemm.hip).
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_global, int64_t m,
                       const uint8_t* b_codes, const uint8_t* b_scales,
                       const float* b_global, int64_t n, int64_t k,
                       void* out, int out_dtype, int64_t ldo, int epilogue,
                       hipStream_t stream);

// Streaming GEMM for shapes with one operand of at most 64 rows, whole
// stages of K (k % 512 == 0 for up to 32 rows, k % 256 == 0 for 33-64) and
// k <= 2^22 (gemm_stream.hip); arguments as launch_gemm.
bool gemm_stream_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_stream(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_global, int64_t m,
                              const uint8_t* b_codes, const uint8_t* b_scales,
                              const float* b_global, int64_t n, int64_t k,
                              void* out, int out_dtype, int64_t ldo, int epilogue,
                              hipStream_t stream);

// The same fused call on the streaming GEMM's tiles, for the shapes where
// w4a4_gemm uses them (gemm_stream_fits(m, n, k)).
hipError_t launch_quantize_gemm_stream(const void* x, int x_dtype, int64_t m, int64_t k,
                                       int64_t ldx, int mode, uint8_t* x_codes,
                                       uint8_t* x_scales, float* x_global,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* w_global, int64_t n, void* out,
                                       int out_dtype, int64_t ldo, hipStream_t stream);

// Small-M (m <= 64) activation quantise + W4A4 GEMM in one cooperative
// launch (gemm.hip); k % 128 == 0 and 16-byte aligned code and scale arrays
// are checked by the caller.
constexpr int64_t kMaxFusedRows = 64;
hipError_t launch_quantize_gemm(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                                int mode, uint8_t* x_codes, uint8_t* x_scales,
                                float* x_global, const uint8_t* w_codes,
                                const uint8_t* w_scales, const float* w_global, int64_t n,
                                void* out, int out_dtype, int64_t ldo, hipStream_t stream);

// The gate pair on the streaming GEMM (gemm_stream.hip): S = the
// activations, L = the fused b|a weight of n <= 64 rows, k a whole number
// of its stages (k % 512 for n <= 32, k % 256 otherwise) and k <= 2^22.
bool gdn_stream_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gdn_stream(const uint8_t* x_codes, const uint8_t* x_scales,
                             const float* x_global, int64_t m, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_global, int64_t n_beta,
                             int64_t n_alpha, int64_t k, const float* a_log,
                             const float* dt_bias, float* beta_out, int64_t ld_beta,
                             float* alpha_out, int64_t ld_alpha, hipStream_t stream);

// Gate pair of a fused b|a projection (gemm.hip); k % 128 == 0, 16-byte
// aligned scale arrays and n_beta + n_alpha <= 256 are checked by the caller.
constexpr int64_t kMaxGateCols = 256;
hipError_t launch_gdn_gates(const uint8_t* x_codes, const uint8_t* x_scales,
                            const float* x_global, int64_t m,
                            const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_global, int64_t n_beta, int64_t n_alpha,
                            int64_t k, const float* a_log, const float* dt_bias,
                            float* beta_out, int64_t ld_beta, float* alpha_out,
                            int64_t ld_alpha, hipStream_t stream);

// Dequantisation and error statistics (dequantize.hip).
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales,
                             const float* global, int64_t rows, int64_t k,
                             void* out, int out_dtype, int64_t ldo,
                             hipStream_t stream);
hipError_t launch_error_stats(const void* x, int x_dtype, int64_t rows, int64_t k,
                              int64_t ldx, const uint8_t* codes,
                              const uint8_t* scales, const float* global,
                              double* stats, hipStream_t stream);

// FP8 KV cache with a static per-tensor scale (fp8kv.hip).
hipError_t launch_kv_amax_update(const void* x, int x_dtype, int64_t rows, int64_t k,
                                 int64_t ldx, float* amax, hipStream_t stream);
hipError_t launch_kv_scale(const float* amax, float* scale, hipStream_t stream);
hipError_t launch_kv_cast(const void* x, int x_dtype, int64_t rows, int64_t k,
                          int64_t ldx, const float* scale, uint8_t* out,
                          int64_t ldo, hipStream_t stream);

}  // namespace nvfp4
