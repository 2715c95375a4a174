/*
 * nvfp4_w4a4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 hot path.
 *
 * The format and the operations follow two pages about the paper
 * "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the
 * Recurrent Half of a Hybrid 27B LLM":
 *   [P1] its arxiv-wiki summary page (sections "접근 방법" = approach,
 *        "개발자 관점" = developer view),
 *   [P3] the ta-paperlens explainer "論文解説: Gated DeltaNet はなぜ4bit量子化に
 *        耐えるのか" (sections "前提1" = what 4-bit rounding is, "前提2" = what
 *        Gated DeltaNet computes).
 *
 * NVFP4 tensor ([P3] 前提1, [P1] 접근 방법): 4-bit E2M1 values (1 sign,
 * 2 exponent, 1 mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), one
 * OCP E4M3 scale per 16 consecutive elements (set from the block maximum
 * over 6), and one FP32 scale per tensor.  W4A4: both GEMM operands are in
 * this format.
 *
 * Layouts (all row-major, no padding, no swizzle):
 *   codes : uint8 [rows][k/2]; element 2j in the low nibble of byte j,
 *           element 2j+1 in the high nibble; bit 3 of a nibble is the sign.
 *   scales: uint8 [rows][k/16]; raw OCP E4M3 bytes (never negative, never
 *           the NaN code 0x7F).
 *   global: one float on the device, the decode scale g: the value of an
 *           element is e2m1(code) * e4m3(scale) * g.  Computed from a tensor
 *           as g = fp32(max|x| / 2688), 2688 = 6 * 448.
 *   Blocks of 16 run along k, the reduction axis of the GEMM.
 *
 * Conventions for every call:
 *   - All buffers are device memory owned by the caller; the library
 *     allocates nothing.  Its only state between calls is a per-device
 *     cache of the co-resident workgroup count of the fused call's kernels
 *     (w4a4_gemm_quantize_a).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls validate
 *     their arguments on the host, enqueue kernels and return without
 *     synchronising.  A kernel fault is reported by the next synchronising
 *     HIP call of the caller.
 *   - A nonzero return is an nvfp4_status; nothing was enqueued unless the
 *     status is NVFP4_ERR_LAUNCH.  nvfp4_status_string() names it.
 *   - Inputs must be finite; that is a precondition and is not checked.
 *   - Calls that overlap on one stream are ordered by it; buffers shared by
 *     calls on different streams need the caller's own ordering.
 */
#ifndef NVFP4_W4A4_H
#define NVFP4_W4A4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_VALUE = 1, /* null pointer, bad size, k % 16 != 0, ... */
    NVFP4_ERR_UNSUPPORTED = 2,   /* unknown dtype / mode / epilogue, or a    */
                                 /* shape outside the call's kernels       */
    NVFP4_ERR_MISALIGNED = 3,    /* a pointer or stride breaks the alignment  */
    NVFP4_ERR_LAUNCH = 4         /* the HIP runtime refused a launch          */
} nvfp4_status;

typedef enum {
    NVFP4_DTYPE_F32 = 0,
    NVFP4_DTYPE_BF16 = 1
} nvfp4_dtype;

typedef enum {
    NVFP4_GLOBAL_COMPUTE = 0, /* g = fp32(max|x| / 2688), written to *global */
    NVFP4_GLOBAL_GIVEN = 1    /* *global is read as a calibrated static g    */
} nvfp4_global_mode;

typedef enum {
    W4A4_EPI_NONE = 0,  /* y                                   */
    W4A4_EPI_ALPHA = 1, /* exp(-softplus(y)): decay gate        */
    W4A4_EPI_BETA = 2   /* sigmoid(y): write-strength gate      */
} w4a4_epilogue;

/*
 * nvfp4_quantize -- NVFP4 quantisation of a [rows][k] tensor.
 * Defined by [P3] 前提1 and [P1] 접근 방법 (16-element blocks, E4M3 block
 * scale from block max / 6, E2M1 values, FP32 per-tensor scale).
 *
 *   x          device, [rows][ldx] elements of x_dtype (F32 or BF16); only
 *              the first k of each row are read.  16-byte aligned; ldx*size
 *              a multiple of 16 bytes.
 *   rows, k    rows >= 1, k >= 16, k % 16 == 0.
 *   ldx        row stride in elements, ldx >= k.
 *   codes      device, out, [rows][k/2] bytes, 8-byte aligned.
 *   scales     device, out, [rows][k/16] bytes.
 *   global     device, one float: written in COMPUTE mode (the tensor's g),
 *              read in GIVEN mode (must be finite and >= 0).
 *   mode       nvfp4_global_mode.
 *
 * Result, per 16-element block with maximum magnitude m: scale
 * s = E4M3(m / (6 g)) and codes c = sign(x) | E2M1(|x| / (e4m3(s) g)), each
 * quotient exact and rounded once to nearest, ties to the even code,
 * saturating at 448 and 6; s = 0 and magnitude 0 when m = 0 or g = 0.
 * Bit-exact with this definition on every finite input.
 * COMPUTE mode enqueues four kernels (init, amax, finalize, quantize);
 * GIVEN mode one.  x must not overlap the outputs.
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t k,
                   int64_t ldx, uint8_t* codes, uint8_t* scales,
                   float* global, int mode, void* stream);

/*
 * nvfp4_harmonize_group -- rewrite the modules of a fused-GEMM group to one
 * shared global scale, folding each module's ratio into its block scales.
 * Defined by [P1] 접근 방법 and 개발자 관점 (the fix for per-module
 * calibrated checkpoints served by kernels that fuse qkv|z and b|a into one
 * GEMM) and the abstract on the paper's listing page.
 *
 *   scales        device, in/out, [n_total][k/16] E4M3 bytes of the fused
 *                 weight, 16-byte aligned (else MISALIGNED); module i owns
 *                 rows [row_offsets[i], row_offsets[i+1]).  The codes are
 *                 not touched.
 *   k             k >= 16, k % 16 == 0.
 *   row_offsets   HOST array of n_modules + 1 increasing values,
 *                 row_offsets[0] == 0, row_offsets[n_modules] = n_total.
 *   n_modules     1 .. 64.
 *   module_globals device, [n_modules] floats g_i (finite, >= 0).
 *   shared_global device, out, one float: g* = max_i g_i.  Must not
 *                 overlap module_globals or scales.
 *
 * Result: every scale s of module i becomes E4M3(e4m3(s) * g_i / g*),
 * exact quotient rounded once (ties to even); rows of modules with
 * g_i == g* are left unchanged.  Afterwards e2m1 * e4m3(s') * g* equals the
 * module's own dequantised weight up to that one rounding of the scale.
 * Calling it twice on the same buffer re-folds the scales (not idempotent).
 */
int nvfp4_harmonize_group(uint8_t* scales, int64_t k,
                          const int64_t* row_offsets, int n_modules,
                          const float* module_globals, float* shared_global,
                          void* stream);

/*
 * w4a4_gemm -- Y = (g_a g_b) * A_hat B_hat^T on NVFP4 operands, with an
 * optional gate epilogue.  The W4A4 linear of [P3] 前提1 / [P1] 접근 방법;
 * the gates are those of [P3] 前提2 (alpha through softplus and exp, beta
 * through a sigmoid), in the form alpha = exp(-softplus(y)),
 * beta = sigmoid(y).
 *
 *   a_codes, a_scales, a_global  activations A [m][k] in the layout above
 *                                (codes and scales 16-byte aligned, else
 *                                MISALIGNED).
 *   b_codes, b_scales, b_global  weights B [n][k] (K-major, the same
 *                                layout and alignment).
 *   m, n, k      m, n >= 1, k >= 16, k % 16 == 0.  k % 128 == 0 takes the
 *                whole-stage kernels; other k (rows whose code and scale
 *                bytes do not fill 16-byte pieces) a kernel that guards
 *                each piece.
 *   out          device, [m][ldo] of out_dtype (F32 or BF16), ldo >= n;
 *                4-byte aligned.  Must not overlap the inputs.
 *   epilogue     w4a4_epilogue, applied in fp32 before the store.
 *
 * Every A_hat[i][k] = e2m1 * e4m3 and B_hat[j][k] is decoded exactly (the
 * products are exact in fp16); products are accumulated in fp32; the
 * global factors multiply the fp32 sum; BF16 output is rounded to nearest
 * even from that fp32 value.
 */
int w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
              const float* a_global, int64_t m,
              const uint8_t* b_codes, const uint8_t* b_scales,
              const float* b_global, int64_t n, int64_t k,
              void* out, int out_dtype, int64_t ldo, int epilogue,
              void* stream);

/*
 * w4a4_gemm_gdn_gates -- the gate pair of one Gated DeltaNet layer from
 * its fused b|a gate projection ([P1] 개발자 관점 names the b/a fused
 * group; [P3] 前提2: b through a sigmoid, a through softplus and an
 * exponential in log space):
 *   y      = (g_x g_w) * X_hat W_hat^T, W = [W_b ; W_a] (n_beta + n_alpha
 *            rows, one harmonised global; see nvfp4_harmonize_group),
 *   beta   = sigmoid(y[:, j]),                      j <  n_beta,
 *   alpha  = exp(-exp(A_log[i]) * softplus(y[:, n_beta + i] + dt_bias[i])).
 *
 *   x_codes, x_scales, x_global  activations X [m][k] (NVFP4, as above).
 *   w_codes, w_scales, w_global  fused weight [n_beta + n_alpha][k].
 *   n_beta, n_alpha  >= 0, 1 <= n_beta + n_alpha <= 256 (else
 *                UNSUPPORTED); k % 128 == 0 (else UNSUPPORTED); codes and
 *                scale arrays 16-byte aligned (else MISALIGNED).
 *   a_log, dt_bias  device, [n_alpha] floats (may be NULL if n_alpha == 0).
 *   beta_out     device, out, [m][ld_beta] floats, ld_beta >= n_beta (NULL
 *                allowed if n_beta == 0).
 *   alpha_out    device, out, [m][ld_alpha] floats, ld_alpha >= n_alpha
 *                (NULL allowed if n_alpha == 0).  Outputs must not overlap
 *                each other or the inputs.
 *
 * y is computed as in w4a4_gemm (exact decode, fp32 accumulation, global
 * factors on the fp32 sum); the gates in fp32.
 */
int w4a4_gemm_gdn_gates(const uint8_t* x_codes, const uint8_t* x_scales,
                        const float* x_global, int64_t m,
                        const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* w_global, int64_t n_beta, int64_t n_alpha,
                        int64_t k, const float* a_log, const float* dt_bias,
                        float* beta_out, int64_t ld_beta, float* alpha_out,
                        int64_t ld_alpha, void* stream);

/*
 * w4a4_gemm_quantize_a -- small-M activation quantisation and W4A4 GEMM in
 * one launch: nvfp4_quantize of X, then w4a4_gemm of the result with the
 * weights (no epilogue).  For decode batches, where [P1] 한계 (limitations)
 * puts a 2-4 % loss on the activation quantisation.
 *
 *   x, x_dtype, m, k, ldx  activations X [m][ldx] as for nvfp4_quantize;
 *                1 <= m <= 64 and k % 128 == 0 (else UNSUPPORTED).
 *   x_codes, x_scales, x_global, mode  out (x_global read in GIVEN mode):
 *                the NVFP4 form of X, bit-identical to nvfp4_quantize with
 *                the same mode; codes and scales 16-byte aligned.
 *   w_codes, w_scales, w_global  weights W [n][k] (NVFP4; codes and scales
 *                16-byte aligned), n >= 1.
 *   out, out_dtype, ldo  Y [m][ldo] of F32 or BF16, ldo >= n, 4-byte
 *                aligned.  Equal bit for bit to w4a4_gemm(x_codes, ..., W,
 *                W4A4_EPI_NONE) on the same device.
 * Outputs must not overlap each other or the inputs.
 *
 * One cooperative launch: the workgroups that own blocks of X quantise them
 * (with COMPUTE, each of them first takes max |x| over all of X), a
 * grid-wide barrier follows, then every workgroup computes GEMM tiles.  The
 * grid is capped at the co-resident workgroup count of the device; larger
 * shapes loop inside the kernel.  NVFP4_ERR_LAUNCH if the runtime refuses
 * the cooperative launch.  Calls on different streams that share these
 * buffers must be ordered by the caller.
 * Cost: on MI355X a cooperative launch and its grid barrier cost more than
 * the launches they save, so at decode sizes this call is slower than
 * nvfp4_quantize followed by w4a4_gemm; it serves callers that need the
 * whole step in one launch.
 */
int w4a4_gemm_quantize_a(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                         uint8_t* x_codes, uint8_t* x_scales, float* x_global, int mode,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         const float* w_global, int64_t n, void* out, int out_dtype,
                         int64_t ldo, void* stream);

/*
 * nvfp4_dequantize -- values of an NVFP4 tensor, the inverse map used for
 * fake quantisation (quantise, then dequantise) in the mechanism study of
 * [P1] 접근 방법; element value sign * E2M1 * E4M3 * g per [P3] 前提1.
 *
 *   codes, scales, global  a [rows][k] NVFP4 tensor in the layout above
 *                          (codes 8-byte aligned; global one float).
 *   rows, k      rows >= 1, k >= 16, k % 16 == 0.
 *   out          device, out, [rows][ldo] of out_dtype (F32 or BF16),
 *                ldo >= k; 16-byte aligned, ldo*size a multiple of 16.
 *                Must not overlap the inputs.
 *
 * Result: each output is the exact value rounded once to nearest even
 * binary32 or bfloat16 (e2m1 * e4m3 is exact; times g it has <= 30
 * significant bits, so no double rounding occurs).
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                     const float* global, int64_t rows, int64_t k, void* out,
                     int out_dtype, int64_t ldo, void* stream);

/*
 * nvfp4_error_stats -- per-row statistics of a tensor and of its NVFP4
 * quantisation, behind the A4 / W4 error percentages and the max/RMS input
 * statistic of [P1] 접근 방법 (Table 2) and the block bound of [P3] 前提1.
 *
 *   x            device, [rows][ldx] of x_dtype (F32 or BF16), the tensor
 *                that was quantised (same alignment rules as
 *                nvfp4_quantize).
 *   codes, scales, global  its NVFP4 form (codes 8-byte aligned).
 *   stats        device, out, [rows][3] doubles, 8-byte aligned:
 *                sum x^2, sum (x - x_hat)^2, max |x| with x_hat the exact
 *                dequantised value; sums in float64 in an unspecified
 *                order.  Must not overlap the inputs.
 *
 * Relative error of a row or tensor = sqrt(sum col 1 / sum col 0);
 * max/RMS of a row = col 2 / sqrt(col 0 / k).
 */
int nvfp4_error_stats(const void* x, int x_dtype, int64_t rows, int64_t k,
                      int64_t ldx, const uint8_t* codes, const uint8_t* scales,
                      const float* global, double* stats, void* stream);

/*
 * FP8 KV cache with a static per-tensor scale ([P1] 접근 방법 and the
 * abstract on the paper's listing page: store the KV cache in FP8 and ship
 * calibrated per-tensor scales with the checkpoint).  OCP E4M3 codes; the
 * scale is a decode factor s = fp32(amax / 448) over the calibration data;
 * a stored code is sign(x) | E4M3(|x| / s), the exact quotient rounded once
 * to nearest, ties to the even code, saturating at 448 (magnitude 0 when
 * s == 0).  Decoded value: e4m3(code) * s.
 *
 * fp8_kv_amax_update -- *amax = max(*amax, max |x|) over a calibration
 *   tensor x [rows][ldx] (same rules as nvfp4_quantize's x).  *amax is a
 *   device float the caller sets to 0 before the first call; calls on one
 *   amax accumulate.
 * fp8_kv_scale_from_amax -- *scale = fp32(*amax / 448) (device floats).
 * fp8_kv_cast -- out [rows][ldo] bytes (16-byte aligned, ldo >= k,
 *   ldo % 16 == 0) = codes of x [rows][ldx] under the device scale *scale
 *   (finite, >= 0).  out must not overlap x or the scale.
 */
int fp8_kv_amax_update(const void* x, int x_dtype, int64_t rows, int64_t k,
                       int64_t ldx, float* amax, void* stream);
int fp8_kv_scale_from_amax(const float* amax, float* scale, void* stream);
int fp8_kv_cast(const void* x, int x_dtype, int64_t rows, int64_t k, int64_t ldx,
                const float* scale, uint8_t* out, int64_t ldo, void* stream);

/* Static text for a status code (never NULL). */
const char* nvfp4_status_string(int status);

/* ABI version of this header: 3 (1 plus w4a4_gemm_gdn_gates, nvfp4_dequantize,
   nvfp4_error_stats and the fp8_kv_* calls in 2, plus w4a4_gemm_quantize_a
   in 3). */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A4_H */
