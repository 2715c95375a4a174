// Device helpers shared by the W4A4 GEMM kernels (gemm.hip,
// gemm_stream.hip): output and epilogue selectors, the exact NVFP4 -> fp16
// decode of 8 codes, bf16 rounding and the gate epilogues.
//
// Decode: e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16 (normal from 2^-14, 11-bit
// significand).  Gates: the explainer page "論文解説: Gated DeltaNet はなぜ4bit
// 量子化に耐えるのか", section 前提2 (alpha through softplus and exp, beta
// through a sigmoid).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace nvfp4 {
namespace {

constexpr int kOutF32 = 0;
constexpr int kEpiNone = 0;
constexpr int kEpiAlpha = 1;
constexpr int kEpiBeta = 2;
constexpr int kEpiGdn = 3;   // gate pair of a fused b|a projection (w4a4_gemm_gdn_gates)

// Arguments of the gate-pair epilogue: columns [0, n_beta) of the product
// give beta (stored to `out`), the others alpha with per-column A_log and
// dt_bias (stored to out2 at column col - n_beta).
struct EpiArgs {
  const float* a_log;
  const float* dt_bias;
  int64_t n_beta;
  float* out2;
  int64_t ldo2;
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));


// Decode 8 codes (one dword, element 2j in the low nibble of byte j) with
// one fp16 block scale into 8 exact fp16 values.
__device__ __forceinline__ half8_t decode8(unsigned codes, half2_t sc) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  const half2_t q0 = p0 * sc, q1 = p1 * sc, q2 = p2 * sc, q3 = p3 * sc;
  half8_t r;
  r[0] = q0[0]; r[1] = q0[1]; r[2] = q1[0]; r[3] = q1[1];
  r[4] = q2[0]; r[5] = q2[1]; r[6] = q3[0]; r[7] = q3[1];
  return r;
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return static_cast<unsigned short>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// e^x from the hardware base-2 exponential (v_exp_f32, about 1 ulp):
// 2^(x log2 e); the rounding of x log2 e adds |x| 2^-24 relative error.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float exp_hw(float x) {
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// The gate pair of a fused b|a projection (the explainer page, section
// 前提2): beta = sigmoid(b) and alpha = exp(-exp(A_log) softplus(a + dt_bias))
// per head, softplus(x) = max(x, 0) + log(1 + e^-|x|).
__device__ __forceinline__ float gdn_beta(float y) {
  return __builtin_amdgcn_rcpf(1.0f + exp_hw(-y));
}
__device__ __forceinline__ float gdn_alpha(float y, float a_log, float dt_bias) {
  const float x = y + dt_bias;
  const float sp = fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + exp_hw(-fabsf(x))) * kLn2;
  return exp_hw(-exp_hw(a_log) * sp);
}

template <int EPI>
__device__ __forceinline__ float epilogue(float y) {
  if constexpr (EPI == kEpiAlpha) {
    // exp(-softplus(y)) = exp(-log(1 + e^y)) = 1 / (1 + e^y); the short form
    // keeps the epilogue small enough to unroll over the accumulator tiles
    // (which must stay in registers).  e^y overflowing to inf gives 0.
    return 1.0f / (1.0f + expf(y));
  } else if constexpr (EPI == kEpiBeta) {
    return 1.0f / (1.0f + expf(-y));
  } else {
    return y;
  }
}


// Buffer loads of 16 or 4 bytes per lane straight into LDS, at the
// wave-uniform `lds` plus lane * size; the source is the resource base +
// voff + soff.  Buffer (not FLAT-encoded global) loads are used so that the
// compiler can keep counting LDS reads in order while these are in flight:
// a pending FLAT load may touch LDS, which makes every later LDS-read wait a
// full drain.
__device__ __forceinline__ void lds_buf16(__amdgpu_buffer_rsrc_t rsrc, void* lds,
                                          unsigned voff, unsigned soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

__device__ __forceinline__ void lds_buf4(__amdgpu_buffer_rsrc_t rsrc, void* lds,
                                         unsigned voff, unsigned soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
#endif
}

// s_waitcnt immediate that waits until at most `keep` vector-memory ops are
// outstanding, without waiting on expcnt/lgkmcnt (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int kVmcntKeepOf(int keep) {
  return (keep & 0xF) | 0x70 | 0xF00 | ((keep >> 4) << 14);
}

// Workgroup barrier without the memory fence that __syncthreads() implies
// (that fence waits for every outstanding load, including the LDS fill of a
// later stage that is meant to stay in flight).  The wait for the stage
// that must be resident is issued explicitly before this; the empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace nvfp4
