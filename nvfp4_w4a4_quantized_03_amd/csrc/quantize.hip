// NVFP4 quantisation for gfx950: tensor amax -> FP32 global, block amax ->
// E4M3 scale, E2M1 encode + pack.
//
// Format: the explainer page "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか",
// section 前提1, and the arxiv-wiki page on the same paper, section 접근 방법:
// E2M1 values, one E4M3 scale per 16 elements from the block maximum over 6,
// one FP32 scale per tensor.  Decisions are exact: every quotient is
// compared with the rounding midpoints without error.
//
// Work split: one lane per 16-element block.  A wave streams 64 consecutive
// blocks (2 KiB of bf16), so loads and the 8-byte code stores are fully
// coalesced; the kernel is HBM-bound and keeps VALU work per element small:
//   * block max on the magnitude bits (integer max, two bf16 per op);
//   * block scale in float64 (exact, amortised over 16 elements);
//   * element codes by the gfx950 fp4 conversion (round to nearest even,
//     saturating, sign kept) applied to x * r for two reciprocals r that
//     bracket 1 / (e4m3(s) g) within 2^-18; when both give the same byte the
//     exact quotient lies between them and rounds the same way.  Otherwise
//     (a value within ~2^-18 of a rounding midpoint, about one element in
//     10^5) the lane re-derives its 16 codes with exact float64 compares.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kDtypeF32 = 0;
constexpr int kModeCompute = 0;

// Exact 4-bit code of x under the block's decoded scale times the global,
// S = e4m3(s) g > 0 exact in float64: count the E2M1 midpoints below |x|
// (ties to the even code), then copy the sign bit.
__device__ __forceinline__ unsigned e2m1_exact(float x, double S) {
  const double a = __builtin_fabs(static_cast<double>(x));
  unsigned c = 0;
  if (S > 0.0) {
    // midpoints of 0 .5 1 1.5 2 3 4 6; the tie goes up when the upper code
    // (index i + 1) is even
    const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const double t = mids[i] * S;
      c += (a > t || (a == t && (i & 1))) ? 1u : 0u;
    }
  }
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

// Packs the codes of 8 values into a dword with the gfx950 conversion
// (x * r rounded to nearest even E2M1, saturating, sign kept; byte j holds
// elements 2j (low nibble) and 2j+1).
__device__ __forceinline__ unsigned cvt8(const float* v, float r) {
  unsigned d = 0;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0] * r, v[1] * r, 1.0f, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2] * r, v[3] * r, 1.0f, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4] * r, v[5] * r, 1.0f, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6] * r, v[7] * r, 1.0f, 3);
  return d;
}

// Loads the 16 values of a block as binary32, and the block's max |x| as
// binary32 bits (an integer max of magnitude bits equals the float max).
template <int DTYPE>
__device__ __forceinline__ unsigned load_block(const void* base, float* v);

template <>
__device__ __forceinline__ unsigned load_block<1>(const void* base, float* v) {
  const uint4* p = static_cast<const uint4*>(base);
  const uint4 a = p[0], b = p[1];
  const unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  unsigned mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    const unsigned mag = w[i] & 0x7FFF7FFFu;
    const unsigned lo = mag & 0xFFFFu, hi = mag >> 16;
    mx = max(mx, max(lo, hi));
  }
  return mx << 16;
}

template <>
__device__ __forceinline__ unsigned load_block<0>(const void* base, float* v) {
  const float4* p = static_cast<const float4*>(base);
  unsigned mx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q = p[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return mx;
}

template <int DTYPE>
__global__ void __launch_bounds__(256)
quantize_kernel(const uint8_t* __restrict__ x, int64_t nblocks, int64_t kb,
                int64_t ldx_bytes, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales, const float* __restrict__ global) {
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const float g = *global;
  const double gd = static_cast<double>(g);

  // block b = (row, column block); contiguous rows need no division
  const uint8_t* src;
  if (ldx_bytes == kb * 16 * kElemBytes) {
    src = x + b * (16 * kElemBytes);
  } else {
    const int64_t row = b / kb;
    src = x + row * ldx_bytes + (b - row * kb) * (16 * kElemBytes);
  }
  float v[16];
  const float m = __uint_as_float(load_block<DTYPE>(src, v));

  // block scale: RNE_SAT_E4M3(m / (6 g)), exact; 0 if m == 0 or g == 0
  unsigned s = 0;
  const double den6 = 6.0 * gd;            // exact
  if (m > 0.0f && g > 0.0f) {
    const double md = static_cast<double>(m);
    s = e4m3_settle(e4m3_candidate(md / den6), md, den6);
  }

  // element codes: bracketed fast path, exact fallback
  const double S = e4m3_value(s) * gd;     // exact
  bool exact = false;
  float r_lo = 0.0f, r_hi = 0.0f;
  if (S > 0.0) {
    const double r = 1.0 / S;
    // outside this range binary32 reciprocals lose the bracketing
    exact = !(r >= 0x1p-100 && r <= 0x1p100);
    r_lo = static_cast<float>(r * (1.0 - 0x1p-18));
    r_hi = static_cast<float>(r * (1.0 + 0x1p-18));
  }
  uint2 c;
  c.x = cvt8(v, r_lo);
  c.y = cvt8(v + 8, r_lo);
  const unsigned h0 = cvt8(v, r_hi), h1 = cvt8(v + 8, r_hi);
  exact = exact || c.x != h0 || c.y != h1;
  if (exact) {
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_exact(v[i], S) << (4 * (i & 7));
    c.x = w[0];
    c.y = w[1];
  }
  reinterpret_cast<uint2*>(codes)[b] = c;
  scales[b] = static_cast<uint8_t>(s);
}

// ---- self-calibrated global: amax over the tensor, then g = amax / 2688 --

__global__ void amax_init_kernel(unsigned* bits) { *bits = 0u; }

template <int DTYPE>
__global__ void __launch_bounds__(256)
amax_kernel(const uint8_t* __restrict__ x, int64_t nblocks, int64_t kb,
            int64_t ldx_bytes, unsigned* __restrict__ out_bits) {
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const bool contiguous = ldx_bytes == kb * 16 * kElemBytes;
  unsigned mx = 0;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       b < nblocks; b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const uint8_t* src;
    if (contiguous) {
      src = x + b * (16 * kElemBytes);
    } else {
      const int64_t row = b / kb;
      src = x + row * ldx_bytes + (b - row * kb) * (16 * kElemBytes);
    }
    float v[16];
    mx = max(mx, load_block<DTYPE>(src, v));
  }
  // wave reduction, then one atomic per workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
  __shared__ unsigned part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = part[0];
    for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) t = max(t, part[i]);
    atomicMax(out_bits, t);
  }
}

// g = RNE_fp32(amax / 2688).  The float64 quotient is rounded once more to
// binary32; A / 2688 is either exact in binary32 or far (relative 2^-30)
// from every binary32 rounding boundary, so this is one correct rounding.
__global__ void amax_finalize_kernel(float* global) {
  const float a = __uint_as_float(*reinterpret_cast<unsigned*>(global));
  *global = static_cast<float>(static_cast<double>(a) / 2688.0);
}

}  // namespace

hipError_t launch_quantize(const void* x, int x_dtype, int64_t rows,
                           int64_t k, int64_t ldx, uint8_t* codes,
                           uint8_t* scales, float* global, int mode,
                           hipStream_t stream) {
  const int64_t kb = k / 16;
  const int64_t nblocks = rows * kb;
  const int64_t esize = x_dtype == kDtypeF32 ? 4 : 2;
  const int64_t ldx_bytes = ldx * esize;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (mode == kModeCompute) {
    unsigned* bits = reinterpret_cast<unsigned*>(global);
    amax_init_kernel<<<1, 1, 0, stream>>>(bits);
    const int64_t want = (nblocks + 255) / 256;
    const unsigned grid = static_cast<unsigned>(want < 2048 ? want : 2048);
    if (x_dtype == kDtypeF32)
      amax_kernel<0><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes, bits);
    else
      amax_kernel<1><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes, bits);
    amax_finalize_kernel<<<1, 1, 0, stream>>>(global);
  }
  const unsigned grid = static_cast<unsigned>((nblocks + 255) / 256);
  if (x_dtype == kDtypeF32)
    quantize_kernel<0><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes,
                                                 codes, scales, global);
  else
    quantize_kernel<1><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes,
                                                 codes, scales, global);
  return hipGetLastError();
}

}  // namespace nvfp4
