// FP8 (OCP E4M3) KV-cache storage with a static per-tensor scale, for gfx950.
//
// The arxiv-wiki page on "Why Gated DeltaNet Survives 4-Bit Quantization"
// (section 접근 방법) and the abstract on the paper's listing page store the
// KV cache in FP8 with a calibrated static per-tensor scale shipped with the
// checkpoint.  Here the scale is a decode factor s = RNE_fp32(amax / 448)
// over the calibration data (amax kept as a running maximum across calls),
// and a stored code is sign(x) | RNE_SAT_E4M3(|x| / s): the exact quotient
// rounded once, ties to the even code, saturating at 448; magnitude 0 when
// s = 0.
//
// Cast: one lane per 16 consecutive elements (a wave covers 2 KiB of bf16;
// 16 code bytes per lane).  Each code comes from the gfx950 fp32 -> E4M3
// conversion of |x| r for two reciprocals bracketing 1 / s within 2^-18;
// equal results prove the exact quotient rounds the same way, otherwise
// that element is settled exactly in float64 (mid * s is exact there).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kDtypeF32 = 0;

template <int DTYPE>
__device__ __forceinline__ void load16(const uint8_t* src, float* v) {
  if constexpr (DTYPE == kDtypeF32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(src)[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 t = reinterpret_cast<const uint4*>(src)[q];
      const unsigned w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
}

// Source of 16-element group b; `flat` (rows stored back to back) skips the
// 64-bit division by the groups per row.
template <int DTYPE>
__device__ __forceinline__ const uint8_t* group_src(const uint8_t* x, int64_t b,
                                                    int64_t kg, int64_t ldx_bytes,
                                                    bool flat) {
  constexpr int64_t kBytes = 16 * (DTYPE == kDtypeF32 ? 4 : 2);
  if (flat) return x + b * kBytes;
  const int64_t row = b / kg;
  return x + row * ldx_bytes + (b - row * kg) * kBytes;
}

// Running maximum of |x| into *amax_bits (non-negative binary32 values
// order like their bit patterns).  512-lane workgroups (at most 512 of
// them): twice the waves of 256-lane ones for the same number of atomics,
// which a cold read needs (as for the quantiser's amax pass).
constexpr int kKvAmaxThreads = 512;
template <int DTYPE>
__global__ void __launch_bounds__(kKvAmaxThreads)
kv_amax_kernel(const uint8_t* __restrict__ x, int64_t ngroups, int64_t kg,
               int64_t ldx_bytes, unsigned* __restrict__ amax_bits) {
  const bool flat = ldx_bytes == kg * 16 * (DTYPE == kDtypeF32 ? 4 : 2);
  unsigned mx = 0u;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       b < ngroups; b += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    float v[16];
    load16<DTYPE>(group_src<DTYPE>(x, b, kg, ldx_bytes, flat), v);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
  __shared__ unsigned part[kKvAmaxThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = part[0];
    for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) t = max(t, part[i]);
    atomicMax(amax_bits, t);
  }
}

// s = RNE_fp32(amax / 448): the float64 quotient rounded to binary32 is one
// correct rounding (amax / (7 * 2^6) is exact or a repeating fraction far
// from every binary32 rounding boundary).
__global__ void kv_scale_kernel(const float* amax, float* scale) {
  *scale = static_cast<float>(static_cast<double>(*amax) / 448.0);
}

// Code magnitude of q = |x| / s with the bracketed hardware conversion of
// |x| r_lo and |x| r_hi (inputs clamped to 448, where the hardware would
// give NaN above 464); disagreement -> exact float64 settle.
__device__ __forceinline__ unsigned kv_code(float ax, float r_lo, float r_hi, double s) {
  const float lo = fminf(ax * r_lo, 448.0f), hi = fminf(ax * r_hi, 448.0f);
  const unsigned pk = static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false));
  const unsigned c = pk & 0xFFu;
  if (c == ((pk >> 8) & 0xFFu)) return c;
  return e4m3_settle(c, static_cast<double>(ax), s);
}

// Codes of one 16-element group, stored as one non-temporal 16-byte piece
// (the codes are a stream; a wave's stores cover 1 KiB).  `normal`: s within
// [2^-100, 2^100], where the bracketed conversion applies; otherwise every
// code is settled in float64 (or is 0 when s == 0).  Both flags are uniform,
// so the per-element work has no branch on them.
template <int DTYPE>
__device__ __forceinline__ void kv_cast_group(const uint8_t* src, uint8_t* dst, bool zero,
                                              bool normal, float r_lo, float r_hi,
                                              double sd) {
  float v[16];
  load16<DTYPE>(src, v);
  unsigned w[4] = {0u, 0u, 0u, 0u};
  if (normal) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const unsigned c = kv_code(__builtin_fabsf(v[i]), r_lo, r_hi, sd) |
                         ((__float_as_uint(v[i]) >> 24) & 0x80u);
      w[i >> 2] |= c << (8 * (i & 3));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double ax = static_cast<double>(__builtin_fabsf(v[i]));
      const unsigned m = zero ? 0u : e4m3_settle(e4m3_candidate(ax / sd), ax, sd);
      const unsigned c = m | ((__float_as_uint(v[i]) >> 24) & 0x80u);
      w[i >> 2] |= c << (8 * (i & 3));
    }
  }
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 o = {w[0], w[1], w[2], w[3]};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
}

// One 16-element group per lane.  A grid that covers every group of a flat
// (rows back to back) tensor, the launcher's normal case, takes a
// straight-line body; the grid-stride loop serves strided tensors and grids
// capped at the launch limit.
template <int DTYPE>
__global__ void __launch_bounds__(256)
kv_cast_kernel(const uint8_t* __restrict__ x, int64_t ngroups, int64_t kg,
               int64_t ldx_bytes, const float* __restrict__ scale,
               uint8_t* __restrict__ out, int64_t ldo) {
  constexpr int64_t kBytes = 16 * (DTYPE == kDtypeF32 ? 4 : 2);
  const float s = *scale;
  const double sd = static_cast<double>(s);
  const bool zero = !(s > 0.0f);
  const bool normal = s >= 0x1p-100f && s <= 0x1p100f;
  float r_lo = 0.0f, r_hi = 0.0f;
  if (normal) {
    const float r = __builtin_amdgcn_rcpf(s);   // within 2^-22 of 1 / s
    r_lo = r * (1.0f - 0x1p-18f);
    r_hi = r * (1.0f + 0x1p-18f);
  }
  const bool flat = ldx_bytes == kg * kBytes && ldo == kg * 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (flat && stride >= ngroups) {
    if (b0 < ngroups)
      kv_cast_group<DTYPE>(x + b0 * kBytes, out + b0 * 16, zero, normal, r_lo, r_hi, sd);
    return;
  }
  for (int64_t b = b0; b < ngroups; b += stride) {
    const int64_t row = b / kg;
    kv_cast_group<DTYPE>(x + row * ldx_bytes + (b - row * kg) * kBytes,
                         out + row * ldo + (b - row * kg) * 16, zero, normal, r_lo, r_hi, sd);
  }
}

unsigned grid_for(int64_t groups) {
  const int64_t want = (groups + 255) / 256;
  return static_cast<unsigned>(want < 0x7FFFFFFF ? want : 0x7FFFFFFF);
}

}  // namespace

hipError_t launch_kv_amax_update(const void* x, int x_dtype, int64_t rows, int64_t k,
                                 int64_t ldx, float* amax, hipStream_t stream) {
  const int64_t kg = k / 16, ngroups = rows * kg;
  const int64_t esize = x_dtype == kDtypeF32 ? 4 : 2;
  // at most 512 workgroups, each ending with one atomic on the same word
  // (2048 measured twice as slow on a 32768 x 1024 slab)
  const int64_t want = (ngroups + kKvAmaxThreads - 1) / kKvAmaxThreads;
  const unsigned grid = static_cast<unsigned>(want < 512 ? want : 512);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  unsigned* bits = reinterpret_cast<unsigned*>(amax);
  if (x_dtype == kDtypeF32)
    kv_amax_kernel<0><<<grid, kKvAmaxThreads, 0, stream>>>(xb, ngroups, kg, ldx * esize, bits);
  else
    kv_amax_kernel<1><<<grid, kKvAmaxThreads, 0, stream>>>(xb, ngroups, kg, ldx * esize, bits);
  return hipGetLastError();
}

hipError_t launch_kv_scale(const float* amax, float* scale, hipStream_t stream) {
  kv_scale_kernel<<<1, 1, 0, stream>>>(amax, scale);
  return hipGetLastError();
}

hipError_t launch_kv_cast(const void* x, int x_dtype, int64_t rows, int64_t k,
                          int64_t ldx, const float* scale, uint8_t* out,
                          int64_t ldo, hipStream_t stream) {
  const int64_t kg = k / 16, ngroups = rows * kg;
  const int64_t esize = x_dtype == kDtypeF32 ? 4 : 2;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (x_dtype == kDtypeF32)
    kv_cast_kernel<0><<<grid_for(ngroups), 256, 0, stream>>>(xb, ngroups, kg, ldx * esize,
                                                             scale, out, ldo);
  else
    kv_cast_kernel<1><<<grid_for(ngroups), 256, 0, stream>>>(xb, ngroups, kg, ldx * esize,
                                                             scale, out, ldo);
  return hipGetLastError();
}

}  // namespace nvfp4
