// NVFP4 dequantisation and quantisation-error statistics for gfx950.
//
// Value of an element: sign * E2M1 * E4M3 * g (the format of the explainer
// page "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか", section 前提1, and
// of the arxiv-wiki page on the same paper, section 접근 방법).  e2m1 * e4m3
// has at most 6 significant bits and is exact in binary32; times the
// binary32 global the exact value has at most 30, so:
//   * binary32 output: one IEEE multiply, a single rounding;
//   * bfloat16 output: the binary32 product rounded to bfloat16 to nearest
//     even, with the exact product deciding where the binary32 value lies
//     exactly on a bfloat16 midpoint; that equals one rounding of the exact
//     value.
// Error statistics (the A4 / W4 error percentages and max/RMS of the
// input statistics on the arxiv-wiki page, section 접근 방법): per row,
// in float64, sum x^2, sum (x - x_hat)^2 and max |x|.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kDtypeF32 = 0;
constexpr int kOutF32 = 0;

// e2m1 * e4m3 of the 16 codes of a block (8 bytes), exact in binary32.
__device__ __forceinline__ void decode_block(uint2 c, float sc, float* v) {
  const unsigned w[2] = {c.x, c.y};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 p = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h], 1.0f, 0)
                    : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h], 1.0f, 1)
                    : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h], 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[h], 1.0f, 3);
      v[8 * h + 2 * j] = p[0] * sc;
      v[8 * h + 2 * j + 1] = p[1] * sc;
    }
}

__device__ __forceinline__ unsigned short bf16_rne_bits(float f) {
  const unsigned u = __float_as_uint(f);
  return static_cast<unsigned short>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Nearest-even bfloat16 of the exact product v * g (v = e2m1 * e4m3, exact).
// f = fl32(v * g) is one correct rounding; rounding f once more to bfloat16
// differs from one rounding of the exact product only where f lies exactly
// on a bfloat16 midpoint (low 16 bits 0x8000): a midpoint is itself a
// binary32 value, so rounding to binary32 can reach one but never cross it.
// There the exact product decides: larger in magnitude than f rounds away
// from zero, smaller toward zero, equal keeps the tie (to even).  The
// residual fma(v, g, -f) is exact for products of normal magnitude; near the
// subnormal range the product is formed in float64 (exact: v * g has at
// most 30 significant bits).
__device__ __forceinline__ unsigned short bf16_of_product(float v, float g) {
  const float f = v * g;
  unsigned u = __float_as_uint(f);
  if ((u & 0xFFFFu) == 0x8000u) {
    int dir = 0;   // sign of |exact| - |f|
    if (__builtin_fabsf(f) >= 0x1p-100f) {
      const float e = __builtin_fmaf(v, g, -f);   // exact - f, exactly
      if (e != 0.0f) dir = ((e > 0.0f) == (f > 0.0f)) ? 1 : -1;
    } else {
      const double p = static_cast<double>(v) * static_cast<double>(g);   // exact
      const double fd = static_cast<double>(f);
      if (p != fd) dir = __builtin_fabs(p) > __builtin_fabs(fd) ? 1 : -1;
    }
    u = dir > 0 ? u + 1u : dir < 0 ? u - 1u : u;   // off the midpoint, or the tie
  }
  return bf16_rne_bits(__uint_as_float(u));
}

// Lanes per block: every lane stores one 16-byte piece of the output (four
// binary32 or eight bfloat16 values), so that a wave's non-temporal store
// covers 1 KiB contiguously.  With one lane per block (several stores per
// lane, 32 or 64 bytes apart) the streaming stores ran 1.5x (bf16) to 8x
// (fp32) slower.
template <int OUT>
constexpr int kLanesPerBlock = OUT == kOutF32 ? 4 : 2;

// 8 code bytes + 1 scale byte in, 16 values out per block, over
// kLanesPerBlock lanes; non-temporal stores, as the output is a stream.
template <int OUT>
__global__ void __launch_bounds__(256)
dequantize_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  const float* __restrict__ global, int64_t nblocks, int64_t kb,
                  void* __restrict__ out, int64_t ldo) {
  const float g = *global;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const bool flat = ldo == kb * 16;   // rows back to back: no division per lane
  if constexpr (OUT == kOutF32) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
         t < nblocks * 4; t += stride) {
      const int64_t b = t >> 2;
      const unsigned c = reinterpret_cast<const unsigned short*>(codes)[t];   // 4 codes
      const float sc = e4m3_f32(scales[b]);
      const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
      const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
      int64_t dst = t * 4;
      if (!flat) {
        const int64_t row = b / kb;
        dst = row * ldo + (b - row * kb) * 16 + (t & 3) * 4;
      }
      // (e2m1 * e4m3) is exact; times g it is rounded once
      const f32x4 o = {(p0[0] * sc) * g, (p0[1] * sc) * g, (p1[0] * sc) * g, (p1[1] * sc) * g};
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(static_cast<float*>(out) + dst));
    }
  } else {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
         t < nblocks * 2; t += stride) {
      const int64_t b = t >> 1;
      const unsigned c = reinterpret_cast<const unsigned*>(codes)[t];   // 8 codes
      const float sc = e4m3_f32(scales[b]);
      unsigned w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x2 p = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)
                      : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1)
                      : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
        w[j] = static_cast<unsigned>(bf16_of_product(p[0] * sc, g)) |
               (static_cast<unsigned>(bf16_of_product(p[1] * sc, g)) << 16);
      }
      int64_t dst = t * 8;
      if (!flat) {
        const int64_t row = b / kb;
        dst = row * ldo + (b - row * kb) * 16 + (t & 1) * 8;
      }
      const u32x4 o = {w[0], w[1], w[2], w[3]};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<unsigned short*>(out) + dst));
    }
  }
}

// A block's raw input bytes (bf16: 32 bytes, fp32: 64) and its values as
// binary32 (exact from bf16 or fp32).
template <int DTYPE>
struct RawX {
  static constexpr int kVec = DTYPE == kDtypeF32 ? 4 : 2;
  uint4 q[kVec];
};

template <int DTYPE>
__device__ __forceinline__ void load_raw(const uint8_t* src, RawX<DTYPE>& r) {
#pragma unroll
  for (int i = 0; i < RawX<DTYPE>::kVec; ++i) r.q[i] = reinterpret_cast<const uint4*>(src)[i];
}

template <int DTYPE>
__device__ __forceinline__ void raw_values(const RawX<DTYPE>& r, float* x) {
  if constexpr (DTYPE == kDtypeF32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[4 * q] = __uint_as_float(r.q[q].x); x[4 * q + 1] = __uint_as_float(r.q[q].y);
      x[4 * q + 2] = __uint_as_float(r.q[q].z); x[4 * q + 3] = __uint_as_float(r.q[q].w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const unsigned w[4] = {r.q[q].x, r.q[q].y, r.q[q].z, r.q[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        x[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
}

// One wave per row: lane l takes blocks l, l + 64, ..., kBatch of them at a
// time, all of a batch's loads issued before any of its arithmetic (a row's
// blocks one after the other left each wave waiting on memory once per
// block); float64 sums, per lane in block order, are reduced across the
// wave.  stats[row] = {sum x^2, sum (x - x_hat)^2, max|x|}.
constexpr int kStatsBatch = 4;
template <int DTYPE>
__global__ void __launch_bounds__(256)
error_stats_kernel(const uint8_t* __restrict__ x, int64_t rows, int64_t kb,
                   int64_t ldx_bytes, const uint8_t* __restrict__ codes,
                   const uint8_t* __restrict__ scales, const float* __restrict__ global,
                   double* __restrict__ stats) {
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole waves leave together
  const double g = static_cast<double>(*global);
  const uint8_t* const xrow = x + row * ldx_bytes;
  const int64_t blk0 = row * kb;
  double sx = 0.0, se = 0.0;
  unsigned mx = 0u;
  for (int64_t b0 = lane; b0 < kb; b0 += 64 * kStatsBatch) {
    RawX<DTYPE> raw[kStatsBatch];
    uint2 cw[kStatsBatch];
    unsigned sb[kStatsBatch];
#pragma unroll
    for (int u = 0; u < kStatsBatch; ++u) {
      const int64_t b = b0 + 64 * u;
      const int64_t bb = b < kb ? b : kb - 1;   // past the row: a valid block, not counted
      load_raw<DTYPE>(xrow + bb * (16 * kElemBytes), raw[u]);
      cw[u] = reinterpret_cast<const uint2*>(codes)[blk0 + bb];
      sb[u] = scales[blk0 + bb];
    }
#pragma unroll
    for (int u = 0; u < kStatsBatch; ++u) {
      if (b0 + 64 * u >= kb) break;
      float xv[16], v[16];
      raw_values<DTYPE>(raw[u], xv);
      decode_block(cw[u], e4m3_f32(sb[u]), v);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double xd = static_cast<double>(xv[i]);
        // v * g is exact in float64 (at most 6 + 24 significant bits), so the
        // fused form rounds x - v g once, as the separate product and
        // difference do: the same value in one float64 operation fewer
        const double d = __builtin_fma(-static_cast<double>(v[i]), g, xd);
        sx = __builtin_fma(xd, xd, sx);
        se = __builtin_fma(d, d, se);
        mx = max(mx, __float_as_uint(xv[i]) & 0x7FFFFFFFu);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sx += __shfl_xor(sx, off);
    se += __shfl_xor(se, off);
    mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
  }
  if (lane == 0) {
    stats[3 * row] = sx;
    stats[3 * row + 1] = se;
    stats[3 * row + 2] = static_cast<double>(__uint_as_float(mx));
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales,
                             const float* global, int64_t rows, int64_t k,
                             void* out, int out_dtype, int64_t ldo,
                             hipStream_t stream) {
  const int64_t kb = k / 16, nblocks = rows * kb;
  const int64_t lanes = nblocks * (out_dtype == kOutF32 ? kLanesPerBlock<0> : kLanesPerBlock<1>);
  const int64_t want = (lanes + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 0x7FFFFFFF ? want : 0x7FFFFFFF);
  if (out_dtype == kOutF32)
    dequantize_kernel<0><<<grid, 256, 0, stream>>>(codes, scales, global, nblocks, kb, out, ldo);
  else
    dequantize_kernel<1><<<grid, 256, 0, stream>>>(codes, scales, global, nblocks, kb, out, ldo);
  return hipGetLastError();
}

hipError_t launch_error_stats(const void* x, int x_dtype, int64_t rows, int64_t k,
                              int64_t ldx, const uint8_t* codes,
                              const uint8_t* scales, const float* global,
                              double* stats, hipStream_t stream) {
  const int64_t esize = x_dtype == kDtypeF32 ? 4 : 2;
  const int64_t want = (rows + 3) / 4;
  if (want > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(want);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (x_dtype == kDtypeF32)
    error_stats_kernel<0><<<grid, 256, 0, stream>>>(xb, rows, k / 16, ldx * esize, codes,
                                                    scales, global, stats);
  else
    error_stats_kernel<1><<<grid, 256, 0, stream>>>(xb, rows, k / 16, ldx * esize, codes,
                                                    scales, global, stats);
  return hipGetLastError();
}

}  // namespace nvfp4
