// Device-side NVFP4 quantisation of one 16-element block, shared by the
// quantisation kernels and the fused small-M quantise + GEMM kernel.
//
// Format: the explainer page "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか",
// section 前提1, and the arxiv-wiki page on the same paper, section 접근 방법:
// E2M1 values, one E4M3 scale per 16 elements from the block maximum over 6,
// one FP32 scale per tensor.  Every rounding decision is exact (the quotient
// is compared with the rounding midpoints without error); results are
// bit-identical to the definition for every finite input.
//   * block max as a packed 16-bit integer max of the magnitude bits;
//   * block scale by the gfx950 fp32 -> E4M3 conversion of m / (6 g) scaled
//     by 1 -+ 2^-18 (two conversions in one instruction); equal results
//     prove the exact quotient rounds the same way, else a float64 settle;
//   * element codes by the gfx950 fp4 conversion (round to nearest even,
//     saturating, sign kept) of x * r for two reciprocals bracketing
//     1 / (e4m3(s) g); where the two disagree (a value within 2^-18 of a
//     rounding midpoint), that element alone is settled with one exact FMA.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"

namespace nvfp4 {
namespace {

// g = RNE_fp32(amax / 2688).  The float64 quotient is rounded once more to
// binary32; A / 2688 is either exact in binary32 or far (relative 2^-30)
// from every binary32 rounding boundary, so this is one correct rounding.
__device__ __forceinline__ float global_from_amax(float a) {
  return static_cast<float>(static_cast<double>(a) / 2688.0);
}

constexpr int kDtypeF32 = 0;
constexpr int kModeCompute = 0;

// binary32 reciprocal of 6 g where 6 g is far from the ends of the binary32
// range (*ok), else 0: encode_block then settles every scale in float64
__device__ __forceinline__ float recip_6g(float g, bool* ok) {
  const float g6 = 6.0f * g;
  *ok = g6 >= 0x1p-100f && g6 <= 0x1p100f;
  return *ok ? __builtin_amdgcn_rcpf(g6) : 0.0f;
}

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

// A block's raw bytes: 32 (bf16) or 64 (fp32), as 16-byte vectors.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int DTYPE>
struct RawBlock {
  static constexpr int kVec = DTYPE == kDtypeF32 ? 4 : 2;
  u32x4 q[kVec];
};

template <int DTYPE>
__device__ __forceinline__ void fetch_block(const uint8_t* src, RawBlock<DTYPE>& r) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int i = 0; i < RawBlock<DTYPE>::kVec; ++i) r.q[i] = __builtin_nontemporal_load(p + i);
}

// Unpacks a block to 16 binary32 values and returns max |x| as binary32
// bits (an integer max over magnitude bits equals the float max).
__device__ __forceinline__ unsigned unpack_block(const RawBlock<1>& r, float* v) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const unsigned w[8] = {r.q[0].x, r.q[0].y, r.q[0].z, r.q[0].w,
                         r.q[1].x, r.q[1].y, r.q[1].z, r.q[1].w};
  u16x2 mx = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  }
  return static_cast<unsigned>(mx[0] > mx[1] ? mx[0] : mx[1]) << 16;
}

__device__ __forceinline__ unsigned unpack_block(const RawBlock<0>& r, float* v) {
  unsigned mx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i] = __uint_as_float(r.q[i].x);
    v[4 * i + 1] = __uint_as_float(r.q[i].y);
    v[4 * i + 2] = __uint_as_float(r.q[i].z);
    v[4 * i + 3] = __uint_as_float(r.q[i].w);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  return mx;
}

// Raw bytes of half a block (8 elements: 16 bytes of bf16, 32 of fp32).
template <int DTYPE>
struct RawHalf {
  u32x4 q[DTYPE == kDtypeF32 ? 2 : 1];
};

template <int DTYPE>
__device__ __forceinline__ void fetch_half(const uint8_t* src, RawHalf<DTYPE>& r) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  r.q[0] = __builtin_nontemporal_load(p);
  if constexpr (DTYPE == kDtypeF32) r.q[1] = __builtin_nontemporal_load(p + 1);
}

// Half a block as binary32 values; returns max |x| as binary32 bits.
template <int DTYPE>
__device__ __forceinline__ unsigned unpack_half(const RawHalf<DTYPE>& r, float* v) {
  if constexpr (DTYPE == kDtypeF32) {
    const u32x4 a = r.q[0], b = r.q[1];
    const unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    unsigned mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = __uint_as_float(w[i]);
      mx = max(mx, w[i] & 0x7FFFFFFFu);
    }
    return mx;
  } else {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const u32x4 a = r.q[0];
    const unsigned w[4] = {a.x, a.y, a.z, a.w};
    u16x2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    }
    return static_cast<unsigned>(mx[0] > mx[1] ? mx[0] : mx[1]) << 16;
  }
}

template <int DTYPE>
__device__ __forceinline__ unsigned load_half(const uint8_t* src, float* v) {
  RawHalf<DTYPE> r;
  fetch_half<DTYPE>(src, r);
  return unpack_half<DTYPE>(r, v);
}

template <int DTYPE>
__device__ __forceinline__ unsigned load_block(const void* base, float* v) {
  RawBlock<DTYPE> r;
  fetch_block<DTYPE>(static_cast<const uint8_t*>(base), r);
  return unpack_block(r, v);
}

// Candidate E4M3 codes of q * (1 - 2^-18) and q * (1 + 2^-18) for q >= 0,
// from one gfx950 fp32 -> OCP E4M3 conversion (round to nearest even; the
// inputs are clamped to 448 first, where the hardware would give NaN above
// 464, so the result saturates as RNE_SAT does).  Equal codes prove that
// every value in between, the exact quotient included, rounds to them.
__device__ __forceinline__ unsigned e4m3_bracket(float q, bool* exact) {
  const float lo = fminf(q * (1.0f - 0x1p-18f), 448.0f);
  const float hi = fminf(q * (1.0f + 0x1p-18f), 448.0f);
  const unsigned pk = static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false));
  *exact = *exact || ((pk ^ (pk >> 8)) & 0xFFu) != 0;
  return pk & 0xFFu;
}

// Exact code magnitude of an element whose two bracketed candidates are the
// adjacent codes lo and lo + 1: compare |x| with the midpoint between them
// times e4m3(s) g.  mid * e4m3(s) has <= 7 significant bits (exact in
// binary32) and the FMA rounds |x| - mid e4m3(s) g once, so the sign of d
// is that of the exact difference (no underflow: e4m3(s) g >= 2^-100 on
// this path).  Ties go to the even code.
__device__ __forceinline__ unsigned settle_e2m1(float ax, unsigned lo, float dec,
                                                float g) {
  const float mid = lo == 0u ? 0.25f : lo == 1u ? 0.75f : lo == 2u ? 1.25f
                  : lo == 3u ? 1.75f : lo == 4u ? 2.5f : lo == 5u ? 3.5f : 5.0f;
  const float d = __builtin_fmaf(-(mid * dec), g, ax);
  return (d > 0.0f || (d == 0.0f && (lo & 1u))) ? lo + 1u : lo;
}

// Per-lane LDS row used to index a block's values by a lane-varying
// element number (registers cannot be indexed that way without going
// through scratch memory).  Row stride 20 floats keeps 16-byte alignment.
constexpr int kRowFloats = 20;

// Re-decides the nibbles of the block's code words (from the smaller
// reciprocal) where the two bracketed conversions disagree, one element per
// loop trip; a wave loops as often as its busiest lane needs (almost always
// once).  `row` is this lane's LDS row; only this lane touches it.
__device__ __forceinline__ void settle_block(uint2* c, unsigned dx, unsigned dy,
                                             const float* v, float dec, float g,
                                             float* row) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<float4*>(row + 4 * j) = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  uint64_t d = static_cast<uint64_t>(dx) | (static_cast<uint64_t>(dy) << 32);
  uint64_t w = static_cast<uint64_t>(c->x) | (static_cast<uint64_t>(c->y) << 32);
  while (d) {
    const unsigned i = static_cast<unsigned>(__builtin_ctzll(d)) >> 2;
    d &= ~(0xFull << (4 * i));
    const unsigned lo = static_cast<unsigned>(w >> (4 * i)) & 7u;
    const unsigned code = settle_e2m1(__builtin_fabsf(row[i]), lo, dec, g);
    w = (w & ~(7ull << (4 * i))) | (static_cast<uint64_t>(code) << (4 * i));
  }
  c->x = static_cast<unsigned>(w);
  c->y = static_cast<unsigned>(w >> 32);
}

// One block: scale byte and 8 code bytes from 16 values and their max.
// `inv6g` = 1 / (6 g) in binary32 when usable (`g_ok`), `g` the global.
__device__ __forceinline__ void encode_block(const float* v, float m, float g,
                                             float inv6g, bool g_ok,
                                             unsigned* s_out, uint2* c_out,
                                             float* row) {
  // block scale RNE_SAT_E4M3(m / (6 g)): bracketed hardware conversion of
  // m * inv6g (relative error < 2^-21), exact float64 settle otherwise
  unsigned s = 0;
  if (m > 0.0f && g > 0.0f) {
    bool slow = !g_ok;
    s = e4m3_bracket(m * inv6g, &slow);
    if (slow) {
      const double md = static_cast<double>(m), den6 = 6.0 * static_cast<double>(g);
      s = e4m3_settle(e4m3_candidate(md / den6), md, den6);
    }
  }
  // element codes: x * r for two reciprocals bracketing 1 / (e4m3(s) g)
  // (zero is decided on s and g: the binary32 product can underflow to 0
  // while e4m3(s) g > 0; such blocks take the exact path)
  const bool zero = s == 0u || g == 0.0f;
  const float dec = e4m3_f32(s);
  const float S = dec * g;
  const bool extreme = !(zero || (S >= 0x1p-100f && S <= 0x1p100f));
  float r_lo = 0.0f, r_hi = 0.0f;
  if (!zero) {
    const float r = __builtin_amdgcn_rcpf(S);
    r_lo = r * (1.0f - 0x1p-18f);
    r_hi = r * (1.0f + 0x1p-18f);
  }
  uint2 c;
  c.x = cvt8(v, r_lo);
  c.y = cvt8(v + 8, r_lo);
  const unsigned dx = c.x ^ cvt8(v, r_hi), dy = c.y ^ cvt8(v + 8, r_hi);
  if (extreme) {
    // e4m3(s) g outside [2^-100, 2^100]: every code by exact float64 compares
    const double Sd = e4m3_value(s) * static_cast<double>(g);   // exact
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_exact(v[i], Sd) << (4 * (i & 7));
    c.x = w[0];
    c.y = w[1];
  } else if (dx | dy) {
    // a value within 2^-18 of a rounding midpoint (bf16 data whose mantissa
    // matches the tensor maximum lands this close under a self-calibrated
    // global): settle just those elements exactly
    settle_block(&c, dx, dy, v, dec, g, row);
  }
  *s_out = s;
  *c_out = c;
}

template <int DTYPE>
__device__ __forceinline__ const uint8_t* block_src(const uint8_t* x, int64_t b,
                                                    bool contiguous, int64_t kb,
                                                    int64_t ldx_bytes) {
  constexpr int64_t kBlockBytes = 16 * (DTYPE == kDtypeF32 ? 4 : 2);
  if (contiguous) return x + b * kBlockBytes;
  const int64_t row = b / kb;
  return x + row * ldx_bytes + (b - row * kb) * kBlockBytes;
}

// One block: load, encode, store.
template <int DTYPE>
__device__ __forceinline__ void quantize_one(const uint8_t* __restrict__ src, int64_t b,
                                             float g, float inv6g, bool g_ok,
                                             uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales, float* row) {
  RawBlock<DTYPE> raw;
  fetch_block<DTYPE>(src, raw);
  float v[16];
  const float m = __uint_as_float(unpack_block(raw, v));
  unsigned sc;
  uint2 cc;
  encode_block(v, m, g, inv6g, g_ok, &sc, &cc, row);
  __builtin_nontemporal_store(cc.x, reinterpret_cast<unsigned*>(codes) + 2 * b);
  __builtin_nontemporal_store(cc.y, reinterpret_cast<unsigned*>(codes) + 2 * b + 1);
  __builtin_nontemporal_store(static_cast<uint8_t>(sc), scales + b);
}

}  // namespace
}  // namespace nvfp4
