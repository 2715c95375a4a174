// W4A4 GEMM on NVFP4 operands for gfx950 (MI355X).
//
// Y[m][n] = g_a g_b * sum_k A_hat[m][k] B_hat[n][k], with A_hat and B_hat
// the NVFP4 tensors of the arxiv-wiki page on "Why Gated DeltaNet Survives
// 4-Bit Quantization" (section 접근 방법) and of the explainer page
// "論文解説: Gated DeltaNet はなぜ4bit量子化に耐えるのか" (section 前提1, where W4A4
// means both GEMM operands are 4-bit), and an optional gate epilogue of the
// same page's section 前提2 (alpha through softplus and exp, beta through a
// sigmoid).
//
// Design (gfx950):
//   * Packed operands are staged in LDS as they are stored: 4-bit codes
//     (0.5 B/element) and block scales, the scales already widened to fp16.
//     A tile of BM x BK codes is 1/4 the bytes of its bf16 form.
//   * Each wave decodes its MFMA fragments in registers: one gfx950
//     conversion turns two codes into two fp16 values of the E2M1 grid and
//     one packed fp16 multiply applies the block scale.  e2m1 * e4m3 has at
//     most 6 significant bits and lies in [2^-10, 2688], so it is exact in
//     fp16 (normal range from 2^-14, 11-bit significand): nothing is
//     rounded before the MFMA.  fp16 is used instead of bf16 because gfx950
//     has the packed fp16 multiply and the same MFMA rate for both types.
//   * v_mfma_f32_32x32x16_f16 accumulates in fp32; products of two decoded
//     values (<= 12 bits) are exact in fp32.
//   * The K order inside a BK tile is permuted identically for A and B
//     (lane half h covers one contiguous K range), which leaves the dot
//     product unchanged and lets every lane read 16 contiguous bytes.
//   * Epilogue: fp32 accumulator * (g_a g_b), optional gate, fp32 or bf16
//     (round to nearest even) store.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

namespace nvfp4 {
namespace {

constexpr int kOutF32 = 0;
constexpr int kEpiNone = 0;
constexpr int kEpiAlpha = 1;
constexpr int kEpiBeta = 2;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;                 // K elements per LDS stage
constexpr int kCodeBytes = kBK / 2;      // 64 code bytes per row per stage
constexpr int kCodeStride = kCodeBytes + 16;  // padded LDS row (bytes)
constexpr int kScalesPerRow = kBK / 16;  // 8 block scales per row per stage

// OCP E4M3 byte (0x00..0x7E) -> fp16 bits, exact.  Normal codes map by a
// shift and an exponent rebias (7 -> 15); subnormals m * 2^-9 go through
// binary32.
__device__ __forceinline__ unsigned short e4m3_to_f16_bits(unsigned c) {
  if (c >= 8u) return static_cast<unsigned short>((c << 7) + 0x2000u);
  const _Float16 h = static_cast<_Float16>(static_cast<float>(c) * 0.001953125f);
  return __builtin_bit_cast(unsigned short, h);
}

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

template <int EPI>
__device__ __forceinline__ float epilogue(float y) {
  if constexpr (EPI == kEpiAlpha) {
    // exp(-softplus(y)), softplus(y) = max(y, 0) + log1p(exp(-|y|))
    const float sp = fmaxf(y, 0.0f) + log1pf(expf(-fabsf(y)));
    return expf(-sp);
  } else if constexpr (EPI == kEpiBeta) {
    return 1.0f / (1.0f + expf(-y));
  } else {
    return y;
  }
}

// Copies one operand's BK-wide stage (ROWS rows of codes and scales) from
// global memory to LDS.  Rows past `rows` and K past `k` read as zero.
template <int ROWS, int NT, bool ALIGNED>
struct StageLoader {
  static constexpr int kChunks = ROWS * (kCodeBytes / 16);   // 16-byte chunks
  static constexpr int kPerThread = (kChunks + NT - 1) / NT;
  static constexpr int kScalePerThread = (ROWS * kScalesPerRow + NT - 1) / NT;
  uint4 code[kPerThread];
  unsigned char sc[kScalePerThread];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales,
                                       int64_t row0, int64_t rows, int64_t k,
                                       int64_t k0, int tid) {
    const int64_t kbytes = k / 2, kblocks = k / 16;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * NT;
      const int r = c / (kCodeBytes / 16), part = c % (kCodeBytes / 16);
      const int64_t grow = row0 + r;
      const int64_t kb = k0 / 2 + part * 16;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < kChunks && grow < rows) {
        const uint8_t* p = codes + grow * kbytes + kb;
        if (ALIGNED && kb + 16 <= kbytes) {
          v = *reinterpret_cast<const uint4*>(p);
        } else {
          if (kb + 8 <= kbytes) {
            const uint2 lo = *reinterpret_cast<const uint2*>(p);
            v.x = lo.x; v.y = lo.y;
          }
          if (kb + 16 <= kbytes) {
            const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
            v.z = hi.x; v.w = hi.y;
          }
        }
      }
      code[i] = v;
    }
#pragma unroll
    for (int i = 0; i < kScalePerThread; ++i) {
      const int c = tid + i * NT;
      const int r = c / kScalesPerRow, j = c % kScalesPerRow;
      const int64_t grow = row0 + r;
      const int64_t blk = k0 / 16 + j;
      unsigned char v = 0;
      if (c < ROWS * kScalesPerRow && grow < rows && blk < kblocks)
        v = scales[grow * kblocks + blk];
      sc[i] = v;
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds_codes,
                                        unsigned short* lds_scales,
                                        int tid) const {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * NT;
      if (c < kChunks) {
        const int r = c / (kCodeBytes / 16), part = c % (kCodeBytes / 16);
        *reinterpret_cast<uint4*>(lds_codes + r * kCodeStride + part * 16) = code[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kScalePerThread; ++i) {
      const int c = tid + i * NT;
      if (c < ROWS * kScalesPerRow) lds_scales[c] = e4m3_to_f16_bits(sc[i]);
    }
  }
};

// One wave's fragments for a stage: for each of T 32-row tiles, 32 code
// bytes (this lane's K half) and 4 fp16 block scales.
template <int T>
struct Frags {
  uint4 code[T][2];
  uint2 scale[T];

  __device__ __forceinline__ void read(const uint8_t* lds_codes,
                                       const unsigned short* lds_scales,
                                       int row_base, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = row_base + t * 32 + r;
      const uint8_t* p = lds_codes + row * kCodeStride + h * 32;
      code[t][0] = *reinterpret_cast<const uint4*>(p);
      code[t][1] = *reinterpret_cast<const uint4*>(p + 16);
      scale[t] = *reinterpret_cast<const uint2*>(lds_scales + row * kScalesPerRow + h * 4);
    }
  }

  // fp16 operand of k-step ks (0..7) for tile t: K range h*64 + 8*ks .. +8,
  // block h*4 + ks/2.
  __device__ __forceinline__ half8_t operand(int t, int ks) const {
    const uint4 q = code[t][ks >> 2];
    const unsigned w = (ks & 3) == 0 ? q.x : (ks & 3) == 1 ? q.y : (ks & 3) == 2 ? q.z : q.w;
    const unsigned sw = (ks >> 2) ? scale[t].y : scale[t].x;
    const unsigned short sb = (ks & 2) ? static_cast<unsigned short>(sw >> 16)
                                       : static_cast<unsigned short>(sw & 0xFFFFu);
    const _Float16 s = __builtin_bit_cast(_Float16, sb);
    half2_t sc;
    sc[0] = s;
    sc[1] = s;
    return decode8(w, sc);
  }
};

template <int WM, int WN, int TM, int TN, bool ALIGNED, int OUT, int EPI>
__global__ void __launch_bounds__(WM * WN * 64, 1)
w4a4_gemm_kernel(const uint8_t* __restrict__ a_codes,
                 const uint8_t* __restrict__ a_scales,
                 const float* __restrict__ a_global, int64_t m,
                 const uint8_t* __restrict__ b_codes,
                 const uint8_t* __restrict__ b_scales,
                 const float* __restrict__ b_global, int64_t n, int64_t k,
                 void* __restrict__ out, int64_t ldo, int tiles_m,
                 int tiles_n) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kCodeStride];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kCodeStride];
  __shared__ __attribute__((aligned(16))) unsigned short lds_sa[2][BM * kScalesPerRow];
  __shared__ __attribute__((aligned(16))) unsigned short lds_sb[2][BN * kScalesPerRow];

  // Tile order: workgroups are dealt round-robin to the 8 XCDs; give each
  // XCD a contiguous range of tiles, walked in column groups of 8 M-tiles so
  // that concurrently running tiles share A and B panels in that XCD's L2.
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if (ntiles % 8 == 0) bid = (bid % 8) * (ntiles / 8) + bid / 8;
  constexpr int kGroup = 8;
  const int group = bid / (kGroup * tiles_n);
  const int first_m = group * kGroup;
  const int gm = min(tiles_m - first_m, kGroup);
  const int tile_m = first_m + (bid % (kGroup * tiles_n)) % gm;
  const int tile_n = (bid % (kGroup * tiles_n)) / gm;
  const int64_t m0 = static_cast<int64_t>(tile_m) * BM;
  const int64_t n0 = static_cast<int64_t>(tile_n) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  StageLoader<BM, NT, ALIGNED> la;
  StageLoader<BN, NT, ALIGNED> lb;
  const int nk = static_cast<int>((k + kBK - 1) / kBK);
  la.load(a_codes, a_scales, m0, m, k, 0, tid);
  lb.load(b_codes, b_scales, n0, n, k, 0, tid);
  la.store(lds_a[0], lds_sa[0], tid);
  lb.store(lds_b[0], lds_sb[0], tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(a_codes, a_scales, m0, m, k, static_cast<int64_t>(kt + 1) * kBK, tid);
      lb.load(b_codes, b_scales, n0, n, k, static_cast<int64_t>(kt + 1) * kBK, tid);
    }
    Frags<TM> fa;
    Frags<TN> fb;
    fa.read(lds_a[cur], lds_sa[cur], wm * TM * 32, lane);
    fb.read(lds_b[cur], lds_sb[cur], wn * TN * 32, lane);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      half8_t av[TM], bv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) av[i] = fa.operand(i, ks);
#pragma unroll
      for (int j = 0; j < TN; ++j) bv[j] = fb.operand(j, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(lds_a[cur ^ 1], lds_sa[cur ^ 1], tid);
      lb.store(lds_b[cur ^ 1], lds_sb[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and, for
  // element e, row 8 (e / 4) + 4 (l / 32) + e % 4.
  // g_a g_b is exact in float64; one rounding to binary32 per output
  const double gab = static_cast<double>(*a_global) * static_cast<double>(*b_global);
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn * TN * 32 + j * 32 + col_l;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * TM * 32 + i * 32 + 8 * (e >> 2) + row_l + (e & 3);
        if (row < m && col < n) {
          const float y = epilogue<EPI>(static_cast<float>(static_cast<double>(acc[i][j][e]) * gab));
          if constexpr (OUT == kOutF32)
            static_cast<float*>(out)[row * ldo + col] = y;
          else
            static_cast<unsigned short*>(out)[row * ldo + col] = f32_to_bf16_rne(y);
        }
      }
    }
}

template <int WM, int WN, int TM, int TN, bool ALIGNED, int OUT, int EPI>
hipError_t launch_cfg(const uint8_t* a_codes, const uint8_t* a_scales,
                      const float* a_global, int64_t m,
                      const uint8_t* b_codes, const uint8_t* b_scales,
                      const float* b_global, int64_t n, int64_t k, void* out,
                      int64_t ldo, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tm = (m + BM - 1) / BM, tn = (n + BN - 1) / BN;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  w4a4_gemm_kernel<WM, WN, TM, TN, ALIGNED, OUT, EPI>
      <<<static_cast<unsigned>(tm * tn), WM * WN * 64, 0, stream>>>(
          a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, n, k,
          out, ldo, static_cast<int>(tm), static_cast<int>(tn));
  return hipGetLastError();
}

template <bool ALIGNED, int OUT, int EPI>
hipError_t dispatch_shape(const uint8_t* a_codes, const uint8_t* a_scales,
                          const float* a_global, int64_t m,
                          const uint8_t* b_codes, const uint8_t* b_scales,
                          const float* b_global, int64_t n, int64_t k,
                          void* out, int64_t ldo, hipStream_t stream) {
  return launch_cfg<2, 2, 4, 4, ALIGNED, OUT, EPI>(
      a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, n, k, out,
      ldo, stream);
}

template <int OUT, int EPI>
hipError_t dispatch_align(const uint8_t* a_codes, const uint8_t* a_scales,
                          const float* a_global, int64_t m,
                          const uint8_t* b_codes, const uint8_t* b_scales,
                          const float* b_global, int64_t n, int64_t k,
                          void* out, int64_t ldo, hipStream_t stream) {
  // 16-byte code loads need 16-byte aligned rows
  const bool aligned = (k / 2) % 16 == 0;
  if (aligned)
    return dispatch_shape<true, OUT, EPI>(a_codes, a_scales, a_global, m,
                                          b_codes, b_scales, b_global, n, k,
                                          out, ldo, stream);
  return dispatch_shape<false, OUT, EPI>(a_codes, a_scales, a_global, m,
                                         b_codes, b_scales, b_global, n, k,
                                         out, ldo, stream);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                       const float* a_global, int64_t m,
                       const uint8_t* b_codes, const uint8_t* b_scales,
                       const float* b_global, int64_t n, int64_t k,
                       void* out, int out_dtype, int64_t ldo, int epilogue,
                       hipStream_t stream) {
#define NVFP4_GEMM_ARGS a_codes, a_scales, a_global, m, b_codes, b_scales, \
                        b_global, n, k, out, ldo, stream
  if (out_dtype == kOutF32) {
    if (epilogue == kEpiAlpha) return dispatch_align<0, kEpiAlpha>(NVFP4_GEMM_ARGS);
    if (epilogue == kEpiBeta) return dispatch_align<0, kEpiBeta>(NVFP4_GEMM_ARGS);
    return dispatch_align<0, kEpiNone>(NVFP4_GEMM_ARGS);
  }
  if (epilogue == kEpiAlpha) return dispatch_align<1, kEpiAlpha>(NVFP4_GEMM_ARGS);
  if (epilogue == kEpiBeta) return dispatch_align<1, kEpiBeta>(NVFP4_GEMM_ARGS);
  return dispatch_align<1, kEpiNone>(NVFP4_GEMM_ARGS);
#undef NVFP4_GEMM_ARGS
}

}  // namespace nvfp4
