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
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "gemm_common.h"
#include "internal.h"
#include "quant_device.h"

namespace nvfp4 {
namespace {

constexpr int kBK = 128;                 // K elements per LDS stage
constexpr int kCodeBytes = kBK / 2;      // 64 code bytes per row per stage
constexpr int kCodeStride = kCodeBytes + 16;  // padded LDS row (bytes)
constexpr int kScalesPerRow = kBK / 16;  // 8 block scales per row per stage

// Copies one operand's BK-wide stage (ROWS rows of codes and scales) from
// global memory to LDS through registers.
//
// ALIGNED (k % 128 == 0; code and scale arrays are 16-byte aligned in
// every call): every 16-byte code
// chunk and every row's 8 scale bytes of a stage lie inside k, so loads are
// unconditional (rows past `rows` read a clamped, valid row) and row validity
// is applied when storing to LDS.  No load result is consumed before the
// store, so all of a stage's loads are in flight together.  Scales are
// widened to fp16 by the gfx950 fp8 conversion (OCP E4M3, exact in fp16).
//
// Otherwise (ragged k) each 8-byte half-chunk and each scale byte is
// guarded individually.
template <int ROWS, int NT, bool ALIGNED>
struct StageLoader {
  static constexpr int kChunks = ROWS * (kCodeBytes / 16);   // 16-byte chunks
  static constexpr int kPerThread = (kChunks + NT - 1) / NT;
  static constexpr int kScaleRows = (ROWS + NT - 1) / NT;     // rows per thread
  uint4 code[kPerThread];
  uint2 sc[kScaleRows];
  unsigned valid;   // bit i: chunk i is inside the matrix; bit 16+j: scale row j

  __device__ __forceinline__ void load(const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ scales,
                                       int64_t row0, int64_t rows, int64_t k,
                                       int64_t k0, int tid) {
    const int64_t kbytes = k / 2, kblocks = k / 16;
    valid = 0u;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * NT;
      const int r = c / (kCodeBytes / 16), part = c % (kCodeBytes / 16);
      const int64_t grow = row0 + r;
      const int64_t kb = k0 / 2 + part * 16;
      if constexpr (ALIGNED) {
        const int64_t srow = grow < rows ? grow : rows - 1;
        code[i] = *reinterpret_cast<const uint4*>(codes + srow * kbytes + kb);
        valid |= (c < kChunks && grow < rows) ? (1u << i) : 0u;
      } else {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (c < kChunks && grow < rows) {
          const uint8_t* p = codes + grow * kbytes + kb;
          if (kb + 8 <= kbytes) {
            const uint2 lo = *reinterpret_cast<const uint2*>(p);
            v.x = lo.x; v.y = lo.y;
          }
          if (kb + 16 <= kbytes) {
            const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
            v.z = hi.x; v.w = hi.y;
          }
        }
        code[i] = v;
        valid |= 1u << i;
      }
    }
#pragma unroll
    for (int j = 0; j < kScaleRows; ++j) {
      const int r = tid + j * NT;
      const int64_t grow = row0 + r;
      const int64_t blk = k0 / 16;
      if constexpr (ALIGNED) {
        const int64_t srow = grow < rows ? grow : rows - 1;
        sc[j] = *reinterpret_cast<const uint2*>(scales + srow * kblocks + blk);
        valid |= (r < ROWS && grow < rows) ? (1u << (16 + j)) : 0u;
      } else {
        unsigned w[2] = {0u, 0u};
        if (r < ROWS && grow < rows) {
#pragma unroll
          for (int b = 0; b < kScalesPerRow; ++b)
            if (blk + b < kblocks)
              w[b >> 2] |= static_cast<unsigned>(scales[grow * kblocks + blk + b]) << (8 * (b & 3));
        }
        sc[j] = make_uint2(w[0], w[1]);
        valid |= 1u << (16 + j);
      }
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
        const uint4 v = (valid >> i) & 1u ? code[i] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(lds_codes + r * kCodeStride + part * 16) = v;
      }
    }
#pragma unroll
    for (int j = 0; j < kScaleRows; ++j) {
      const int r = tid + j * NT;
      if (r < ROWS) {
        const bool ok = (valid >> (16 + j)) & 1u;
        const unsigned lo = ok ? sc[j].x : 0u, hi = ok ? sc[j].y : 0u;
        // four gfx950 conversions: 8 E4M3 bytes -> 8 fp16 (exact)
        const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
        const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
        const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
        const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
        uint4 out;
        out.x = __builtin_bit_cast(unsigned, h0);
        out.y = __builtin_bit_cast(unsigned, h1);
        out.z = __builtin_bit_cast(unsigned, h2);
        out.w = __builtin_bit_cast(unsigned, h3);
        *reinterpret_cast<uint4*>(lds_scales + r * kScalesPerRow) = out;
      }
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
  // g_a g_b is exact in float64; the product with the accumulator is formed
  // in float64 and rounded to binary32
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

// LDS ring depth of the pipelined kernel (slots of 36 KB); 3 measured ~1.5%
// faster than 4 (fewer loads outstanding per wave).
constexpr int kPipeStages = 3;

// ---------------------------------------------------------------------------
// Pipelined kernel for large, whole-stage shapes (k % 128 == 0).
//
// * Operand stages go from global memory straight into LDS with buffer
//   loads (buffer_load_dwordx4 / _dword ... lds: no staging registers, no
//   LDS store instructions).  Codes are stored unpadded, 64 bytes per row per
//   stage, with the four 16-byte chunks of row r permuted by XOR with
//   ((r >> 1) ^ (r >> 3)) % 4: with it 4, 8 or 16 lanes reading consecutive
//   rows hit distinct banks, and it measured ~1% faster than (r / 4) % 4
//   (which the LDS bank-conflict counter favours; the time did not).
//   Scales stay raw E4M3 (8 bytes per row per stage) and are
//   widened to fp16 when an operand is decoded.
// * NS (3 or 4) LDS slots form a ring: stages kt + 1 .. kt + NS - 1 are in
//   flight or resident while stage kt is consumed, so the next half-stage's
//   fragments are read one half ahead and the next k-step's operands are
//   decoded while the 16 MFMAs of the current k-step issue.  Each stage
//   issues the same loads (past the last stage they repeat it into the slot
//   just freed), A's with the first k-step's MFMAs and B's with the
//   fourth's.  One wait (the fills of the NS - 2 newest stages stay in
//   flight) and one barrier per stage, between its two halves, keep the ring
//   ordered: stage kt + 1, loaded by every wave, has landed before the second
//   half of stage kt reads its first half; and stage kt + NS - 1 goes into
//   the slot of stage kt - 1, whose last reads came before the mid-stage
//   barrier of stage kt - 1.
// * Rows past m or n load a clamped (valid) row; their outputs are never
//   stored.  Offsets within a tile are 32-bit, so the launcher takes this
//   kernel only for k <= 2^22.

constexpr int kPipeRowBytes = kCodeBytes;        // 64, unpadded
constexpr int kPipeScaleBytes = kScalesPerRow;   // 8 raw E4M3 bytes

__device__ __forceinline__ int pipe_chunk(int row, int part) {
  return row * 4 + (part ^ (((row >> 1) ^ (row >> 3)) & 3));
}

// A wave's fragments for one half-stage (4 k-steps, 64 K per lane half):
// per 32-row tile, 16 code bytes and the two raw E4M3 scales of its blocks
// (low 16 bits).  The scales are widened to fp16 only when an operand is
// decoded, so that nothing consumes a fragment right after its LDS read.
template <int T>
struct HalfFrags {
  uint4 code[T];
  unsigned scale[T];

  __device__ __forceinline__ void read(const uint8_t* lds_codes,
                                       const uint8_t* lds_scales,
                                       int row_base, int lane, int half) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = row_base + t * 32 + r;
      // a native vector load: through uint4 the compiler splits it into
      // two 8-byte reads (ds_read2_b64), with 4x the LDS bank conflicts
      typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
      const u32x4v q = *reinterpret_cast<const u32x4v*>(lds_codes + pipe_chunk(row, 2 * h + half) * 16);
      code[t] = make_uint4(q.x, q.y, q.z, q.w);
      scale[t] = *reinterpret_cast<const unsigned short*>(lds_scales + row * kPipeScaleBytes + 4 * h + 2 * half);
    }
  }

  // operand of k-step j (0..3) of this half: 8 codes, block j / 2.
  __device__ __forceinline__ half8_t operand(int t, int j) const {
    const uint4 q = code[t];
    const unsigned w = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    const unsigned wide = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale[t], 1.0f, false));
    const unsigned short sb = (j >> 1) ? static_cast<unsigned short>(wide >> 16)
                                       : static_cast<unsigned short>(wide & 0xFFFFu);
    const _Float16 sv = __builtin_bit_cast(_Float16, sb);
    half2_t sc;
    sc[0] = sv;
    sc[1] = sv;
    return decode8(w, sc);
  }
};

template <int TM, int TN>
struct Operands {
  half8_t a[TM];
  half8_t b[TN];
};

template <int TM, int TN>
__device__ __forceinline__ void decode_step(Operands<TM, TN>& o, const HalfFrags<TM>& fa,
                                            const HalfFrags<TN>& fb, int j) {
#pragma unroll
  for (int i = 0; i < TM; ++i) o.a[i] = fa.operand(i, j);
#pragma unroll
  for (int i = 0; i < TN; ++i) o.b[i] = fb.operand(i, j);
}

// One k-step: TM x TN MFMAs in a zig-zag order (odd rows of tiles walk the B
// tiles backwards, so consecutive MFMAs at a row change share their B
// operand; ~1% faster than a plain row-major order).
template <int TM, int TN>
__device__ __forceinline__ void mfma_step(float16_t (&acc)[TM][TN], const Operands<TM, TN>& o) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int j = (i & 1) ? TN - 1 - jj : jj;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
    }
}

// Scheduling hint for one k-step: alternate one MFMA with a few VALU ops
// (the next k-step's decode, 4 per MFMA on average), so the matrix core and
// the VALU overlap.  5 per MFMA front-loads the decode slightly and measured
// ~1% faster than 4 (6 and 8 slower).
template <int NMFMA, int NVMEM = 0>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
    if (i < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
  }
}

// Per-lane sources of one operand's stage loads: this wave's share of the
// ROWS x 64 code bytes (16-byte chunks, LDS order) and ROWS x 8 scale bytes
// (dwords).  Offsets are relative to the matrix base and exclude k0.
template <int ROWS, int NWAVES>
struct PipeLoader {
  static constexpr int kCodeInsts = ROWS * 4 / 64 / NWAVES;   // per wave
  static constexpr int kScaleInsts = ROWS * 2 / 64 / NWAVES;
  static_assert(ROWS * 4 % (64 * NWAVES) == 0 && ROWS * 2 % (64 * NWAVES) == 0,
                "tile rows must split evenly across the waves");
  static constexpr int kIssues = kCodeInsts + kScaleInsts;   // per wave per stage
  __amdgpu_buffer_rsrc_t code_rsrc, scale_rsrc;
  unsigned code_off[kCodeInsts];
  unsigned scale_off[kScaleInsts];

  // Offsets are 32-bit and relative to the tile's first row, so the tile's
  // rows times k / 2 bytes must stay below 2^32 (the launcher checks k).
  __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* scales,
                                       int64_t row0, int64_t rows, int64_t k,
                                       int wave, int lane) {
    const int64_t kbytes = k / 2, kblocks = k / 16;
    const int last = static_cast<int>(rows - 1 - row0 < ROWS - 1 ? rows - 1 - row0 : ROWS - 1);
    code_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes + row0 * kbytes), 0,
        static_cast<int>((last + 1) * kbytes), 0x00020000);
    scale_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + row0 * kblocks), 0,
        static_cast<int>((last + 1) * kblocks), 0x00020000);
#pragma unroll
    for (int i = 0; i < kCodeInsts; ++i) {
      const int q = (wave * kCodeInsts + i) * 64 + lane;   // LDS chunk
      const int row = q >> 2;
      const int part = (q & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
      code_off[i] = static_cast<unsigned>((row < last ? row : last) * kbytes + part * 16);
    }
#pragma unroll
    for (int j = 0; j < kScaleInsts; ++j) {
      const int d = (wave * kScaleInsts + j) * 64 + lane;  // LDS dword
      const int row = d >> 1;
      scale_off[j] = static_cast<unsigned>((row < last ? row : last) * kblocks + (d & 1) * 4);
    }
  }

  __device__ __forceinline__ void issue(int64_t k0, uint8_t* lds_codes,
                                        uint8_t* lds_scales, int wave) const {
#pragma unroll
    for (int i = 0; i < kCodeInsts; ++i)
      lds_buf16(code_rsrc, lds_codes + (wave * kCodeInsts + i) * 1024, code_off[i],
                static_cast<unsigned>(k0 / 2));
#pragma unroll
    for (int j = 0; j < kScaleInsts; ++j)
      lds_buf4(scale_rsrc, lds_scales + (wave * kScaleInsts + j) * 256, scale_off[j],
               static_cast<unsigned>(k0 / 16));
  }
};

// LDS ring of NS stages; each slot is a separate __shared__ object (holding
// A codes, B codes, A scales, B scales) so that the compiler can prove that
// filling one slot does not alias reads of the others (it would otherwise
// wait for in-flight fills before every read).
template <int NS>
struct Ring {
  uint8_t* a[NS];
  uint8_t* b[NS];
  uint8_t* sa[NS];
  uint8_t* sb[NS];
};

// One K stage (BK = 128) of the pipelined main loop, consuming slot U.
template <int U, int NS, int TM, int TN, int NW, int BM, int BN>
__device__ __forceinline__ void pipe_stage(
    const Ring<NS>& ring, int kt, int nk, float16_t (&acc)[TM][TN],
    Operands<TM, TN>& cur, HalfFrags<TM>& fa, HalfFrags<TN>& fb,
    const PipeLoader<BM, NW>& la, const PipeLoader<BN, NW>& lb,
    const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
    const uint8_t* b_scales, int arow, int brow, int lane, int wave) {
  constexpr int next = U == NS - 1 ? 0 : U + 1;
  constexpr int fill_slot = U == 0 ? NS - 1 : U - 1;   // stage kt - 1's slot
  constexpr int kIssuesA = PipeLoader<BM, NW>::kIssues, kIssuesB = PipeLoader<BN, NW>::kIssues;
  constexpr int kIssues = kIssuesA + kIssuesB;
  // Every stage issues the same loads, so the wait below is one count.  Past
  // the last stage the fill repeats stage nk - 1 into the slot just freed,
  // which no later stage reads.  The slot filled here (stage kt - 1's) was
  // last read in the first half of stage kt - 1, before that stage's barrier.  A's loads go out with the first k-step's
  // MFMAs and B's with the fourth's: spreading them keeps the memory queue
  // from stalling the in-order MFMA issue (~3% faster than one burst).
  const int fs = kt + NS - 1 < nk ? kt + NS - 1 : nk - 1;
  const int64_t k0 = static_cast<int64_t>(fs) * kBK;
  la.issue(k0, ring.a[fill_slot], ring.sa[fill_slot], wave);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half == 1) {
      // The second half starts by reading the first half of stage kt + 1,
      // whose rows other waves loaded: this wave waits for its own loads of
      // stage kt + 1 (those of stages kt + 2 .. kt + NS - 1 may stay in
      // flight), and the barrier then covers everyone's.  Placed here rather
      // than at the end of the stage, the one barrier per stage also orders
      // this stage's reads of its slot before the next stage refills it.
      __builtin_amdgcn_s_waitcnt(kVmcntKeepOf((NS - 2) * kIssues));
      stage_barrier();
    }
    // fragments of the following half-stage (the next stage's first half
    // when this is the second half; a resident slot is read even after the
    // last stage, and never used)
    HalfFrags<TM> na;
    HalfFrags<TN> nb;
    if (half == 0) {
      na.read(ring.a[U], ring.sa[U], arow, lane, 1);
      nb.read(ring.b[U], ring.sb[U], brow, lane, 1);
    } else {
      na.read(ring.a[next], ring.sa[next], arow, lane, 0);
      nb.read(ring.b[next], ring.sb[next], brow, lane, 0);
    }
    // (no scheduling hint here: with LDS waits counted precisely, forcing the
    // reads to the front of the region measured ~4% slower)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Operands<TM, TN> nxt;
      if (j < 3)
        decode_step(nxt, fa, fb, j + 1);
      else
        decode_step(nxt, na, nb, 0);
      if (half == 0 && j == 3) lb.issue(k0, ring.b[fill_slot], ring.sb[fill_slot], wave);
      mfma_step(acc, cur);
      if (half == 0 && j == 0)
        interleave_hint<TM * TN, kIssuesA>();
      else if (half == 0 && j == 3)
        interleave_hint<TM * TN, kIssuesB>();
      else
        interleave_hint<TM * TN, 0>();
      // one scheduling region per k-step: the next half's fragments are
      // consumed only by the last step's decode, so their LDS wait stays there
      __builtin_amdgcn_sched_barrier(0);
      cur = nxt;
    }
    fa = na;
    fb = nb;
  }
}

template <int WM, int WN, int TM, int TN, int OUT, int EPI>
__global__ void __launch_bounds__(WM * WN * 64, 1)
w4a4_gemm_pipelined(const uint8_t* __restrict__ a_codes,
                    const uint8_t* __restrict__ a_scales,
                    const float* __restrict__ a_global, int64_t m,
                    const uint8_t* __restrict__ b_codes,
                    const uint8_t* __restrict__ b_scales,
                    const float* __restrict__ b_global, int64_t n, int64_t k,
                    void* __restrict__ out, int64_t ldo, int tiles_m,
                    int tiles_n) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int NS = kPipeStages;
  static_assert(NS >= 3 && NS <= 4, "ring depth");
  // one LDS object per slot (A codes, B codes, A scales, B scales)
  constexpr int kSlotBytes = (BM + BN) * (kPipeRowBytes + kPipeScaleBytes);
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kSlotBytes], s1[kSlotBytes],
      s2[kSlotBytes], s3[NS > 3 ? kSlotBytes : 16];
  Ring<NS> ring;
  {
    uint8_t* const slots[4] = {s0, s1, s2, s3};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      ring.a[i] = slots[i];
      ring.b[i] = slots[i] + BM * kPipeRowBytes;
      ring.sa[i] = slots[i] + (BM + BN) * kPipeRowBytes;
      ring.sb[i] = slots[i] + (BM + BN) * kPipeRowBytes + BM * kPipeScaleBytes;
    }
  }

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
  const int arow = wm * TM * 32, brow = wn * TN * 32;

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = static_cast<int>(k / kBK);
  PipeLoader<BM, NW> la;
  PipeLoader<BN, NW> lb;
  la.init(a_codes, a_scales, m0, m, k, wave, lane);
  lb.init(b_codes, b_scales, n0, n, k, wave, lane);
  // prologue: stages 0 .. NS-2 into slots 0 .. NS-2 (past the last stage,
  // stage nk - 1 again, which only the unused prefetch after it reads); stage
  // 0 must have landed, the later ones may stay in flight
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    const int64_t k0 = static_cast<int64_t>(st < nk ? st : nk - 1) * kBK;
    la.issue(k0, ring.a[st], ring.sa[st], wave);
    lb.issue(k0, ring.b[st], ring.sb[st], wave);
  }
  constexpr int kIssues = PipeLoader<BM, NW>::kIssues + PipeLoader<BN, NW>::kIssues;
  __builtin_amdgcn_s_waitcnt(kVmcntKeepOf((NS - 2) * kIssues));
  stage_barrier();

  HalfFrags<TM> fa;
  HalfFrags<TN> fb;
  fa.read(ring.a[0], ring.sa[0], arow, lane, 0);
  fb.read(ring.b[0], ring.sb[0], brow, lane, 0);
  Operands<TM, TN> cur;
  decode_step(cur, fa, fb, 0);

  // The stage loop is unrolled by the ring depth so that each stage reads
  // and fills slots known at compile time.
  for (int kt0 = 0; kt0 < nk; kt0 += NS) {
#define NVFP4_PIPE_STAGE(U)                                                    \
    if (kt0 + U < nk)                                                          \
      pipe_stage<U, NS, TM, TN, NW, BM, BN>(ring, kt0 + U, nk, acc, cur, fa, fb, la, lb, \
                                    a_codes, a_scales, b_codes, b_scales,      \
                                    arow, brow, lane, wave);
    NVFP4_PIPE_STAGE(0)
    NVFP4_PIPE_STAGE(1)
    NVFP4_PIPE_STAGE(2)
    if constexpr (NS > 3) { NVFP4_PIPE_STAGE(3) }
#undef NVFP4_PIPE_STAGE
  }
  // no fill may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);

  // the output (often larger than the memory-side cache) is streamed out
  // with non-temporal stores, so that it does not linger there as dirty
  // lines for the next kernel to write back
  const double gab = static_cast<double>(*a_global) * static_cast<double>(*b_global);
  if constexpr (OUT != kOutF32) {
    // bf16, a full tile, a 16-byte aligned output with whole 16-byte pieces
    // per row: each 32-row slice of the wave's tiles goes through the first
    // ring slot (idle once every wave is past the main loop) so that a lane
    // stores 16 contiguous bytes, 4 rows x 256 bytes per wave store; the
    // accumulator layout (2 bytes per lane, 64-byte row pieces) made the
    // stores cost about 2% more of the kernel
    constexpr int kStride = TN * 32 * 2 + 16;   // staged row bytes, padded off the bank period
    static_assert(NW * 32 * kStride <= kSlotBytes, "staging fits one ring slot");
    const bool whole = m0 + BM <= m && n0 + BN <= n &&
                       reinterpret_cast<uintptr_t>(out) % 16 == 0 && ldo % 8 == 0;
    if (whole) {
      __syncthreads();
      uint8_t* stage = s0 + wave * 32 * kStride;
      const int c = lane & 31, h = lane >> 5;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 8 * (e >> 2) + 4 * h + (e & 3);
            const float y = epilogue<EPI>(static_cast<float>(static_cast<double>(acc[i][j][e]) * gab));
            *reinterpret_cast<unsigned short*>(stage + r * kStride + (j * 32 + c) * 2) =
                f32_to_bf16_rne(y);
          }
        __syncthreads();
        constexpr int kPieces = 32 * TN * 4;   // 16-byte pieces of the slice
        static_assert(kPieces % 64 == 0, "whole pieces per lane");
#pragma unroll
        for (int it = 0; it < kPieces / 64; ++it) {
          const int q = it * 64 + lane;
          const int r = q / (TN * 4), cb = (q % (TN * 4)) * 16;
          const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kStride + cb);
          typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 w = {v.x, v.y, v.z, v.w};
          __builtin_nontemporal_store(
              w, reinterpret_cast<u32x4*>(static_cast<unsigned short*>(out) +
                                          (m0 + arow + i * 32 + r) * ldo + n0 + brow + cb / 2));
        }
        __syncthreads();   // the slice is read before the next one is written
      }
      return;
    }
  }
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + brow + j * 32 + col_l;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + arow + i * 32 + 8 * (e >> 2) + row_l + (e & 3);
        if (row < m && col < n) {
          const float y = epilogue<EPI>(static_cast<float>(static_cast<double>(acc[i][j][e]) * gab));
          if constexpr (OUT == kOutF32)
            __builtin_nontemporal_store(y, static_cast<float*>(out) + row * ldo + col);
          else
            __builtin_nontemporal_store(f32_to_bf16_rne(y), static_cast<unsigned short*>(out) + row * ldo + col);
        }
      }
    }
}

template <int WM, int WN, int TM, int TN, int OUT, int EPI>
hipError_t launch_pipelined(const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_global, int64_t m,
                            const uint8_t* b_codes, const uint8_t* b_scales,
                            const float* b_global, int64_t n, int64_t k,
                            void* out, int64_t ldo, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tm = (m + BM - 1) / BM, tn = (n + BN - 1) / BN;
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  w4a4_gemm_pipelined<WM, WN, TM, TN, OUT, EPI>
      <<<static_cast<unsigned>(tm * tn), WM * WN * 64, 0, stream>>>(
          a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, n, k,
          out, ldo, static_cast<int>(tm), static_cast<int>(tn));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny kernel: one operand has at most 64 rows (decode batches, the
// per-head gate projections).  The other operand streams from HBM once, so
// the shape is bandwidth-bound: there is no LDS staging; operands go from
// global memory straight into registers in the MFMA layout.  K is split
// into groups of CPG 64-K chunks (CPG = 4, or 2 when k % 256 != 0); per
// group and row a lane loads its 16 code bytes of each chunk (32 K, its
// half of the chunk) and, in one load, the row's 4 * CPG block scales of
// the whole group (loads touch one cache line per row, so fewer and wider
// scale loads matter more than their bytes).  A workgroup owns one
// TMT x TNT grid of 32 x 32 output tiles; its NWV waves take interleaved
// groups, KG of them in flight per wave, and their partial accumulators
// are summed through LDS, one tile at a time, before the epilogue.  Rows
// past m or n read a clamped valid row and are never stored.
// Requires k % (64 * CPG) == 0.

template <int CPG>
struct SkinnyScales;
template <>
struct SkinnyScales<4> { using type = uint4; };
template <>
struct SkinnyScales<2> { using type = uint2; };

template <int CPG>
struct GroupFrag {
  uint4 code[CPG];                          // 32 K of one row per chunk
  typename SkinnyScales<CPG>::type sc;      // the row's 4 * CPG block scales
};

template <int CPG>
__device__ __forceinline__ void load_group(GroupFrag<CPG>& f, const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales,
                                           int64_t row, int64_t kbytes, int64_t kblocks,
                                           int64_t group, int h) {
  const uint8_t* c = codes + row * kbytes + group * (CPG * 32) + h * 16;
#pragma unroll
  for (int q = 0; q < CPG; ++q) f.code[q] = *reinterpret_cast<const uint4*>(c + q * 32);
  f.sc = *reinterpret_cast<const typename SkinnyScales<CPG>::type*>(
      scales + row * kblocks + group * (CPG * 4));
}

// the two E4M3 scales of chunk q's half h (low byte = first block)
template <int CPG>
__device__ __forceinline__ unsigned group_scale_pair(const GroupFrag<CPG>& f, int q, int h) {
  unsigned w;
  if constexpr (CPG == 4)
    w = q == 0 ? f.sc.x : q == 1 ? f.sc.y : q == 2 ? f.sc.z : f.sc.w;
  else
    w = q == 0 ? f.sc.x : f.sc.y;
  return h ? w >> 16 : w & 0xFFFFu;
}

// operand of k-step j (0..3) of one chunk: codes dword j, block j / 2
__device__ __forceinline__ half8_t chunk_operand(const uint4& code, unsigned sc2, int j) {
  const unsigned w = j == 0 ? code.x : j == 1 ? code.y : j == 2 ? code.z : code.w;
  const unsigned short sb = (j >> 1) ? static_cast<unsigned short>(sc2 >> 16)
                                     : static_cast<unsigned short>(sc2 & 0xFFFFu);
  const _Float16 sv = __builtin_bit_cast(_Float16, sb);
  half2_t s;
  s[0] = sv;
  s[1] = sv;
  return decode8(w, s);
}

// One workgroup's output tile `tile` (row-major over tiles_n tile columns);
// a_g and b_g are the two global scales.
template <int TMT, int TNT, int NWV, int KG, int CPG, int OUT, int EPI>
__device__ __forceinline__ void
skinny_tile(int tile, const uint8_t* __restrict__ a_codes,
            const uint8_t* __restrict__ a_scales, float a_g, int64_t m,
            const uint8_t* __restrict__ b_codes,
            const uint8_t* __restrict__ b_scales, float b_g, int64_t n, int64_t k,
            void* __restrict__ out, int64_t ldo, int tiles_n, EpiArgs ep) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = static_cast<int64_t>(tile / tiles_n) * (32 * TMT);
  const int64_t n0 = static_cast<int64_t>(tile % tiles_n) * (32 * TNT);
  const int64_t kbytes = k / 2, kblocks = k / 16;
  const int64_t ngroups = k / (64 * CPG);

  int64_t arow[TMT], brow[TNT];
#pragma unroll
  for (int i = 0; i < TMT; ++i) {
    const int64_t g = m0 + i * 32 + r;
    arow[i] = g < m ? g : m - 1;
  }
#pragma unroll
  for (int j = 0; j < TNT; ++j) {
    const int64_t g = n0 + j * 32 + r;
    brow[j] = g < n ? g : n - 1;
  }

  float16_t acc[TMT][TNT];
#pragma unroll
  for (int i = 0; i < TMT; ++i)
#pragma unroll
    for (int j = 0; j < TNT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // wave w takes groups w, w + NWV, w + 2 NWV, ...
  for (int64_t g0 = wave; g0 < ngroups; g0 += NWV * KG) {
    GroupFrag<CPG> fa[KG][TMT], fb[KG][TNT];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const int64_t g = g0 + u * NWV;
      const int64_t gg = g < ngroups ? g : ngroups - 1;   // clamped, unused
#pragma unroll
      for (int i = 0; i < TMT; ++i) load_group(fa[u][i], a_codes, a_scales, arow[i], kbytes, kblocks, gg, h);
#pragma unroll
      for (int j = 0; j < TNT; ++j) load_group(fb[u][j], b_codes, b_scales, brow[j], kbytes, kblocks, gg, h);
    }
    // every group is computed; a group past k (clamped load) gets block
    // scale 0, so all its products are exactly 0
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const bool valid = g0 + u * NWV < ngroups;
#pragma unroll
      for (int q = 0; q < CPG; ++q) {
        unsigned sa[TMT], sb[TNT];
#pragma unroll
        for (int i = 0; i < TMT; ++i)
          sa[i] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                      valid ? group_scale_pair(fa[u][i], q, h) : 0u, 1.0f, false));
#pragma unroll
        for (int j = 0; j < TNT; ++j)
          sb[j] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                      valid ? group_scale_pair(fb[u][j], q, h) : 0u, 1.0f, false));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          half8_t av[TMT], bv[TNT];
#pragma unroll
          for (int i = 0; i < TMT; ++i) av[i] = chunk_operand(fa[u][i].code[q], sa[i], ks);
#pragma unroll
          for (int j = 0; j < TNT; ++j) bv[j] = chunk_operand(fb[u][j].code[q], sb[j], ks);
#pragma unroll
          for (int i = 0; i < TMT; ++i)
#pragma unroll
            for (int j = 0; j < TNT; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // sum the waves' partial accumulators, one 32 x 32 tile at a time:
  // red[wave][e][lane]
  __shared__ float red[NWV][16][64];
  const double gab = static_cast<double>(a_g) * static_cast<double>(b_g);
#pragma unroll
  for (int t = 0; t < TMT * TNT; ++t) {
    const int ti = t / TNT, tj = t % TNT;
    if (t > 0) __syncthreads();   // the previous tile's sums are read
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][e][lane] = acc[ti][tj][e];
    __syncthreads();
    // not unrolled: the gate epilogue's code stays out of the tile loop
#pragma unroll 1
    for (int v0 = 0; v0 < 16 * 64; v0 += NWV * 64) {
      const int v = v0 + threadIdx.x;
      if ((16 * 64) % (NWV * 64) == 0 || v < 16 * 64) {
        const int l = v & 63, e = v >> 6;
        float sum = red[0][e][l];
#pragma unroll
        for (int w = 1; w < NWV; ++w) sum += red[w][e][l];
        const int64_t row = m0 + ti * 32 + 8 * (e >> 2) + (l >> 5) * 4 + (e & 3);
        const int64_t col = n0 + tj * 32 + (l & 31);
        if (row < m && col < n) {
          const float y = static_cast<float>(static_cast<double>(sum) * gab);
          if constexpr (EPI == kEpiGdn) {
            if (col < ep.n_beta) {
              static_cast<float*>(out)[row * ldo + col] = gdn_beta(y);
            } else {
              const int64_t j = col - ep.n_beta;
              ep.out2[row * ep.ldo2 + j] = gdn_alpha(y, ep.a_log[j], ep.dt_bias[j]);
            }
          } else if constexpr (OUT == kOutF32) {
            static_cast<float*>(out)[row * ldo + col] = epilogue<EPI>(y);
          } else {
            static_cast<unsigned short*>(out)[row * ldo + col] = f32_to_bf16_rne(epilogue<EPI>(y));
          }
        }
      }
    }
  }
}

template <int TMT, int TNT, int NWV, int KG, int CPG, int OUT, int EPI>
__global__ void __launch_bounds__(NWV * 64)
w4a4_gemm_skinny(const uint8_t* __restrict__ a_codes,
                 const uint8_t* __restrict__ a_scales,
                 const float* __restrict__ a_global, int64_t m,
                 const uint8_t* __restrict__ b_codes,
                 const uint8_t* __restrict__ b_scales,
                 const float* __restrict__ b_global, int64_t n, int64_t k,
                 void* __restrict__ out, int64_t ldo, int tiles_n, EpiArgs ep) {
  skinny_tile<TMT, TNT, NWV, KG, CPG, OUT, EPI>(blockIdx.x, a_codes, a_scales, *a_global, m,
                                                b_codes, b_scales, *b_global, n, k, out, ldo,
                                                tiles_n, ep);
}

template <int TMT, int TNT, int NWV, int KG, int OUT, int EPI>
hipError_t launch_skinny(const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_global, int64_t m,
                         const uint8_t* b_codes, const uint8_t* b_scales,
                         const float* b_global, int64_t n, int64_t k,
                         void* out, int64_t ldo, hipStream_t stream,
                         EpiArgs ep = EpiArgs{}) {
  const int64_t tm = (m + 32 * TMT - 1) / (32 * TMT), tn = (n + 32 * TNT - 1) / (32 * TNT);
  if (tm * tn > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned grid = static_cast<unsigned>(tm * tn);
  if (k % 256 == 0)
    w4a4_gemm_skinny<TMT, TNT, NWV, KG, 4, OUT, EPI><<<grid, NWV * 64, 0, stream>>>(
        a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, n, k, out, ldo,
        static_cast<int>(tn), ep);
  else
    w4a4_gemm_skinny<TMT, TNT, NWV, 2 * KG, 2, OUT, EPI><<<grid, NWV * 64, 0, stream>>>(
        a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, n, k, out, ldo,
        static_cast<int>(tn), ep);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small-M activation quantise + GEMM in one launch.  The limitations
// section (한계) of the arxiv-wiki page on the paper puts a 2-4 % small-batch
// decode loss on the quantisation of the activations; quantising X in the
// GEMM's own launch removes the separate amax, finalise and quantise kernels.  One cooperative launch
// (every workgroup resident at once) in two phases:
//   1. the workgroups that own 16-element blocks of X (256 per workgroup)
//      quantise them exactly as the quantisation kernel does; with a
//      self-calibrated global each of them first takes max |x| over all of
//      X itself (X has at most 64 rows), so no cross-workgroup reduction is
//      needed, and workgroup 0 stores g;
//   2. after one grid barrier (device-scope release and acquire) every
//      workgroup runs skinny GEMM tiles on the codes just written, with the
//      tile shape and K order that w4a4_gemm uses for the same m, so Y is
//      bit-identical to quantise-then-w4a4_gemm.
// Both phases stride over the grid, which the launcher caps at the number
// of co-resident workgroups.

template <int DTYPE, int TMT, int KG, int CPG, int OUT>
__global__ void __launch_bounds__(256)
w4a4_quantize_gemm(const uint8_t* __restrict__ x, int64_t m, int64_t k, int64_t ldx_bytes,
                   int mode, uint8_t* __restrict__ x_codes, uint8_t* __restrict__ x_scales,
                   float* __restrict__ x_global, const uint8_t* __restrict__ w_codes,
                   const uint8_t* __restrict__ w_scales, const float* __restrict__ w_global,
                   int64_t n, void* __restrict__ out, int64_t ldo, int tiles, int tiles_n) {
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const int64_t kb = k / 16, nblocks = m * kb;
  const bool contiguous = ldx_bytes == kb * 16 * kElemBytes;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * 256;
  if (first < nblocks) {   // uniform over the workgroup
    float g;
    if (mode == kModeCompute) {
      unsigned mx = 0;
      for (int64_t i = threadIdx.x; i < nblocks; i += 256) {
        float v[16];
        mx = max(mx, load_block<DTYPE>(block_src<DTYPE>(x, i, contiguous, kb, ldx_bytes), v));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
        mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
      __shared__ unsigned part[4];
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
      __syncthreads();
      mx = max(max(part[0], part[1]), max(part[2], part[3]));
      g = global_from_amax(__uint_as_float(mx));
      if (blockIdx.x == 0 && threadIdx.x == 0) *x_global = g;
    } else {
      g = *x_global;
    }
    bool g_ok;
    const float inv6g = recip_6g(g, &g_ok);
    __shared__ __attribute__((aligned(16))) float lds_rows[256 * kRowFloats];
    float* row = lds_rows + threadIdx.x * kRowFloats;
    for (int64_t b = first + threadIdx.x; b < nblocks; b += stride)
      quantize_one<DTYPE>(block_src<DTYPE>(x, b, contiguous, kb, ldx_bytes), b, g, inv6g, g_ok,
                          x_codes, x_scales, row);
  }
  // every code, scale and the global of X are written and visible
  // device-wide after the barrier
  cooperative_groups::this_grid().sync();
  const float a_g = __hip_atomic_load(x_global, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float b_g = *w_global;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    if (tile != static_cast<int>(blockIdx.x)) __syncthreads();   // LDS of the previous tile is free
    skinny_tile<TMT, 1, 4, KG, CPG, OUT, kEpiNone>(tile, x_codes, x_scales, a_g, m, w_codes,
                                                  w_scales, b_g, n, k, out, ldo, tiles_n,
                                                  EpiArgs{});
  }
}

// Co-resident workgroups of `kernel` on the current device (0 if the
// runtime cannot tell), cached per device in the caller's `cache`.
template <typename Kernel>
int resident_workgroups(Kernel kernel, int block, std::atomic<int> (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int total = per_cu * cus;
  if (dev < 64) cache[dev].store(total, std::memory_order_relaxed);
  return total;
}

template <int DTYPE, int TMT, int KG, int CPG, int OUT>
hipError_t launch_quantize_gemm_cfg(const void* x, int64_t m, int64_t k, int64_t ldx,
                                    int mode, uint8_t* x_codes, uint8_t* x_scales,
                                    float* x_global, const uint8_t* w_codes,
                                    const uint8_t* w_scales, const float* w_global, int64_t n,
                                    void* out, int64_t ldo, hipStream_t stream) {
  auto kernel = w4a4_quantize_gemm<DTYPE, TMT, KG, CPG, OUT>;
  const int64_t tm = (m + 32 * TMT - 1) / (32 * TMT), tn = (n + 31) / 32;
  const int64_t tiles = tm * tn;
  const int64_t qwgs = (m * (k / 16) + 255) / 256;
  static std::atomic<int> resident_cache[64];   // one per kernel instance
  const int resident = resident_workgroups(kernel, 256, resident_cache);
  if (resident < 1) return hipErrorCooperativeLaunchTooLarge;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  int64_t grid = tiles > qwgs ? tiles : qwgs;
  if (grid > resident) grid = resident;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  int64_t ldx_bytes = ldx * (DTYPE == kDtypeF32 ? 4 : 2);
  int tiles_i = static_cast<int>(tiles), tn_i = static_cast<int>(tn);
  void* args[] = {&xb, &m, &k, &ldx_bytes, &mode, &x_codes, &x_scales, &x_global, &w_codes,
                  &w_scales, &w_global, &n, &out, &ldo, &tiles_i, &tn_i};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel),
                                    dim3(static_cast<unsigned>(grid)), dim3(256), args, 0,
                                    stream);
}

template <int DTYPE, int OUT>
hipError_t launch_quantize_gemm_k(const void* x, int64_t m, int64_t k, int64_t ldx, int mode,
                                  uint8_t* x_codes, uint8_t* x_scales, float* x_global,
                                  const uint8_t* w_codes, const uint8_t* w_scales,
                                  const float* w_global, int64_t n, void* out, int64_t ldo,
                                  hipStream_t stream) {
  // the same tile shapes and K groups as the skinny dispatch of w4a4_gemm
#define NVFP4_QG_ARGS x, m, k, ldx, mode, x_codes, x_scales, x_global, w_codes, w_scales, \
                      w_global, n, out, ldo, stream
  if (m <= 32) {
    if (k % 256 == 0) return launch_quantize_gemm_cfg<DTYPE, 1, 1, 4, OUT>(NVFP4_QG_ARGS);
    return launch_quantize_gemm_cfg<DTYPE, 1, 2, 2, OUT>(NVFP4_QG_ARGS);
  }
  if (k % 256 == 0) return launch_quantize_gemm_cfg<DTYPE, 2, 1, 4, OUT>(NVFP4_QG_ARGS);
  return launch_quantize_gemm_cfg<DTYPE, 2, 2, 2, OUT>(NVFP4_QG_ARGS);
#undef NVFP4_QG_ARGS
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
#define NVFP4_ARGS a_codes, a_scales, a_global, m, b_codes, b_scales, b_global, \
                   n, k, out, ldo, stream
  if constexpr (ALIGNED) {
    // one operand of at most 64 rows: the streaming kernel (whole 128-K
    // chunks, 32-bit offsets within a workgroup's rows)
    if (gemm_stream_fits(m, n, k))
      return launch_gemm_stream(a_codes, a_scales, a_global, m, b_codes, b_scales, b_global,
                                n, k, out, OUT, ldo, EPI, stream);
    // k % 128 == 0 here, so the skinny kernel's groups of 2 or 4 64-K
    // chunks tile k
    if (m <= 32) return launch_skinny<1, 1, 4, 1, OUT, EPI>(NVFP4_ARGS);
    if (m <= 64) return launch_skinny<2, 1, 4, 1, OUT, EPI>(NVFP4_ARGS);
    if (n <= 32) return launch_skinny<1, 1, 4, 1, OUT, EPI>(NVFP4_ARGS);
    if (n <= 64) return launch_skinny<2, 2, 4, 1, OUT, EPI>(NVFP4_ARGS);
    // the pipelined kernels address a tile with 32-bit offsets
    if (k <= (int64_t{1} << 22)) return launch_pipelined<2, 2, 4, 4, OUT, EPI>(NVFP4_ARGS);
  }
  return launch_cfg<2, 2, 4, 4, ALIGNED, OUT, EPI>(NVFP4_ARGS);
#undef NVFP4_ARGS
}

template <int OUT, int EPI>
hipError_t dispatch_align(const uint8_t* a_codes, const uint8_t* a_scales,
                          const float* a_global, int64_t m,
                          const uint8_t* b_codes, const uint8_t* b_scales,
                          const float* b_global, int64_t n, int64_t k,
                          void* out, int64_t ldo, hipStream_t stream) {
  // whole stages (k % 128 == 0; the caller has checked 16-byte aligned
  // code and scale arrays): unconditional 16-byte code loads and wide (8- or
  // 16-byte) scale loads; ragged k takes the guarded, byte-wise path
  if (k % kBK == 0)
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

hipError_t launch_quantize_gemm(const void* x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                                int mode, uint8_t* x_codes, uint8_t* x_scales,
                                float* x_global, const uint8_t* w_codes,
                                const uint8_t* w_scales, const float* w_global, int64_t n,
                                void* out, int out_dtype, int64_t ldo, hipStream_t stream) {
  // the GEMM phase runs the tiles w4a4_gemm runs for the same shape
  if (gemm_stream_fits(m, n, k))
    return launch_quantize_gemm_stream(x, x_dtype, m, k, ldx, mode, x_codes, x_scales, x_global,
                                       w_codes, w_scales, w_global, n, out, out_dtype, ldo,
                                       stream);
#define NVFP4_QG_ARGS x, m, k, ldx, mode, x_codes, x_scales, x_global, w_codes, w_scales, \
                      w_global, n, out, ldo, stream
  if (x_dtype == kDtypeF32) {
    if (out_dtype == kOutF32) return launch_quantize_gemm_k<0, 0>(NVFP4_QG_ARGS);
    return launch_quantize_gemm_k<0, 1>(NVFP4_QG_ARGS);
  }
  if (out_dtype == kOutF32) return launch_quantize_gemm_k<1, 0>(NVFP4_QG_ARGS);
  return launch_quantize_gemm_k<1, 1>(NVFP4_QG_ARGS);
#undef NVFP4_QG_ARGS
}

hipError_t launch_gdn_gates(const uint8_t* x_codes, const uint8_t* x_scales,
                            const float* x_global, int64_t m,
                            const uint8_t* w_codes, const uint8_t* w_scales,
                            const float* w_global, int64_t n_beta, int64_t n_alpha,
                            int64_t k, const float* a_log, const float* dt_bias,
                            float* beta_out, int64_t ld_beta, float* alpha_out,
                            int64_t ld_alpha, hipStream_t stream) {
  const int64_t n = n_beta + n_alpha;
  if (gdn_stream_fits(m, n, k))
    return launch_gdn_stream(x_codes, x_scales, x_global, m, w_codes, w_scales, w_global, n_beta,
                             n_alpha, k, a_log, dt_bias, beta_out, ld_beta, alpha_out, ld_alpha,
                             stream);
  const EpiArgs ep{a_log, dt_bias, n_beta, alpha_out, ld_alpha};
#define NVFP4_GDN_ARGS x_codes, x_scales, x_global, m, w_codes, w_scales, w_global, n, k, \
                       beta_out, ld_beta, stream, ep
  if (n <= 64) return launch_skinny<2, 2, 4, 1, kOutF32, kEpiGdn>(NVFP4_GDN_ARGS);
  if (n <= 128) return launch_skinny<2, 4, 8, 1, kOutF32, kEpiGdn>(NVFP4_GDN_ARGS);
  return launch_skinny<1, 8, 4, 1, kOutF32, kEpiGdn>(NVFP4_GDN_ARGS);
#undef NVFP4_GDN_ARGS
}

}  // namespace nvfp4
