// Fused-group scale harmonisation for gfx950.
//
// Serving kernels that fuse several modules (qkv|z, b|a of a Gated DeltaNet
// layer) into one GEMM apply one global scale to the fused weight, while a
// per-module calibrated checkpoint carries one global per module.  The fix
// (arxiv-wiki page on "Why Gated DeltaNet Survives 4-Bit Quantization",
// sections 접근 방법 and 개발자 관점; the abstract on the paper's listing page)
// rewrites the globals to one shared value and folds each module's ratio
// into its E4M3 block scales.  Shared global: g* = max_i g_i (then no folded
// scale can exceed 448).  New scale: RNE_SAT_E4M3(e4m3(s) g_i / g*), exact;
// modules with g_i == g* keep their bytes; codes are not touched.
//
// 4 scale bytes per lane.  The candidate code comes from the gfx950
// fp32 -> E4M3 conversion of e4m3(s) * g_i * (1 / g*) scaled by 1 -+ 2^-18
// (the product is within 2^-21 of the exact quotient); equal results prove
// the rounding, otherwise the two codes are adjacent and one exact float64
// comparison with their midpoint decides.  A shared global near the ends of
// the binary32 range takes an all-float64 path.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

// first scale byte of each module, and the total
struct Offsets {
  int64_t first[kMaxModules + 1];
};

// The refolded code of scale byte s of a module with global gi (gi < g*).
__device__ __forceinline__ unsigned refold(unsigned s, float gi, float gstar, float rgstar,
                                           bool fast) {
  const double den = static_cast<double>(gstar);
  if (fast) {
    // 0 <= g_i / g* <= 1; where the quotient is below the binary32 normal
    // range, so far below the smallest E4M3 midpoint 2^-10, both candidates
    // are 0 as the exact rounding is
    const float q = e4m3_f32(s) * (gi * rgstar);
    const float lo = fminf(q * (1.0f - 0x1p-18f), 448.0f);
    const float hi = fminf(q * (1.0f + 0x1p-18f), 448.0f);
    const unsigned pk = static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0, false));
    unsigned c = pk & 0xFFu;
    if (((pk ^ (pk >> 8)) & 0xFFu) != 0) {
      // codes c and c + 1: the midpoint (<= 5 significant bits) times g*
      // is exact in float64, as is num; ties go to the even code
      const double num = e4m3_value(s) * static_cast<double>(gi);
      const double t = 0.5 * (e4m3_value(c) + e4m3_value(c + 1u)) * den;
      c = (num > t || (num == t && (c & 1u))) ? c + 1u : c;
    }
    return c;
  }
  const double num = e4m3_value(s) * static_cast<double>(gi);   // exact
  return e4m3_settle(e4m3_candidate(num / den), num, den);
}

// BPL consecutive scale bytes per lane, one load and store of BPL bytes
// (the array is 16-byte aligned; only the lane holding the array's last,
// partial word goes byte by byte); a lane's bytes may span module
// boundaries, so the module is advanced per byte.
template <int BPL>
__global__ void __launch_bounds__(256)
harmonize_kernel(uint8_t* __restrict__ scales, int64_t total, Offsets offs, int n_modules,
                 const float* __restrict__ module_globals,
                 float* __restrict__ shared_global) {
  float gstar = module_globals[0];
  for (int i = 1; i < n_modules; ++i) gstar = fmaxf(gstar, module_globals[i]);
  const int64_t lane = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (lane == 0) *shared_global = gstar;
  const int64_t i0 = lane * BPL;
  if (i0 >= total) return;
  const bool fast = gstar >= 0x1p-100f && gstar <= 0x1p100f;
  const float rgstar = fast ? __builtin_amdgcn_rcpf(gstar) : 0.0f;
  int mod = 0;
  while (mod + 1 < n_modules && i0 >= offs.first[mod + 1]) ++mod;
  float gi = module_globals[mod];
  int64_t next = mod + 1 < n_modules ? offs.first[mod + 1] : total;
  constexpr int kWords = BPL / 4;
  const bool vec = i0 + BPL <= total;
  unsigned w[kWords];
#pragma unroll
  for (int q = 0; q < kWords; ++q) w[q] = 0u;
  if (vec) {
#pragma unroll
    for (int q = 0; q < kWords; ++q) w[q] = reinterpret_cast<const unsigned*>(scales + i0)[q];
  }
  bool changed = false;
#pragma unroll
  for (int j = 0; j < BPL; ++j) {
    if (i0 + j >= total) break;
    if (i0 + j >= next) {
      while (mod + 1 < n_modules && i0 + j >= offs.first[mod + 1]) ++mod;
      gi = module_globals[mod];
      next = mod + 1 < n_modules ? offs.first[mod + 1] : total;
    }
    if (gi == gstar) continue;   // also covers g* = 0
    const unsigned s = vec ? (w[j >> 2] >> (8 * (j & 3))) & 0xFFu : scales[i0 + j];
    const unsigned c = refold(s, gi, gstar, rgstar, fast);
    if (vec) {
      w[j >> 2] = (w[j >> 2] & ~(0xFFu << (8 * (j & 3)))) | (c << (8 * (j & 3)));
      changed = true;
    } else {
      scales[i0 + j] = static_cast<uint8_t>(c);
    }
  }
  if (changed) {
#pragma unroll
    for (int q = 0; q < kWords; ++q) reinterpret_cast<unsigned*>(scales + i0)[q] = w[q];
  }
}

}  // namespace

hipError_t launch_harmonize(uint8_t* scales, int64_t k,
                            const int64_t* row_offsets, int n_modules,
                            const float* module_globals,
                            float* shared_global, hipStream_t stream) {
  Offsets offs{};
  const int64_t kb = k / 16;
  for (int i = 0; i <= n_modules; ++i) offs.first[i] = row_offsets[i] * kb;
  const int64_t total = offs.first[n_modules];
  // 4 bytes per lane: 13.7 us on a 17536 x 320-byte group against 18.7 us
  // with one byte per lane (28 us with a float64 division per byte); 16
  // bytes per lane measured the same as 4
  constexpr int kBpl = 4;
  const int64_t lanes = (total + kBpl - 1) / kBpl;
  const int64_t blocks = lanes > 0 ? (lanes + 255) / 256 : 1;
  harmonize_kernel<kBpl><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      scales, total, offs, n_modules, module_globals, shared_global);
  return hipGetLastError();
}

}  // namespace nvfp4
