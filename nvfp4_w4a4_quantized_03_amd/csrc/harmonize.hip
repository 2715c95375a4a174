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
// One lane per scale byte; the work is a few MB of bytes, latency-bound.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "formats.h"
#include "internal.h"

namespace nvfp4 {
namespace {

struct Offsets {
  int64_t row[kMaxModules + 1];
};

__global__ void __launch_bounds__(256)
harmonize_kernel(uint8_t* __restrict__ scales, int64_t kb, int64_t total,
                 Offsets offs, int n_modules,
                 const float* __restrict__ module_globals,
                 float* __restrict__ shared_global) {
  float gstar = module_globals[0];
  for (int i = 1; i < n_modules; ++i) gstar = fmaxf(gstar, module_globals[i]);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx == 0) *shared_global = gstar;
  if (idx >= total) return;
  const int64_t row = idx / kb;
  int mod = 0;
  while (mod + 1 < n_modules && row >= offs.row[mod + 1]) ++mod;
  const float gi = module_globals[mod];
  if (gi == gstar) return;
  const unsigned s = scales[idx];
  const double num = e4m3_value(s) * static_cast<double>(gi);   // exact
  const double den = static_cast<double>(gstar);
  scales[idx] = static_cast<uint8_t>(e4m3_settle(e4m3_candidate(num / den), num, den));
}

}  // namespace

hipError_t launch_harmonize(uint8_t* scales, int64_t k,
                            const int64_t* row_offsets, int n_modules,
                            const float* module_globals,
                            float* shared_global, hipStream_t stream) {
  Offsets offs{};
  for (int i = 0; i <= n_modules; ++i) offs.row[i] = row_offsets[i];
  const int64_t kb = k / 16;
  const int64_t total = row_offsets[n_modules] * kb;
  const int64_t blocks = total > 0 ? (total + 255) / 256 : 1;
  harmonize_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      scales, kb, total, offs, n_modules, module_globals, shared_global);
  return hipGetLastError();
}

}  // namespace nvfp4
