// NVFP4 quantisation for gfx950: tensor amax -> FP32 global, block amax ->
// E4M3 scale, E2M1 encode + pack.  The per-element encoding (exact rounding
// decisions) is in quant_device.h.
//
// Work split: one lane per 16-element block; a wave streams 64 consecutive
// blocks (2 KiB of bf16), so loads and the 8-byte code stores coalesce.  The
// kernel is HBM-bound; the VALU work per element is kept to a few ops.  (Two
// lanes per block, 16 contiguous bytes each, with the block maximum
// exchanged over DPP and 4 scale bytes gathered per dword store, measured
// 20% slower: the per-block scale work and exchanges add more VALU than the
// access pattern saves.)  The self-calibration pass reads half blocks, 16
// contiguous bytes per lane.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"
#include "quant_device.h"

namespace nvfp4 {
namespace {

// One block per lane: a wave's loads cover 64 consecutive blocks (2 KiB of
// bf16).  Many short-lived waves per CU overlap the loads of some with the
// encoding work of others.  A grid that covers every block (the launcher's
// normal case) takes a straight-line body; the grid-stride loop only serves
// grids capped at the launch limit.
template <int DTYPE>
__global__ void __launch_bounds__(256)
quantize_kernel(const uint8_t* __restrict__ x, int64_t nblocks, int64_t kb,
                int64_t ldx_bytes, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales, const float* __restrict__ global) {
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const float g = *global;
  bool g_ok;
  const float inv6g = recip_6g(g, &g_ok);
  const bool contiguous = ldx_bytes == kb * 16 * kElemBytes;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  __shared__ __attribute__((aligned(16))) float lds_rows[256 * kRowFloats];
  float* row = lds_rows + threadIdx.x * kRowFloats;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (stride >= nblocks && contiguous) {
    if (b0 < nblocks)
      quantize_one<DTYPE>(x + b0 * (16 * kElemBytes), b0, g, inv6g, g_ok, codes, scales, row);
    return;
  }
  for (int64_t b = b0; b < nblocks; b += stride)
    quantize_one<DTYPE>(block_src<DTYPE>(x, b, contiguous, kb, ldx_bytes), b, g, inv6g,
                        g_ok, codes, scales, row);
}

// ---- self-calibrated global: amax over the tensor, then g = amax / 2688 --

__global__ void amax_init_kernel(unsigned* bits) { *bits = 0u; }

// max |x| over the tensor: per trip a wave reads 64 consecutive blocks,
// lane 2j + h half h of blocks j and j + 32 (16 contiguous bytes of bf16 or
// 32 of fp32 each); one atomic per workgroup.  Workgroups of 512 lanes: at
// the cap of 512 workgroups that is 4096 waves, which a cold 335 MB read
// needs (32768 x 5120 bf16: 50.7 us against 63 us with 256 lanes, the same
// number of atomics).
constexpr int kAmaxThreads = 512;
template <int DTYPE>
__global__ void __launch_bounds__(kAmaxThreads)
amax_kernel(const uint8_t* __restrict__ x, int64_t nblocks, int64_t kb,
            int64_t ldx_bytes, unsigned* __restrict__ out_bits) {
  constexpr int kHalfBytes = DTYPE == kDtypeF32 ? 32 : 16;
  const bool contiguous = ldx_bytes == kb * 2 * kHalfBytes;
  const int lane = threadIdx.x & 63, h = lane & 1;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x / 64);
  const int64_t wave0 = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  unsigned mx = 0;
  for (int64_t w = wave0; w * 64 < nblocks; w += waves) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t b = w * 64 + u * 32 + (lane >> 1);
      const int64_t bb = b < nblocks ? b : nblocks - 1;   // past the end: the last block again
      const uint8_t* src = contiguous ? x + bb * (2 * kHalfBytes)
                                      : block_src<DTYPE>(x, bb, false, kb, ldx_bytes);
      float v[8];
      mx = max(mx, load_half<DTYPE>(src + h * kHalfBytes, v));
    }
  }
  // wave reduction, then one atomic per workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
  __shared__ unsigned part[kAmaxThreads / 64];
  const int wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = part[0];
    for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) t = max(t, part[i]);
    atomicMax(out_bits, t);
  }
}

// g = RNE_fp32(amax / 2688), in place
__global__ void amax_finalize_kernel(float* global) {
  *global = global_from_amax(__uint_as_float(*reinterpret_cast<unsigned*>(global)));
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
    // at most 512 workgroups: each ends with one atomic on the same word, and
    // more of them (2048) measured slower
    const int64_t want = (nblocks + kAmaxThreads - 1) / kAmaxThreads;
    const unsigned grid = static_cast<unsigned>(want < 512 ? want : 512);
    if (x_dtype == kDtypeF32)
      amax_kernel<0><<<grid, kAmaxThreads, 0, stream>>>(xb, nblocks, kb, ldx_bytes, bits);
    else
      amax_kernel<1><<<grid, kAmaxThreads, 0, stream>>>(xb, nblocks, kb, ldx_bytes, bits);
    amax_finalize_kernel<<<1, 1, 0, stream>>>(global);
  }
  // one block per lane (a one-shot grid measured faster than a resident
  // grid-stride one); the loop inside covers grids capped at 2^31 - 1
  const int64_t want = (nblocks + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 0x7FFFFFFF ? want : 0x7FFFFFFF);
  if (x_dtype == kDtypeF32)
    quantize_kernel<0><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes,
                                                 codes, scales, global);
  else
    quantize_kernel<1><<<grid, 256, 0, stream>>>(xb, nblocks, kb, ldx_bytes,
                                                 codes, scales, global);
  return hipGetLastError();
}

}  // namespace nvfp4
