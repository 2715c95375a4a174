// Streaming W4A4 GEMM for gfx950: one operand ("L") has at most 64 rows,
// the other ("S") streams from HBM once -- decode batches (L = the
// activations, S = the weight) and the per-head gate projections (L = the
// weight, S = the activations).  Y = g_a g_b * A_hat B_hat^T on NVFP4
// operands as defined by the explainer page "論文解説: Gated DeltaNet はなぜ4bit
// 量子化に耐えるのか", section 前提1 (both GEMM operands 4-bit), with the gate
// epilogues of its section 前提2.
//
// The shape is bandwidth-bound (the arxiv-wiki page on the paper, section
// 주요 결과, puts decode throughput on weight streaming), so the kernel is
// built around the memory system:
//   * A workgroup owns SR rows of S and all (up to 64) rows of L, over the
//     whole of K; the grid is one workgroup per SR-row slice of S.
//   * K goes in stages of KS (512 or 256).  A stage's bytes -- the SR rows'
//     codes and scales of S, the L rows' codes and scales -- are loaded with
//     16-byte buffer loads into a register ring two stages deep, then
//     written to one of two LDS slots.  Consecutive lanes load consecutive
//     16-byte pieces of a row, so every load instruction reads whole
//     128-byte lines (the MFMA-layout loads of 32 rows x 32 bytes measured
//     2-4x slower).  Rows past the matrix and the padding of the scale
//     regions read past the buffer resource's range and land as zeros.
//   * One wait and one workgroup barrier per stage order the LDS slots.
//   * Each wave owns KS/32/NW of a stage's 16x16x32 k-steps: it reads its
//     code dwords and scale bytes of every S and L tile from LDS, decodes
//     them exactly to fp16 (one conversion per two codes, one packed
//     multiply by the block scale) and issues ST x LT
//     v_mfma_f32_16x16x32_f16.  Every fragment is decoded once per
//     workgroup.  Code rows in LDS are XOR-swizzled in 16-byte pieces so
//     that the 16 rows of a fragment read hit distinct banks.
//   * The waves' partial sums meet in LDS after the last stage; the
//     epilogue applies g_a g_b (in float64, rounded to binary32), the
//     optional gate and the fp32 / bf16 store.
// K order: lane (r, q) of a 16x16x32 step j of chunk c (128 K) holds the
// 8 codes at K = 128 c + 32 q + 8 j .. +7 of its row, for A and B alike, so
// the MFMA sums exactly the products of one K range (a permutation of the
// K order inside the chunk, which leaves the dot product unchanged).
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "gemm_common.h"
#include "internal.h"
#include "quant_device.h"

namespace nvfp4 {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
// A native 8-byte vector: read through the uint2 struct, the compiler
// splits the LDS read into two halves and may drop the second half's
// alias information, after which every LDS read waits for every ring fill
// in flight.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// LDS layout of one ring slot for SR rows of S and LR rows of L at KS K per
// stage: [S codes SR x KS/2][S scales, padded to whole KiB]
// [L codes LR x KS/2][L scales, padded].  Each region is filled by whole
// 1 KiB load instructions (64 lanes x 16 bytes).
template <int SR, int LR, int KS>
struct StreamLayout {
  static constexpr int kCodeRow = KS / 2;       // code bytes per row per stage
  static constexpr int kScaleRow = KS / 16;     // scale bytes per row per stage
  static constexpr int kPieces = kCodeRow / 16; // 16-byte pieces per code row
  static constexpr int kInstSC = SR * kCodeRow / 1024;
  static constexpr int kInstSS = (SR * kScaleRow + 1023) / 1024;
  static constexpr int kInstLC = LR * kCodeRow / 1024;
  static constexpr int kInstLS = (LR * kScaleRow + 1023) / 1024;
  static constexpr int kInst = kInstSC + kInstSS + kInstLC + kInstLS;
  static constexpr int kOffSS = kInstSC * 1024;
  static constexpr int kOffLC = kOffSS + kInstSS * 1024;
  static constexpr int kOffLS = kOffLC + kInstLC * 1024;
  static constexpr int kSlot = kInst * 1024;
  static_assert(SR * kCodeRow % 1024 == 0 && LR * kCodeRow % 1024 == 0,
                "code regions must be whole load instructions");
};

// Piece slot of global piece p of code row r (XOR swizzle; bank-conflict
// free for 16 consecutive rows reading the same piece).
template <int KS>
__device__ __forceinline__ int stream_slot(int r, int p) {
  if constexpr (KS == 512)
    return p ^ (r & 15);          // 256-byte rows: 16 pieces
  else
    return p ^ ((r >> 1) & 7);    // 128-byte rows: 8 pieces
}

// A raw buffer resource over [base, base + bytes) whose fields are known to
// be uniform over the wave (read from the first lane), so that it stays in
// scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint8_t* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  const uint8_t* p = reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, n, 0x00020000);
}

// This wave's share of a stage's load instructions: for each, the buffer
// resource of its region (the S or L matrix's codes or scales, from this
// workgroup's first row; rows past the matrix fall outside the range and
// read as zeros), the lane's offset in the region's rows, the stride of the
// stage's K offset, and the LDS destination.  Everything but the stage
// offset is fixed at init, so a stage costs one scalar multiply per load.
template <int SR, int LR, int KS, int NW>
struct StreamLoader {
  using L = StreamLayout<SR, LR, KS>;
  static constexpr int kPerWave = (L::kInst + NW - 1) / NW;
  __amdgpu_buffer_rsrc_t rsrc[kPerWave];
  unsigned voff[kPerWave];
  unsigned stride[kPerWave];   // KS / 2 (codes) or KS / 16 (scales)
  unsigned lds[kPerWave];      // byte offset in the slot (wave-uniform)
  int count;                   // this wave's instructions per stage (wave-uniform)

  // kbytes = k / 2, kblocks = k / 16; s_rows / l_rows rows of this
  // workgroup are inside the matrices
  __device__ __forceinline__ void init(const uint8_t* s_codes, const uint8_t* s_scales,
                                       int64_t s_rows, const uint8_t* l_codes,
                                       const uint8_t* l_scales, int64_t l_rows,
                                       int64_t kbytes, int64_t kblocks, int wave, int lane) {
    count = 0;
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int i = wave + j * NW;   // instruction index in the stage
      if (i < L::kInst) ++count;
      const int ii = i < L::kInst ? i : L::kInst - 1;   // (past the count: never stored)
      lds[j] = static_cast<unsigned>(ii) * 1024u;
      if (ii < L::kInstSC || (ii >= L::kInstSC + L::kInstSS &&
                              ii < L::kInstSC + L::kInstSS + L::kInstLC)) {
        // code region: row r, LDS piece slot `slot` holds global piece
        // slot ^ swizzle(r)
        const bool is_s = ii < L::kInstSC;
        const int q = (is_s ? ii : ii - L::kInstSC - L::kInstSS) * 64 + lane;
        const int r = q / L::kPieces, slot = q % L::kPieces;
        const int p = stream_slot<KS>(r, slot);
        rsrc[j] = uniform_rsrc(is_s ? s_codes : l_codes, (is_s ? s_rows : l_rows) * kbytes);
        voff[j] = static_cast<unsigned>(r * kbytes + p * 16);
        stride[j] = KS / 2;
      } else {
        // scale region: row r's KS/16 bytes, two or one 16-byte pieces;
        // lanes past the region read past any range (zeros)
        const bool is_s = ii < L::kInstSC + L::kInstSS;
        const int q = (is_s ? ii - L::kInstSC : ii - L::kInstSC - L::kInstSS - L::kInstLC) * 64 + lane;
        constexpr int kPer = L::kScaleRow / 16;   // pieces per row (2 or 1)
        const int r = q / kPer, part = q % kPer;
        const int rows = is_s ? SR : LR;
        rsrc[j] = uniform_rsrc(is_s ? s_scales : l_scales, (is_s ? s_rows : l_rows) * kblocks);
        voff[j] = r < rows ? static_cast<unsigned>(r * kblocks + part * 16) : 0x80000000u;
        stride[j] = KS / 16;
      }
      // a slot past this wave's count reads outside the range (zeros, no
      // memory access)
      if (i >= L::kInst) voff[j] = 0x80000000u;
    }
  }

  // this wave's pieces of stage `stage` into registers (16 bytes a lane per
  // instruction, consecutive lanes consecutive bytes of a row).  Every wave
  // issues kPerWave loads (past its count, one outside the buffer that is
  // never stored), so that no load depends on a runtime condition.  Stages
  // are whole (k % KS == 0), so a valid row's offset plus the stage offset
  // stays inside that row.  A stage past the last one (stage >= nst) is
  // loaded at kPastEnd: every offset is then beyond the range of its
  // resource (at most 128 rows x 2^21 bytes < 2^30), so the load returns
  // zeros without a memory access, and its value is never used.
  static constexpr unsigned kPastEnd = 0x40000000u;
  __device__ __forceinline__ void load(int stage, int nst, u32x4 (&v)[kPerWave]) const {
    const int st = __builtin_amdgcn_readfirstlane(stage);
#pragma unroll
    for (int j = 0; j < kPerWave; ++j)
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc[j], voff[j], st < nst ? static_cast<unsigned>(st) * stride[j] : kPastEnd, 0);
  }

  // ... and from registers into the LDS slot (the layout the fragment reads
  // expect: piece i of the stage at slot byte 1024 * instruction + 16 * lane)
  __device__ __forceinline__ void store(const u32x4 (&v)[kPerWave], uint8_t* slot, int lane) const {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j)
      if (j < count) *reinterpret_cast<u32x4*>(slot + lds[j] + 16 * lane) = v[j];
  }
};

// 8 codes (dword) of one fragment with its fp16 block scale -> MFMA operand
__device__ __forceinline__ half8_t stream_operand(unsigned codes, unsigned scale_byte) {
  const half2_t s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scale_byte, 1.0f, false);
  half2_t sc;
  sc[0] = s2[0];
  sc[1] = s2[0];
  return decode8(codes, sc);
}

// The workgroup's fragments of one stage: each wave's kMine k-steps of
// every S and L tile, decoded and multiplied into the accumulators.
template <int SR, int LR, int KS, int KMINE>
__device__ __forceinline__ void stream_compute(const uint8_t* base,
                                               float4_t (&acc)[(SR + 15) / 16][LR / 16],
                                               int chunk, int dw0, int r, int q) {
  using Lay = StreamLayout<SR, LR, KS>;
  constexpr int ST = (SR + 15) / 16, LT = LR / 16;
  const int piece = 4 * chunk + q;   // global 16-byte piece of this lane
  const int sb = 8 * chunk + 2 * q + (dw0 >> 1);   // block of these dwords
  unsigned sc[ST][KMINE], ssc[ST], lc[LT][KMINE], lsc[LT];
#pragma unroll
  for (int t = 0; t < ST; ++t) {
    const int row = t * 16 + r;
    const uint8_t* p = base + row * Lay::kCodeRow + stream_slot<KS>(row, piece) * 16 + dw0 * 4;
    if constexpr (KMINE == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      sc[t][0] = v.x;
      sc[t][1] = v.y;
    } else {
      sc[t][0] = *reinterpret_cast<const unsigned*>(p);
    }
    ssc[t] = base[Lay::kOffSS + row * Lay::kScaleRow + sb];
  }
#pragma unroll
  for (int t = 0; t < LT; ++t) {
    const int row = t * 16 + r;
    const uint8_t* p = base + Lay::kOffLC + row * Lay::kCodeRow +
                       stream_slot<KS>(row, piece) * 16 + dw0 * 4;
    if constexpr (KMINE == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      lc[t][0] = v.x;
      lc[t][1] = v.y;
    } else {
      lc[t][0] = *reinterpret_cast<const unsigned*>(p);
    }
    lsc[t] = base[Lay::kOffLS + row * Lay::kScaleRow + sb];
  }
#pragma unroll
  for (int j = 0; j < KMINE; ++j) {
    // a wave's steps (dw0, dw0 + 1 with dw0 even) lie in one block
    half8_t sa[ST], la[LT];
#pragma unroll
    for (int t = 0; t < ST; ++t) sa[t] = stream_operand(sc[t][j], ssc[t]);
#pragma unroll
    for (int t = 0; t < LT; ++t) la[t] = stream_operand(lc[t][j], lsc[t]);
#pragma unroll
    for (int a = 0; a < ST; ++a)
#pragma unroll
      for (int b = 0; b < LT; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa[a], la[b], acc[a][b], 0, 0, 0);
  }
}

// Operands of one streaming GEMM: S (streamed, s_rows rows) and L (at most
// 64 rows), both [rows][k] NVFP4 (codes, scales), and the output.
struct StreamArgs {
  const uint8_t* s_codes;
  const uint8_t* s_scales;
  int64_t s_rows;
  const uint8_t* l_codes;
  const uint8_t* l_scales;
  int64_t l_rows;
  int64_t k;
  void* out;
  int64_t ldo;
  EpiArgs ep;   // the gate pair's (EPI == kEpiGdn only)
};

// LDS bytes of a workgroup: two stage slots, or the round of partial tiles
// of the reduction, whichever is larger.
template <int SR, int LR, int KS, int NW>
struct StreamLds {
  static constexpr int kSlot = StreamLayout<SR, LR, KS>::kSlot;
  static constexpr int kTiles = ((SR + 15) / 16) * (LR / 16);
  static constexpr int kRedMax = (160 * 1024) / (NW * 1024);   // tiles per round
  static constexpr int kRound = kTiles < kRedMax ? kTiles : kRedMax;
  static constexpr int kBytes = 2 * kSlot > NW * kRound * 1024 ? 2 * kSlot : NW * kRound * 1024;
};

// One workgroup's output tile `tile` (S rows [tile * SR, tile * SR + SR) by
// all L rows) of Y = (g_s g_l) S_hat L_hat^T, stored as Y[s][l] (S_IS_M) or
// Y[l][s]; `lds` holds StreamLds::kBytes.
template <int SR, int LR, int KS, int NW, int D, bool S_IS_M, int OUT, int EPI>
__device__ __forceinline__ void stream_tile(int tile, uint8_t* lds, const StreamArgs& args,
                                            float s_g, float l_g) {
  using Lay = StreamLayout<SR, LR, KS>;
  using Ldr = StreamLoader<SR, LR, KS, NW>;
  using Lds = StreamLds<SR, LR, KS, NW>;
  constexpr int ST = (SR + 15) / 16, LT = LR / 16;
  constexpr int kSteps = KS / 32;                 // 16x16x32 k-steps per stage
  static_assert(kSteps % NW == 0, "k-steps split evenly over the waves");
  constexpr int kMine = kSteps / NW;              // k-steps per wave per stage
  static_assert(kMine == 1 || kMine == 2, "1 or 2 k-steps per wave");
  static_assert(D >= 2 && D % 2 == 0, "register ring of an even depth");
  constexpr int kSlot = Lay::kSlot;
  constexpr int kTiles = Lds::kTiles, kRound = Lds::kRound;
  // two LDS slots: stage st is stored into slot st % 2, read, and
  // overwritten by stage st + 2 only after the barrier of stage st + 1;
  // after the main loop the array takes the waves' partial sums
  uint8_t* const r0 = lds;
  uint8_t* const r1 = lds + kSlot;
  const uint8_t* const s_codes = args.s_codes;
  const uint8_t* const s_scales = args.s_scales;
  const uint8_t* const l_codes = args.l_codes;
  const uint8_t* const l_scales = args.l_scales;
  const int64_t s_rows = args.s_rows, l_rows = args.l_rows, k = args.k, ldo = args.ldo;
  void* const out = args.out;

  const double gab = static_cast<double>(s_g) * static_cast<double>(l_g);
  // the wave index is uniform over the wave; saying so keeps the buffer
  // resources and LDS addresses in scalar registers
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t s0 = static_cast<int64_t>(tile) * SR;
  const int64_t kbytes = k / 2, kblocks = k / 16;
  const int64_t s_here = s_rows - s0 < SR ? s_rows - s0 : SR;
  const int nst = static_cast<int>(k / KS);   // whole stages (k % KS == 0)

  Ldr ldr;
  ldr.init(s_codes + s0 * kbytes, s_scales + s0 * kblocks, s_here, l_codes, l_scales,
           l_rows, kbytes, kblocks, wave, lane);

  // this wave's k-steps: kMine consecutive steps of one chunk
  const int step0 = wave * kMine;
  const int chunk = step0 / 4, dw0 = step0 % 4;
  const int r = lane & 15, q = lane >> 4;

  float4_t acc[ST][LT];
#pragma unroll
  for (int i = 0; i < ST; ++i)
#pragma unroll
    for (int j = 0; j < LT; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Register ring of D stages: every stage of K up to D stages deep is in
  // flight from the start (a workgroup's whole share when k <= D * KS).
  // Every load is unconditional -- past the last stage it reads outside
  // its buffer (zeros, no memory access) and is never used -- so that the
  // compiler's wait before each register use counts exactly the younger
  // loads in flight (a load under a runtime condition makes it wait for all
  // of them).  (the scheduling barriers keep the loads in stage order: the
  // register waits count on it)
  u32x4 buf[D][Ldr::kPerWave];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    ldr.load(u, nst, buf[u]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the stage loop, unrolled by D so that every register index is a
  // constant, over whole rounds of D stages (the stages past the last one
  // only store, wait and load)
  for (int st0 = 0; st0 < nst; st0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int st = st0 + u;
      uint8_t* const slot = (u & 1) ? r1 : r0;
      ldr.store(buf[u], slot, lane);
      // this wave's stores are done; after the barrier everyone's are, and
      // every wave has finished stage st - 1 (the other slot) and stage
      // st - 2 (this slot, now overwritten)
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
      stage_barrier();
      __builtin_amdgcn_sched_barrier(0);
      ldr.load(st + D, nst, buf[u]);
      __builtin_amdgcn_sched_barrier(0);
      if (st < nst) stream_compute<SR, LR, KS, kMine>(slot, acc, chunk, dw0, r, q);
    }
  }
  __syncthreads();

  // Reduce-scatter of the waves' partial tiles, kRound tiles at a time:
  // every wave writes its partials in the accumulator layout
  // (red[w][t][lane], 16 bytes), then tile t of the round is summed by wave
  // t % NW, each lane adding its own 16 bytes from the NW copies.  16x16
  // accumulator layout: lane l holds C[4 (l / 16) + i][l % 16] (i = 0..3);
  // C rows are S rows, C columns L rows.
  float4_t* red = reinterpret_cast<float4_t*>(lds);
  const int cl = lane & 15, c4 = (lane >> 4) * 4;   // C column, first C row
#pragma unroll
  for (int t0 = 0; t0 < kTiles; t0 += kRound) {
    if (t0 > 0) __syncthreads();   // the previous round's partials are read
#pragma unroll
    for (int t = 0; t < kRound; ++t)
      if (t0 + t < kTiles) red[(wave * kRound + t) * 64 + lane] = acc[(t0 + t) / LT][(t0 + t) % LT];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kRound; ++t) {
      if (t0 + t >= kTiles || t % NW != wave) continue;
      float4_t sum = red[t * 64 + lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) sum += red[(v * kRound + t) * 64 + lane];
      const int tile = t0 + t, ts = tile / LT, tl = tile % LT;
      const int64_t lrow = tl * 16 + cl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = ts * 16 + c4 + i;
        const int64_t srow = s0 + sl;
        if (sl < SR && srow < s_rows && lrow < l_rows) {
          const float yg = static_cast<float>(static_cast<double>(sum[i]) * gab);
          if constexpr (EPI == kEpiGdn) {
            // S = the activations, L = the fused b|a weight: column lrow is
            // beta below n_beta, alpha of head lrow - n_beta above
            static_assert(S_IS_M && OUT == kOutF32, "gate pair: Y[token][head], fp32");
            const EpiArgs& ep = args.ep;
            if (lrow < ep.n_beta) {
              static_cast<float*>(out)[srow * ldo + lrow] = gdn_beta(yg);
            } else {
              const int64_t j = lrow - ep.n_beta;
              ep.out2[srow * ep.ldo2 + j] = gdn_alpha(yg, ep.a_log[j], ep.dt_bias[j]);
            }
          } else {
            const float y = epilogue<EPI>(yg);
            const int64_t o = S_IS_M ? srow * ldo + lrow : lrow * ldo + srow;
            if constexpr (OUT == kOutF32)
              static_cast<float*>(out)[o] = y;
            else
              static_cast<unsigned short*>(out)[o] = f32_to_bf16_rne(y);
          }
        }
      }
    }
  }
}

template <int SR, int LR, int KS, int NW, int D, bool S_IS_M, int OUT, int EPI>
__global__ void __launch_bounds__(NW * 64, 1)
w4a4_gemm_stream(StreamArgs args, const float* __restrict__ s_global,
                 const float* __restrict__ l_global) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[StreamLds<SR, LR, KS, NW>::kBytes];
  stream_tile<SR, LR, KS, NW, D, S_IS_M, OUT, EPI>(static_cast<int>(blockIdx.x), lds, args,
                                                   *s_global, *l_global);
}

// A streaming-GEMM configuration as a type (for the launchers below).
template <int SR_, int LR_, int KS_, int NW_, int D_>
struct StreamCfg {
  static constexpr int SR = SR_, LR = LR_, KS = KS_, NW = NW_, D = D_;
};

// The K granularity the streaming GEMM needs for an L operand of l_rows
// rows: 512-K stages, or 256 for 33-64 rows (which take 512 where they can).
inline int64_t stream_stage_k(int64_t l_rows) { return l_rows <= 32 ? 512 : 256; }

// Calls f(StreamCfg<...>{}) with the configuration for s_rows x l_rows x k
// (k % stream_stage_k(l_rows) == 0):
//   * L rows padded to 16, 32 or 64 (K stages of 512; for 64, 512 or 256,
//     below);
//   * S rows per workgroup: about one workgroup per CU (256) when S is
//     tall, 16, 24, 32, 40, 64 or 128 rows;
//   * a register ring of two stages.  Deeper rings measured slower on the
//     32 x 10240 x 5120 decode shape (D = 4: 12-13 us, 10: 13-16 us, against
//     10.4-11.4 us for D = 2, with the flushed and the warm memory-side
//     cache alike): with every stage requested at once the memory system
//     returns them in no useful order, and the first stage's compute waits
//     for most of the workgroup's data.
template <int LR, int KS, int SR, class F>
hipError_t stream_visit_d(int64_t, F&& f) {
  return f(StreamCfg<SR, LR, KS, 8, 2>{});
}

template <int LR, int KS, class F>
hipError_t stream_visit_rows(int64_t s_rows, int64_t k, F&& f) {
  const int64_t per = (s_rows + 255) / 256;
  if (per <= 16) return stream_visit_d<LR, KS, 16>(k, f);
  if (per <= 24) return stream_visit_d<LR, KS, 24>(k, f);
  if (per <= 32) return stream_visit_d<LR, KS, 32>(k, f);
  if (per <= 40) return stream_visit_d<LR, KS, 40>(k, f);
  if constexpr (LR == 64 && KS == 512) {
    return stream_visit_d<LR, KS, 64>(k, f);   // the caller keeps per <= 64
  } else {
    if (per <= 64) return stream_visit_d<LR, KS, 64>(k, f);
    return stream_visit_d<LR, KS, 128>(k, f);
  }
}

// L of 33-64 rows takes 512-K stages where the registers allow it (S slices
// of at most 64 rows) and k is a whole number of them: 12.0 against 14.9 us
// at 48 x 5120 x 5120, 16.1 against 17.9 us at 64 x 10240 x 5120; with
// 128-row slices (tall S) 256-K stages (the gate shape 32768 x 64 x 5120:
// 32.8 us, against 35.9 us for 64-row slices at 512).
template <class F>
hipError_t stream_visit(int64_t s_rows, int64_t l_rows, int64_t k, F&& f) {
  if (l_rows <= 16) return stream_visit_rows<16, 512>(s_rows, k, f);
  if (l_rows <= 32) return stream_visit_rows<32, 512>(s_rows, k, f);
  if (k % 512 == 0 && (s_rows + 255) / 256 <= 64) return stream_visit_rows<64, 512>(s_rows, k, f);
  return stream_visit_rows<64, 256>(s_rows, k, f);
}

template <bool S_IS_M, int OUT, int EPI>
hipError_t launch_stream(const StreamArgs& args, const float* s_global, const float* l_global,
                         hipStream_t stream) {
  return stream_visit(args.s_rows, args.l_rows, args.k, [&](auto cfg) -> hipError_t {
    using C = decltype(cfg);
    const int64_t grid = (args.s_rows + C::SR - 1) / C::SR;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    w4a4_gemm_stream<C::SR, C::LR, C::KS, C::NW, C::D, S_IS_M, OUT, EPI>
        <<<static_cast<unsigned>(grid), C::NW * 64, 0, stream>>>(args, s_global, l_global);
    return hipGetLastError();
  });
}

// ---------------------------------------------------------------------------
// Small-M activation quantise + GEMM in one launch, on the streaming GEMM's
// tiles.  The limitations section (한계) of the arxiv-wiki page on the paper
// puts a 2-4 % small-batch decode loss on the quantisation of the
// activations; quantising X in the GEMM's own launch removes the separate
// amax, finalise and quantise kernels.  One cooperative launch (every
// workgroup resident at once) in two phases:
//   1. the workgroups that own 16-element blocks of X (blockDim per
//      workgroup) quantise them exactly as the quantisation kernel does
//      (quant_device.h); with a self-calibrated global each of them first
//      takes max |x| over all of X itself (X has at most 64 rows), so no
//      cross-workgroup reduction is needed, and workgroup 0 stores g;
//   2. after one grid barrier (device-scope release and acquire) the
//      workgroups run the streaming GEMM's tiles over the codes just
//      written, with the configuration w4a4_gemm picks for the same shape,
//      so Y is bit-identical to quantise-then-w4a4_gemm.
// Both phases stride over the grid, which the launcher caps at the number of
// co-resident workgroups.
template <int DTYPE, int SR, int LR, int KS, int NW, int D, int OUT>
__global__ void __launch_bounds__(NW * 64, 1)
w4a4_quantize_gemm_stream(const uint8_t* __restrict__ x, int64_t ldx_bytes, int mode,
                          float* __restrict__ x_global, const float* __restrict__ w_global,
                          StreamArgs args, int tiles) {
  constexpr int kThreads = NW * 64;
  constexpr int kQuantLds = kThreads * kRowFloats * 4;
  constexpr int kLds = StreamLds<SR, LR, KS, NW>::kBytes > kQuantLds
                           ? StreamLds<SR, LR, KS, NW>::kBytes : kQuantLds;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  uint8_t* const x_codes = const_cast<uint8_t*>(args.l_codes);
  uint8_t* const x_scales = const_cast<uint8_t*>(args.l_scales);
  const int64_t m = args.l_rows, k = args.k;
  constexpr int kElemBytes = DTYPE == kDtypeF32 ? 4 : 2;
  const int64_t kb = k / 16, nblocks = m * kb;
  const bool contiguous = ldx_bytes == kb * 16 * kElemBytes;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads;
  if (first < nblocks) {   // uniform over the workgroup
    float g;
    if (mode == kModeCompute) {
      unsigned mx = 0;
      for (int64_t i = threadIdx.x; i < nblocks; i += kThreads) {
        float v[16];
        mx = max(mx, load_block<DTYPE>(block_src<DTYPE>(x, i, contiguous, kb, ldx_bytes), v));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
        mx = max(mx, static_cast<unsigned>(__shfl_xor(static_cast<int>(mx), off)));
      unsigned* part = reinterpret_cast<unsigned*>(lds);
      if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = max(mx, part[w]);
      __syncthreads();   // part is free for the settle rows below
      g = global_from_amax(__uint_as_float(mx));
      if (blockIdx.x == 0 && threadIdx.x == 0) *x_global = g;
    } else {
      g = *x_global;
    }
    bool g_ok;
    const float inv6g = recip_6g(g, &g_ok);
    float* row = reinterpret_cast<float*>(lds) + threadIdx.x * kRowFloats;
    for (int64_t b = first + threadIdx.x; b < nblocks; b += stride)
      quantize_one<DTYPE>(block_src<DTYPE>(x, b, contiguous, kb, ldx_bytes), b, g, inv6g, g_ok,
                          x_codes, x_scales, row);
  }
  // every code, scale and the global of X are written and visible
  // device-wide after the barrier
  cooperative_groups::this_grid().sync();
  const float x_g = __hip_atomic_load(x_global, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float w_g = *w_global;
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    if (tile != static_cast<int>(blockIdx.x)) __syncthreads();   // LDS of the previous tile is free
    stream_tile<SR, LR, KS, NW, D, false, OUT, kEpiNone>(tile, lds, args, w_g, x_g);
  }
}

// Co-resident workgroups of `kernel` on the current device (0 if the
// runtime cannot tell), cached per device in the caller's `cache`.
template <typename Kernel>
int stream_resident(Kernel kernel, int block, std::atomic<int> (&cache)[64]) {
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

template <int DTYPE, int OUT>
hipError_t launch_quantize_gemm_stream_t(const void* x, int64_t ldx, int mode, float* x_global,
                                         const float* w_global, const StreamArgs& args,
                                         hipStream_t stream) {
  return stream_visit(args.s_rows, args.l_rows, args.k, [&](auto cfg) -> hipError_t {
    using C = decltype(cfg);
    auto kernel = w4a4_quantize_gemm_stream<DTYPE, C::SR, C::LR, C::KS, C::NW, C::D, OUT>;
    static std::atomic<int> resident_cache[64];   // one per kernel instance
    const int resident = stream_resident(kernel, C::NW * 64, resident_cache);
    if (resident < 1) return hipErrorCooperativeLaunchTooLarge;
    const int64_t tiles = (args.s_rows + C::SR - 1) / C::SR;
    const int64_t qwgs = (args.l_rows * (args.k / 16) + C::NW * 64 - 1) / (C::NW * 64);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    int64_t grid = tiles > qwgs ? tiles : qwgs;
    if (grid > resident) grid = resident;
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    int64_t ldx_bytes = ldx * (DTYPE == kDtypeF32 ? 4 : 2);
    StreamArgs a = args;
    int tiles_i = static_cast<int>(tiles);
    void* kargs[] = {&xb, &ldx_bytes, &mode, &x_global, const_cast<float**>(&w_global), &a,
                     &tiles_i};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel),
                                      dim3(static_cast<unsigned>(grid)), dim3(C::NW * 64), kargs,
                                      0, stream);
  });
}

}  // namespace

// The gate pair takes the streaming GEMM for up to 64 gate columns (L = the
// fused b|a weight); wider pairs stay on the skinny kernel: with 128 L rows,
// 64-row S slices need two rounds of workgroups (32768 x 128 x 5120: 76.5 us
// against 70-72 us), and 128-row slices on 4 waves spill.
bool gdn_stream_fits(int64_t m, int64_t n, int64_t k) {
  return m >= 1 && n >= 1 && n <= 64 && k <= (int64_t{1} << 22) && k % stream_stage_k(n) == 0;
}

hipError_t launch_gdn_stream(const uint8_t* x_codes, const uint8_t* x_scales,
                             const float* x_global, int64_t m, const uint8_t* w_codes,
                             const uint8_t* w_scales, const float* w_global, int64_t n_beta,
                             int64_t n_alpha, int64_t k, const float* a_log,
                             const float* dt_bias, float* beta_out, int64_t ld_beta,
                             float* alpha_out, int64_t ld_alpha, hipStream_t stream) {
  const int64_t n = n_beta + n_alpha;
  const StreamArgs args{x_codes, x_scales, m, w_codes, w_scales, n, k, beta_out, ld_beta,
                        EpiArgs{a_log, dt_bias, n_beta, alpha_out, ld_alpha}};
  return launch_stream<true, kOutF32, kEpiGdn>(args, x_global, w_global, stream);
}

bool gemm_stream_fits(int64_t m, int64_t n, int64_t k) {
  if (!(m <= 64 || n <= 64) || k > (int64_t{1} << 22)) return false;
  const int64_t l_rows = m <= 64 ? m : n;
  return k % stream_stage_k(l_rows) == 0;
}

hipError_t launch_gemm_stream(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_global, int64_t m,
                              const uint8_t* b_codes, const uint8_t* b_scales,
                              const float* b_global, int64_t n, int64_t k,
                              void* out, int out_dtype, int64_t ldo, int epilogue,
                              hipStream_t stream) {
  // m <= 64: L = A (activations), S = B (Y[l][s]); else (n <= 64) S = A,
  // L = B (Y[s][l])
  const bool s_is_m = m > 64;
  const StreamArgs args = s_is_m
      ? StreamArgs{a_codes, a_scales, m, b_codes, b_scales, n, k, out, ldo}
      : StreamArgs{b_codes, b_scales, n, a_codes, a_scales, m, k, out, ldo};
  const float* sg = s_is_m ? a_global : b_global;
  const float* lg = s_is_m ? b_global : a_global;
#define NVFP4_DISPATCH(OUT, EPI)                                                   \
  return s_is_m ? launch_stream<true, OUT, EPI>(args, sg, lg, stream)              \
                : launch_stream<false, OUT, EPI>(args, sg, lg, stream);
  if (out_dtype == kOutF32) {
    if (epilogue == kEpiAlpha) NVFP4_DISPATCH(kOutF32, kEpiAlpha)
    if (epilogue == kEpiBeta) NVFP4_DISPATCH(kOutF32, kEpiBeta)
    NVFP4_DISPATCH(kOutF32, kEpiNone)
  }
  if (epilogue == kEpiAlpha) NVFP4_DISPATCH(1, kEpiAlpha)
  if (epilogue == kEpiBeta) NVFP4_DISPATCH(1, kEpiBeta)
  NVFP4_DISPATCH(1, kEpiNone)
#undef NVFP4_DISPATCH
}

hipError_t launch_quantize_gemm_stream(const void* x, int x_dtype, int64_t m, int64_t k,
                                       int64_t ldx, int mode, uint8_t* x_codes,
                                       uint8_t* x_scales, float* x_global,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* w_global, int64_t n, void* out,
                                       int out_dtype, int64_t ldo, hipStream_t stream) {
  const StreamArgs args{w_codes, w_scales, n, x_codes, x_scales, m, k, out, ldo};
  if (x_dtype == kDtypeF32) {
    if (out_dtype == kOutF32)
      return launch_quantize_gemm_stream_t<0, kOutF32>(x, ldx, mode, x_global, w_global, args, stream);
    return launch_quantize_gemm_stream_t<0, 1>(x, ldx, mode, x_global, w_global, args, stream);
  }
  if (out_dtype == kOutF32)
    return launch_quantize_gemm_stream_t<1, kOutF32>(x, ldx, mode, x_global, w_global, args, stream);
  return launch_quantize_gemm_stream_t<1, 1>(x, ldx, mode, x_global, w_global, args, stream);
}

}  // namespace nvfp4
