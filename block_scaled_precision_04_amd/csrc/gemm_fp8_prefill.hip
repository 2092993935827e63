// Large-M (prefill) block-FP8 W8A8 GEMM on gfx950.
//
// C[m, n] = sum_g As[m, g] * Ws[n/128, g] * sum_{k in group g} A[m, k] W[n, k]
// with e4m3 operands, one activation scale per token per 128-wide K group and
// one weight scale per 128x128 block (radiance_kernels.py page: the
// block_scaled_mm route and the weight / scale guards of install_load_hook).
//
// One 16x16x128 MFMA spans exactly one K group, so every K step gives each
// 16x16 block a fresh group product, which is scaled on the VALU and added
// to an fp32 accumulator: acc += P_g * (As[m, g] * Ws[n/128, g]).  The
// accumulators therefore live in ordinary VGPRs (the VALU cannot read the
// accumulator file), which bounds a wave's tile at 64 x 128 (128 fp32 per
// lane); two waves per SIMD let one wave's scaling run under the other's
// MFMAs.
//
// Tiling: a workgroup computes a 256 x 256 tile with 4 x 2 waves of 64 (m) x
// 128 (n).  The weight is the first MFMA operand (rows = n) and the
// activation the second (rows = m), so lane l holds four consecutive n of the
// single row m = l % 16 of each block: one activation scale per lane per
// 16-row block and K step; the epilogue regroups the bf16 results in LDS so
// that stores write whole output rows.  A wave's 128 columns
// lie inside one 128-wide weight-scale block, so its weight scale is one
// value per K step.
//
// Staging: each K step's activation tile (256 rows x 128 bytes, 16-byte
// chunks XOR-swizzled by row), weight tile (16 pre-laid-out 2 KiB fragment
// blocks, copied as they are) and the 256 activation scales of the step (one
// 4-byte direct-to-LDS load per row, any strides) move global -> LDS without
// passing through registers, double buffered: step k+1 is in flight while
// step k is computed.  Keeping every per-step global access on that path
// matters: a register load issued after the direct-to-LDS loads makes the
// compiler's vmcnt waits (which count all of the wave's loads, in order) wait
// for the whole next stage.  So do the weight scales of the tile's two
// 128-column blocks (a scalar load would hold up the LDS waits instead).
// Inside a step, the four MFMAs of one 16-column block are issued before the
// scaling FMAs of the previous block, so the VALU work runs under the matrix
// core instead of waiting on each result.  Tile order: the XCD-aware grouped
// raster of common.h.
#include "common.h"

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kWM = 4, kWN = 2;                      // waves along m and n
constexpr int kThreads = 64 * kWM * kWN;             // 512
constexpr int kWaves = kWM * kWN;
constexpr int kMB = kBM / kWM / 16;                  // 16-row blocks per wave (4)
constexpr int kNB = kBN / kWN / 16;                  // 16-column blocks per wave (8)
constexpr int kAStage = kBM * 128;                   // activation bytes per stage
constexpr int kBStage = kBN * 128;                   // weight bytes per stage
constexpr int kSStage = kBM * 4;                     // activation scales per stage
constexpr int kWStage = 256;                         // weight scales (one per 128 columns) per stage
constexpr int kStage = kAStage + kBStage + kSStage + kWStage;
constexpr int kAIters = kAStage / (kThreads * 16);   // direct-to-LDS loads per lane
constexpr int kBIters = kBStage / (kThreads * 16);
constexpr int kSWaves = kBM / 64;                    // waves that load one scale dword per lane
static_assert(kSWaves < kWaves, "one more wave loads the weight scales");
static_assert(kAStage % (kThreads * 16) == 0 && kBStage % (kThreads * 16) == 0, "stage / thread mismatch");
static_assert(kBN / kWN == 128, "a wave's columns must fill one weight-scale block");

// 16-byte chunk c of activation row r sits at slot c ^ ((r / 2) % 8): a
// fragment read (one chunk of 16 consecutive rows) then covers the 16 slots of
// a 256-byte LDS line once, which gfx950's 64 banks serve in one pass
BS_INLINE int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
BS_INLINE v8i pack8(uint4 x, uint4 y) {
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}
BS_INLINE v4f mfma_group(v8i w, v8i a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, v4f{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
}

__global__ __launch_bounds__(kThreads, 1) void k_fp8_prefill(const uint8_t* __restrict__ a, int lda,
                                                             const float* __restrict__ as, int64_t as_m,
                                                             int64_t as_g, const uint8_t* __restrict__ w,
                                                             const float* __restrict__ wsc, uint16_t* __restrict__ c,
                                                             int64_t ldc, int M, int N, int KS, int group_m) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStage];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int wm = wave / kWN, wn = wave % kWN;
  const int NT = N >> 4;
  const int m_tiles = (M + kBM - 1) / kBM, n_tiles = (N + kBN - 1) / kBN;
  int mt, ntile;
  xcd_tile(blockIdx.x, m_tiles, n_tiles, group_m, mt, ntile);
  const int m0 = mt * kBM, n0 = ntile * kBN;
  const int nt0 = n0 >> 4;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // ---- direct-to-LDS sources: 64-bit tile bases, unsigned 32-bit per-lane
  // offsets within the tile (< 256 * lda and < 16 * KS * 2 KiB; the host
  // keeps both below 2^32).  A load instruction
  // writes lane i's 16 bytes at (uniform LDS base) + 16*i, so each lane
  // fetches the chunk that belongs at its LDS position.  Rows past M and
  // 16-column tiles past N fetch the last valid row / tile (finite data,
  // never stored).
  const uint8_t* a_tile = a + static_cast<size_t>(m0) * lda;
  const uint8_t* w_tile = w + static_cast<size_t>(nt0) * KS * 2048;
  uint32_t aoff[kAIters];
#pragma unroll
  for (int i = 0; i < kAIters; ++i) {
    const int p = (i * kWaves + wave) * 64 + l;      // 16-byte position in the activation stage
    const int row = p >> 3, slot = p & 7;
    aoff[i] = static_cast<uint32_t>(min(m0 + row, M - 1) - m0) * static_cast<uint32_t>(lda) +
              static_cast<uint32_t>(16 * swz(row, slot));
  }
  // weight stage: 1 KiB half-blocks h = 2 * (16-column tile) + half, in the
  // pre-laid-out order (lane-major 16-byte chunks)
  uint32_t boff[kBIters];
#pragma unroll
  for (int j = 0; j < kBIters; ++j) {
    const int h = j * kWaves + wave;
    const int ntl = min(nt0 + (h >> 1), NT - 1) - nt0;
    boff[j] = static_cast<uint32_t>(ntl) * static_cast<uint32_t>(KS) * 2048u + static_cast<uint32_t>((h & 1) * 1024 + l * 16);
  }
  // activation scales: wave w < kSWaves loads rows 64w .. 64w+63 of the tile
  // (tile base + K-step offset are 64-bit scalars; the row offset < 256 * as_m)
  const float* as_tile = as + static_cast<int64_t>(m0) * as_m;
  const uint32_t soff = static_cast<uint32_t>((min(m0 + wave * 64 + l, M - 1) - m0) * as_m * 4);
  // weight scales of the tile's 128-column blocks: lane j -> block (n0/128 + j)
  const uint32_t woff = static_cast<uint32_t>(min((n0 >> 7) + l, (N >> 7) - 1)) * static_cast<uint32_t>(KS) * 4u;
  // the i-th 16-byte load of stage ks (activation pieces, then weight pieces)
  auto dma_piece = [&](int i, int ks, int buf) {
    const uint32_t base = lds0 + buf * kStage;
    if (i < kAIters) {
      dma16(base + (i * kWaves + wave) * 1024, a_tile + ks * 128, aoff[i]);
    } else {
      const int j = i - kAIters;
      dma16(base + kAStage + (j * kWaves + wave) * 1024, w_tile + static_cast<size_t>(ks) * 2048, boff[j]);
    }
  };
  auto dma_scales = [&](int ks, int buf) {
    const uint32_t base = lds0 + buf * kStage;
    if (wave < kSWaves) dma4(base + kAStage + kBStage + wave * 256, as_tile + ks * as_g, soff);
    else if (wave == kSWaves) dma4(base + kAStage + kBStage + kSStage, wsc + ks, woff);
  };
  auto dma_stage = [&](int ks, int buf) {
#pragma unroll
    for (int i = 0; i < kAIters + kBIters; ++i) dma_piece(i, ks, buf);
    dma_scales(ks, buf);
  };
  // next-stage loads issued before a step's first MFMA, then two after each
  // 16-column block's MFMAs until all are out (see the K loop)
  constexpr int kDmaEarly = 2;
  static_assert(kAIters + kBIters <= kDmaEarly + 2 * kNB, "the K loop issues every load of the next stage");

  // ---- fragment offsets within a stage.  Both operands hold K = 32*(l/16)
  // .. +31 of their row in lane l (the pre-layout's order; the pairing inside
  // the MFMA is positional, so any K order shared by both sides is exact).
  const int q = l >> 4;
  int afr[kMB][2];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int row = wm * (kBM / kWM) + mb * 16 + (l & 15);
    afr[mb][0] = row * 128 + 16 * swz(row, 2 * q);
    afr[mb][1] = row * 128 + 16 * swz(row, 2 * q + 1);
  }
  const int bfr = kAStage + wn * kNB * 2048 + l * 16;

  // ---- scales: the lane's row of each 16-row block (LDS), the wave's weight block
  int sfr[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) sfr[mb] = kAStage + kBStage + (wm * (kBM / kWM) + mb * 16 + (l & 15)) * 4;
  const int ncol0 = n0 + wn * (kBN / kWN);
  const bool live_n = ncol0 < N;  // wave-uniform: N % 128 == 0
  const int wfr = kAStage + kBStage + kSStage + wn * 4;

  v4f acc[kMB][kNB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = v4f{0, 0, 0, 0};

  dma_stage(0, 0);
  wait_vm<0>();
  __syncthreads();

  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    // The next stage's eight 16-byte loads per lane go out early in the step
    // but not as one burst: two before the first MFMA, then two after each
    // of the first three 16-column blocks' MFMAs, so they have most of the
    // step to land before the wait that closes it.  A burst of all of them
    // (plus the scales) before the MFMAs backs up the load unit and each
    // wave stalls on it; one per block, spread over the whole step, leaves
    // the last loads too little time (M=8192 N=5120 K=17408: one per block
    // 752-763 us, this schedule 692-701, the burst 720; M=4096 N=10240
    // K=5120 241-258 -> 225-235 us).  After the last step they reload the
    // last stage into the idle buffer (never read).
    const int kn = min(ks + 1, KS - 1);
    dma_scales(kn, buf ^ 1);
    if (!live_n) {
#pragma unroll
      for (int i = 0; i < kAIters + kBIters; ++i) dma_piece(i, kn, buf ^ 1);
    } else {
      const uint8_t* st = lds + buf * kStage;
      float s[kMB];
      v8i af[kMB];
      const float sw = *reinterpret_cast<const float*>(st + wfr);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        af[mb] = pack8(*reinterpret_cast<const uint4*>(st + afr[mb][0]),
                       *reinterpret_cast<const uint4*>(st + afr[mb][1]));
        s[mb] = *reinterpret_cast<const float*>(st + sfr[mb]) * sw;
      }
      auto bfrag = [&](int nb) {
        return pack8(*reinterpret_cast<const uint4*>(st + bfr + nb * 2048),
                     *reinterpret_cast<const uint4*>(st + bfr + nb * 2048 + 1024));
      };
      v8i bcur = bfrag(0);
#pragma unroll
      for (int i = 0; i < kDmaEarly; ++i) dma_piece(i, kn, buf ^ 1);
      v4f t[kMB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const v8i bnext = bfrag(min(nb + 1, kNB - 1));
        v4f tn[kMB];
        // the block's MFMAs at raised wave priority: where both waves of a
        // SIMD are ready, the one with MFMAs to issue goes first and the
        // other's scaling FMAs fill in behind them (M=4096 N=10240 K=5120
        // 241-250 -> 225-235 us, M=8192 N=10240 420-433 -> 403-423, K=17408
        // unchanged)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) tn[mb] = mfma_group(bcur, af[mb]);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = kDmaEarly + 2 * nb; i < kDmaEarly + 2 * nb + 2 && i < kAIters + kBIters; ++i)
          dma_piece(i, kn, buf ^ 1);
        if (nb > 0) {
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) acc[mb][nb - 1] += t[mb] * s[mb];
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) t[mb] = tn[mb];
        bcur = bnext;
      }
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[mb][kNB - 1] += t[mb] * s[mb];
    }
    wait_vm<0>();     // stage ks+1 has landed
    __syncthreads();  // ... and every wave is done with buffer ks & 1
  }

  // ---- epilogue: bf16 RNE, then through LDS so that each store instruction
  // writes whole output rows.  A lane holds four consecutive n of one m, and
  // the 16 lanes of a quarter wave hold 16 different rows; each wave writes
  // its 8-byte pieces into an LDS copy of the tile (row-major, 512 bytes per
  // row, piece index XOR (row % 8) * 4, which puts the 64 pieces of one write
  // on 32 distinct bank slots), then lane j of a row stores piece j with the
  // non-temporal hint (the output is written once).  The
  // tile (128 KiB) fits in the two stage buffers, idle after the last barrier
  // of the loop.  Waves whose columns lie past N take part in the barrier;
  // their pieces are never stored.
  constexpr int kPieces = kBN / 4;
  constexpr int kRowsPerPass = kThreads / kPieces;
  static_assert(kBM * kBN * 2 <= 2 * kStage, "output tile must fit the stage buffers");
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int r = wm * (kBM / kWM) + mb * 16 + (l & 15);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int piece = wn * (kBN / kWN / 4) + nb * 4 + q;
      const v4f v = acc[mb][nb];
      const uint32_t lo = bf16x2_rne(v[0], v[1]);
      const uint32_t hi = bf16x2_rne(v[2], v[3]);
      *reinterpret_cast<uint2*>(lds + r * (kBN * 2) + (piece ^ ((r & 7) << 2)) * 8) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
  if (m0 + kBM <= M && n0 + kBN <= N && ldc % 8 == 0) {
    // whole tile, 16-byte rows (wave-uniform test): the swizzle moves pieces
    // in groups of four, so pieces 2p and 2p+1 stay adjacent and in order;
    // lane p of a row stores pair p, the row address advances by a scalar
    // stride and a batch's LDS reads are issued before its stores
    constexpr int kPairs = kBN / 8, kRows2 = kThreads / kPairs, kIters = kBM / kRows2, kBatch = 8;
    static_assert(kThreads % kPairs == 0 && kIters % kBatch == 0, "store batch shape");
    const int p = tid % kPairs, r0 = tid / kPairs;
    uint16_t* crow = c + static_cast<int64_t>(m0 + r0) * ldc + n0 + 8 * p;
    const int64_t rstep = kRows2 * ldc;
#pragma unroll
    for (int b0 = 0; b0 < kIters; b0 += kBatch) {
      uint4 o[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int r = r0 + (b0 + u) * kRows2;
        o[u] = *reinterpret_cast<const uint4*>(lds + r * (kBN * 2) + ((2 * p) ^ ((r & 7) << 2)) * 8);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) st_stream16(reinterpret_cast<uint4*>(crow + (b0 + u) * rstep), o[u]);
    }
    return;
  }
  const int j = tid % kPieces, r0 = tid / kPieces;
  const bool n_ok = n0 + 4 * j < N;
#pragma unroll 4
  for (int r = r0; r < kBM; r += kRowsPerPass) {
    const uint2 v = *reinterpret_cast<const uint2*>(lds + r * (kBN * 2) + (j ^ ((r & 7) << 2)) * 8);
    if (n_ok && m0 + r < M) st_stream8(reinterpret_cast<uint2*>(c + static_cast<int64_t>(m0 + r) * ldc + n0 + 4 * j), v.x, v.y);
  }
}

}  // namespace

// Whether the tiled kernel takes the call instead of the decode kernel, which
// runs 64 rows per launch and streams the whole weight once per launch.  From
// 512 rows always.  Up to 64 rows never: one decode launch streams the weight
// once, and a 256x256 tile would waste most of its rows.  In between, a cost
// model fitted to graph-replayed timings on MI355X (pooled weights) picks the
// cheaper side.  The tiled kernel sweeps all of K in every tile with no
// split, so it costs about 4 + 1.6 * K/128 us per round of 256 tiles (66-72
// us at K = 5120, 210-222 us at K = 17408).  A 64-row decode launch costs
// about 2 us plus 0.38 us per million weight bytes (13 / 21 / 35 us for
// 26 / 52 / 89 MB).  Measured crossovers it reproduces: at N = K = 5120 the
// decode launches win at M = 320 (63-64 against 66 us) and lose at 384
// (76-77 against 66-67); at N = 10240, K = 5120 they win at 192 (63 against
// 70) and lose at 256 (82 against 72); at N = 5120, K = 17408 they win at 256
// (140 against 222), tie at 384 (209-211 against 209) and lose at 448 (244
// against 213).
bool bs_fp8_use_tiled(int M, int N, int K) {
  if (M >= 512) return true;
  if (M <= 64) return false;
  const int64_t tiles = static_cast<int64_t>((M + 255) / 256) * ((N + 255) / 256);
  // both estimates in units of 0.1 us
  const int64_t tiled = (tiles + 255) / 256 * (40 + 16 * static_cast<int64_t>(K / 128));
  const int64_t decode =
      static_cast<int64_t>((M + 63) / 64) * (20 + static_cast<int64_t>(N) * static_cast<int64_t>(K) * 38 / 10000000);
  return tiled < decode;
}

int bs_launch_fp8_block_prefill(const uint8_t* a, int64_t lda, const float* as, int64_t as_m, int64_t as_g,
                                const uint8_t* w, const float* ws, uint16_t* c, int64_t ldc, int M, int N, int K,
                                hipStream_t st) {
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  k_fp8_prefill<<<dim3(tiles), dim3(kThreads), 0, st>>>(a, static_cast<int>(lda), as, as_m, as_g, w, ws, c, ldc, M,
                                                       N, K / 128, 4);
  return bs_launch_status();
}
