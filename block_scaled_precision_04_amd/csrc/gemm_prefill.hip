// Large-M (prefill) MXFP4 W4A8 GEMM on gfx950 scaled MFMA.
//
// The radiance_mxfp4.py page (module docstring) explains why this path is
// hand-written: the compiler route upconverts e2m1 to 16 bits and never
// issues the low-precision matrix instruction, while the hardware's own
// 8-bit matrix instruction is about twice as fast.  On gfx950 the scaled
// MFMA V_MFMA_SCALE_F32_32X32X64_F8F6F4 takes the e2m1 weight and the e4m3
// activation directly and applies the MX e8m0 block scale (one per 32 K) in
// hardware, so the exact dequantised product of the page's _exact_ref is
// accumulated in fp32 with no software decode at all.  The mixed fp4 x fp8
// instruction issues at the FP8 rate.
//
// Tiling: a workgroup computes a BM x BN output tile with WM x WN waves; each
// wave owns (BM/WM) x (BN/WN) as 32x32 MFMA sub-tiles with fp32 accumulators
// (the large tiles keep them in the accumulator registers).  K advances in
// 128-wide steps.  Each step's activation tile (BM rows x 128 bytes), weight
// tile (BN/16 fragment-order 1 KiB blocks, copied as they are) and the e8m0
// dwords of the tile's 16-column blocks (one dword per lane per four steps,
// as pre-laid-out) are moved global -> LDS by the direct-to-LDS 16-byte load
// (no register staging) into one of three stage buffers: the loads of step
// k+2 are issued while step k is computed.  Activation rows are stored
// without padding; their eight 16-byte chunks are XOR-swizzled by bits 1..3
// of the row index.  gfx950's LDS has 64 four-byte banks and serves a 16-byte
// read 16 lanes at a time, so a read is conflict-free when its 16 lanes hit
// 16 distinct 16-byte slots of a 256-byte line; the fragment reads take one
// chunk of 16 consecutive rows, two rows per 256 bytes, and the swizzle by
// (row / 2) % 8 gives each row pair the eight slots (measured: the swizzle by
// row % 8 served these reads in two passes).  The per-token activation
// scale multiplies the accumulator in the epilogue, then bf16 RNE and store.
// The first MFMA operand is the weight (rows = n), the second the
// activation (rows = m), so each lane holds four consecutive n of one m; the
// epilogue regroups them in LDS into whole output rows before storing (as
// bf16 where the accumulators are ordinary registers, as fp32 straight from
// the accumulator registers otherwise).  Which tile size runs where (and the
// column strip that avoids a partial last round of large tiles) is decided by
// prefill_plan below.
//
// Workgroup -> tile order: gfx950 hands workgroup b to XCD b % 8, and each
// XCD has its own L2.  The tile sequence is cut into eight contiguous chunks,
// one per XCD, and inside a chunk tiles follow a grouped raster (GROUP_M
// m-tiles sweep the n-tiles together), so the workgroups resident on one XCD
// at any moment share a few activation and weight tiles in that XCD's L2.
#include <algorithm>
#include <numeric>
#include <type_traits>

#include "common.h"

namespace {

BS_INLINE int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

constexpr std::true_type kWithDma{};
constexpr std::false_type kNoDma{};

template <int BM, int BN, int WM, int WN>
struct PrefillCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWaves = WM * WN;
  static constexpr int kTM = BM / WM / 32;  // 32-row sub-tiles per wave along m
  static constexpr int kTN = BN / WN / 32;  // along n
  static constexpr int kAStage = BM * 128;  // bytes of one staged activation tile
  static constexpr int kBStage = BN * 64;   // bytes of one staged weight tile
  static constexpr int kSStage = BN * 16;   // e8m0 dwords of the tile's n-tiles for four K steps
  static constexpr int kStage = kAStage + kBStage + kSStage;
  static constexpr int kAIters = kAStage / (kThreads * 16);
  static constexpr int kBIters = kBStage / (kThreads * 16);
  static constexpr int kSIters = (kSStage + kThreads * 16 - 1) / (kThreads * 16);
  static constexpr int kSPieces = kSStage / 1024;  // one wave-wide 16-byte load each
  // direct-to-LDS loads per stage, the same for every wave: where the e8m0
  // region has fewer 1 KiB pieces than the waves' loads cover, the waves past
  // it repeat an earlier wave's piece (same source, same LDS bytes, identical
  // values), so no load is conditional on the wave and the K loop has no
  // branch for the scheduler to stop at
  static constexpr int kDma = kAIters + kBIters + kSIters;
  static_assert(kAStage % (kThreads * 16) == 0 && kBStage % (kThreads * 16) == 0, "tile / thread mismatch");
  static_assert(kSStage % 1024 == 0, "scale stage must be whole waves");
  static_assert(kTM >= 1 && kTN >= 1, "wave tile too small");
};

// Tile position b is computed by workgroup b, or (large tiles, see the
// kernel) by workgroup b - G, which runs on the same XCD: workgroup b runs
// on XCD b % 8 and G is a multiple of 256.  The tile sequence is cut into
// eight contiguous chunks, one per XCD, so the tiles resident on one XCD at
// any moment are neighbours in the grouped raster and share activation /
// weight tiles in that XCD's L2.
// Split launches, grid (tiles, S): workgroup (x, y) computes tile x over the
// y-th of S equal runs of K steps; the partial tile goes to the workspace
// slab and the last of the S workgroups of a tile adds them in split order.
// AT = true: the activation arrives in the activation-tiled order (32-row
// blocks of 4 KiB per K step, each half step the 32 bytes of every lane of
// one 32x32x64 MFMA operand, written so by the tiled producer).  A stage's
// activation tile is then BM/32 contiguous 4 KiB blocks, copied as they are,
// and a fragment is read at a fixed lane offset: no swizzle, no re-layout.
// The work of one output tile, bx (the tile's position in the launch order);
// the kernel below runs it for one tile or, for the large tiles, two.
template <int BM, int BN, int WM, int WN, int OCC, bool SPLIT, bool IL, bool AT>
__device__ __forceinline__ void prefill_tile(
    int bx, const uint8_t* __restrict__ a, int lda, const float* __restrict__ as, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ wsc, uint16_t* __restrict__ c, int64_t ldc, int M, int N, int KS, int group_m,
    float* __restrict__ slab, int* __restrict__ counters) {
  using C = PrefillCfg<BM, BN, WM, WN>;
  constexpr int STAGES = 3;
  // the stage buffers, then the tile's BM per-token activation scales
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * C::kStage + BM * 4];
  __shared__ int last;
  const int S = SPLIT ? static_cast<int>(gridDim.y) : 1, sp = SPLIT ? static_cast<int>(blockIdx.y) : 0;
  const int k_begin = SPLIT ? KS * sp / S : 0;   // KS < 2^24 (K < 2^31), so KS * S fits in 32 bits
  const int k_end = SPLIT ? KS * (sp + 1) / S : KS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int NT = N >> 4;
  const int KQ = (KS + 3) >> 2;
  const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const float* s_tok = reinterpret_cast<const float*>(lds + STAGES * C::kStage);
  int mt, ntile;
  xcd_tile(bx, m_tiles, n_tiles, group_m, mt, ntile);
  const int m0 = mt * BM, n0 = ntile * BN;
  const int nt0 = n0 >> 4;

  // ---- per-lane 32-bit source offsets of the direct-to-LDS loads.  A load
  // instruction writes lane i's 16 bytes at (uniform LDS base) + 16*i, so each
  // lane fetches the chunk that belongs at its LDS position.  Rows past M and
  // n-tiles past N fetch the last valid row / tile (finite data, never stored).
  uint32_t aoff[C::kAIters];
#pragma unroll
  for (int i = 0; i < C::kAIters; ++i) {
    const int p = (i * C::kWaves + wave) * 64 + l;  // 16-byte position in the activation stage
    if constexpr (AT) {
      // tiled: position p is byte 16 (p % 256) of the stage's (p / 256)-th
      // 32-row block; blocks past the padded M re-read the last one
      const int rb = min((m0 >> 5) + (p >> 8), ((M + 31) >> 5) - 1);
      aoff[i] = static_cast<uint32_t>(rb) * static_cast<uint32_t>(KS) * 4096u + static_cast<uint32_t>((p & 255) * 16);
    } else {
      const int row = p >> 3, slot = p & 7;
      aoff[i] = static_cast<uint32_t>(min(m0 + row, M - 1)) * static_cast<uint32_t>(lda) +
                static_cast<uint32_t>(16 * swz(row, slot));
    }
  }
  uint32_t boff_g[C::kBIters];
#pragma unroll
  for (int i = 0; i < C::kBIters; ++i) {
    const int nt = min(nt0 + i * C::kWaves + wave, NT - 1);
    boff_g[i] = static_cast<uint32_t>(nt) * static_cast<uint32_t>(KS) * 1024u + static_cast<uint32_t>(l * 16);
  }
  uint32_t soff_g[C::kSIters];
#pragma unroll
  for (int i = 0; i < C::kSIters; ++i) {
    const int p = ((i * C::kWaves + wave) % C::kSPieces) * 64 + l;
    const int nt = min(nt0 + (p >> 4), NT - 1);
    soff_g[i] = static_cast<uint32_t>(nt) * static_cast<uint32_t>(KQ) * 256u + static_cast<uint32_t>((p & 15) * 16);
  }
  // the i-th direct-to-LDS load of step ks (i < kDma) into buffer buf
  auto dma_one = [&](int i, int ks, int buf) {
    const uint32_t base = lds0 + buf * C::kStage;
    if (i < C::kAIters) {
      dma16(base + (i * C::kWaves + wave) * 1024, a + static_cast<size_t>(ks) * (AT ? 4096 : 128), aoff[i]);
    } else if (i < C::kAIters + C::kBIters) {
      const int j = i - C::kAIters;
      dma16(base + C::kAStage + (j * C::kWaves + wave) * 1024, w + static_cast<size_t>(ks) * 1024, boff_g[j]);
    } else {
      const int j = i - C::kAIters - C::kBIters;
      dma16(base + C::kAStage + C::kBStage + ((j * C::kWaves + wave) % C::kSPieces) * 1024, wsc + (ks >> 2) * 256,
            soff_g[j]);
    }
  };

  v16f acc[C::kTN][C::kTM];
#pragma unroll
  for (int p = 0; p < C::kTN; ++p)
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) acc[p][q] = v16f{};

  // fragment LDS offsets (within a stage) that do not depend on the K step
  int boff[C::kTN][2], soff[C::kTN][2];
#pragma unroll
  for (int p = 0; p < C::kTN; ++p) {
    const int nl = wn * (BN / WN) + 32 * p + (l & 31);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int lanep = (nl & 15) + 16 * (2 * hh + (l >> 5));
      boff[p][hh] = C::kAStage + (nl >> 4) * 1024 + lanep * 16;
      soff[p][hh] = C::kAStage + C::kBStage + (nl >> 4) * 256 + lanep * 4;
    }
  }
  int arow[C::kTM];
#pragma unroll
  for (int q = 0; q < C::kTM; ++q) arow[q] = wm * (BM / WM) + 32 * q + (l & 31);

  // the activation fragment of 32-row sub-tile q, half step hh, from stage st
  auto a_frag = [&](const uint8_t* st, int hh, int q) {
    uint4 u, v;
    if constexpr (AT) {
      // the lane's 32 bytes of the sub-tile's block, as the producer laid them out
      const uint8_t* src = st + (arow[q] >> 5) * 4096 + hh * 2048 + l * 32;
      u = *reinterpret_cast<const uint4*>(src);
      v = *reinterpret_cast<const uint4*>(src + 16);
    } else {
      // chunks 4hh + g and 4hh + 2 + g of the row (the 8-bit operand's order)
      const int r = arow[q];
      const int c0 = 4 * hh + (l >> 5);
      u = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * swz(r, c0));
      v = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * swz(r, c0 + 2));
    }
    return v8i{(int)u.x, (int)u.y, (int)u.z, (int)u.w, (int)v.x, (int)v.y, (int)v.z, (int)v.w};
  };
  // fragments of one half step (64 K): weight, activation, e8m0 dword per p
  struct Frag {
    v8i b[C::kTN];
    v8i a[C::kTM];
    uint32_t s[C::kTN];
  };
  auto lds_frags = [&](const uint8_t* st, int hh, Frag& f) {
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      const uint4 v = *reinterpret_cast<const uint4*>(st + boff[p][hh]);
      f.b[p] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      f.s[p] = *reinterpret_cast<const uint32_t*>(st + soff[p][hh]);
    }
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) f.a[q] = a_frag(st, hh, q);
  };
  // MFMAs of one half step; with DMA the loads of step dks (into buffer
  // dbuf) are issued between them (one after each MFMA), so the load unit is
  // fed steadily and the wave never stalls on a burst of loads
  // (DMA is a compile-time flag, so that the K loop holds no branch on it)
  auto mma = [&](const Frag& f, int sh, auto dma, int dks, int dbuf) {
    constexpr bool DMA = decltype(dma)::value;
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      const int sc = static_cast<int>(f.s[p] >> sh);
#pragma unroll
      for (int q = 0; q < C::kTM; ++q) {
        acc[p][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[p], f.a[q], acc[p][q], 4, 0, 0, sc, 0, 127);
        const int i = p * C::kTM + q;
        if (DMA && i < C::kDma) {
          __builtin_amdgcn_sched_barrier(0);
          dma_one(i, dks, dbuf);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // loads left over when a half step has fewer MFMAs than loads
#pragma unroll
    for (int i = C::kTN * C::kTM; i < C::kDma; ++i)
      if (DMA) dma_one(i, dks, dbuf);
  };

  // one LDS read "piece" of a fragment set: pieces 0..kTN-1 are the weight
  // fragments (+ e8m0 dword), kTN..kTN+kTM-1 the activation fragments
  auto lds_piece = [&](const uint8_t* st, int hh, Frag& f, int i) {
    if (i < C::kTN) {
      const int p = i;
      const uint4 v = *reinterpret_cast<const uint4*>(st + boff[p][hh]);
      f.b[p] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      f.s[p] = *reinterpret_cast<const uint32_t*>(st + soff[p][hh]);
    } else {
      f.a[i - C::kTN] = a_frag(st, hh, i - C::kTN);
    }
  };
  // MFMAs of one half step; after MFMA i, DMA i of step dks (if dks >= 0)
  // and LDS-read piece i of the set rf (from stage rst, half rhh)
  auto mma_il = [&](const Frag& f, int sh, int dks, int dbuf, const uint8_t* rst, int rhh, Frag& rf) {
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      const int sc = static_cast<int>(f.s[p] >> sh);
#pragma unroll
      for (int q = 0; q < C::kTM; ++q) {
        acc[p][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[p], f.a[q], acc[p][q], 4, 0, 0, sc, 0, 127);
        const int i = p * C::kTM + q;
        __builtin_amdgcn_sched_barrier(0);
        if (i < C::kDma && dks >= 0) dma_one(i, dks, dbuf);
        if (i < C::kTN + C::kTM) lds_piece(rst, rhh, rf, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = C::kTN * C::kTM; i < C::kDma; ++i)
      if (dks >= 0) dma_one(i, dks, dbuf);
#pragma unroll
    for (int i = C::kTN * C::kTM; i < C::kTN + C::kTM; ++i) lds_piece(rst, rhh, rf, i);
  };
  // Pipeline (the plain schedule, used with the 128x128 tile): three LDS
  // buffers (buffer of step s = s % 3) and fragment register sets rotating
  // over the 64-K halves.  A half step has only four MFMAs per wave (128 ns),
  // about the latency of its fragment reads, so every read is issued under
  // the MFMAs of the half before it.  Step s, with sets (X, Y, Z):
  //   MFMAs on X (first half of s), the LDS reads of Y (second half of s)
  //   issued after the first of them; wait until this wave's loads of step s+1
  //   have landed and its reads are done; barrier in mid-step (step s+1
  //   published; every wave is done with buffer s); MFMAs on Y, with the
  //   loads of step s+3 into buffer s and the reads of Z (first half of
  //   s+1) issued between them.
  // The next step uses (Z, X, Y).  The loads of a step are issued a step and
  // a half before the barrier that publishes it.
  auto mma_rd = [&](const Frag& f, int sh, auto dma, int dks, int dbuf, const uint8_t* rst, int rhh, Frag& rf) {
    constexpr bool DMA = decltype(dma)::value;
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      const int sc = static_cast<int>(f.s[p] >> sh);
#pragma unroll
      for (int q = 0; q < C::kTM; ++q) {
        acc[p][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[p], f.a[q], acc[p][q], 4, 0, 0, sc, 0, 127);
        const int i = p * C::kTM + q;
        __builtin_amdgcn_sched_barrier(0);
        if (DMA && i < C::kDma) dma_one(i, dks, dbuf);
        if (i == 0) {
          // every read of the next set, in the order its MFMAs use them:
          // weight 0, the activations, then the other weights
          lds_piece(rst, rhh, rf, 0);
#pragma unroll
          for (int j = 0; j < C::kTM; ++j) lds_piece(rst, rhh, rf, C::kTN + j);
#pragma unroll
          for (int j = 1; j < C::kTN; ++j) lds_piece(rst, rhh, rf, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = C::kTN * C::kTM; i < C::kDma; ++i)
      if (DMA) dma_one(i, dks, dbuf);
  };
  // The tile's per-token scales go to LDS ahead of the first stage (64 rows
  // per wave-wide 4-byte load; with BM < 256 the waves past BM / 64 repeat an
  // earlier wave's load), so the epilogue does not wait on global loads.
  {
    constexpr int kTokLoads = BM / 64;
    static_assert(BM % 64 == 0 && kTokLoads <= C::kWaves, "one 64-row scale load per wave");
    const int part = wave % kTokLoads;
    dma4(lds0 + STAGES * C::kStage + part * 256, as,
         static_cast<uint32_t>(min(m0 + part * 64 + l, M - 1)) * 4u);
  }
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) dma_one(i, k_begin, 0);
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) dma_one(i, min(k_begin + 1, k_end - 1), 1);
  if constexpr (!IL) {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) dma_one(i, min(k_begin + 2, k_end - 1), 2);
    wait_vm<2 * C::kDma>();
  } else {
    wait_vm<C::kDma>();
  }
  __syncthreads();
  Frag f0, f1, f2;
  lds_frags(lds, 0, f0);

  int buf = 0;
  // A set whose MFMAs were just issued is dead to the register allocator,
  // which then hands its registers to the next refill: the LDS reads would
  // overwrite operands of MFMAs still in the queue.  keep() marks a set live
  // up to the point where it stands, so each refill gets registers of its own.
  auto keep = [&](const Frag& f) {
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      keep_vgprs(__builtin_shufflevector(f.b[p], f.b[p], 0, 1, 2, 3));
      keep_vgprs(f.s[p]);
    }
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) keep_vgprs(f.a[q]);
  };
  auto step = [&](int ks, Frag& fx, Frag& fy, Frag& fz) {
    const int sh = 8 * (ks & 3);
    const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
    __builtin_amdgcn_sched_barrier(0);
    mma_rd(fx, sh, kNoDma, 0, 0, lds + buf * C::kStage, 1, fy);
    keep(fx);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<C::kDma>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // (after the last step this reads a buffer whose values are never used)
    mma_rd(fy, sh, kWithDma, min(ks + 3, k_end - 1), buf, lds + nbuf * C::kStage, 0, fz);
    keep(fy);
    buf = nbuf;
  };
  // The interleaved schedule (IL, used with the 256x256 tile), step s: this
  // wave's loads of step s+1 landed and its LDS reads done ->
  // barrier (step s+1 published, buffer s-1 free) -> MFMAs of the first half
  // of s, interleaved with the loads of step s+2 (into buffer s-1) and the LDS
  // reads of the second half of s -> MFMAs of the second half, interleaved
  // with the LDS reads of the first half of s+1.
  auto step2 = [&](int ks, Frag& fx, Frag& fy, Frag& fz) {
    const int sh = 8 * (ks & 3);
    const int b0 = (ks - k_begin) % STAGES;
    const int b1 = b0 + 1 == STAGES ? 0 : b0 + 1;
    const int b2 = b1 + 1 == STAGES ? 0 : b1 + 1;
    wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    mma_il(fx, sh, min(ks + 2, k_end - 1), b2, lds + b0 * C::kStage, 1, fy);
    __builtin_amdgcn_sched_barrier(0);
    mma_il(fy, sh, -1, 0, lds + b1 * C::kStage, 0, fz);
    __builtin_amdgcn_sched_barrier(0);
  };
  int ks = k_begin;
  if constexpr (IL) {
    for (; ks + 3 <= k_end; ks += 3) {
      step2(ks, f0, f1, f2);
      step2(ks + 1, f2, f0, f1);
      step2(ks + 2, f1, f2, f0);
    }
    if (ks < k_end) step2(ks++, f0, f1, f2);
    if (ks < k_end) step2(ks++, f2, f0, f1);
    (void)buf;
  } else {
    for (; ks + 3 <= k_end; ks += 3) {
      step(ks, f0, f1, f2);
      step(ks + 1, f2, f0, f1);
      step(ks + 2, f1, f2, f0);
    }
    if (ks < k_end) step(ks++, f0, f1, f2);
    if (ks < k_end) step(ks++, f2, f0, f1);
  }
  wait_vm<0>();

  // ---- epilogue: x per-token scale, bf16 RNE, then through LDS so that each
  // store instruction writes whole output rows.  A lane's MFMA results are
  // four consecutive n of one m, and the 32 lanes of a half wave hold 32
  // different rows: stored directly, every instruction would touch 32 rows.
  // Instead each wave writes its 8-byte pieces into an LDS copy of the tile
  // (row-major, BN * 2 bytes per row, 8-byte pieces XOR-swizzled by the low
  // five row bits so the 32 rows of a write land in distinct banks), and
  // then every wave stores whole rows: lane j of a row writes piece j, with
  // the non-temporal hint (the output is written once and never re-read
  // here, so it should not displace operand lines from L2).  The
  // tile (at most 128 KiB) fits in the stage buffers, which are idle once
  // every wave's loads have landed and its LDS reads are done.
  auto store_tile = [&]() {
    constexpr int kPieces = BN / 4;                 // 8-byte pieces per row
    constexpr int kRowsPerPass = C::kThreads / kPieces;
    static_assert(BM * BN * 2 <= STAGES * C::kStage, "output tile must fit the stage buffers");
    static_assert(C::kThreads % kPieces == 0 && BM % kRowsPerPass == 0, "store pass shape");
    wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) {
      const int r = arow[q];
      const float sc = s_tok[r];
#pragma unroll
      for (int p = 0; p < C::kTN; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int piece = (wn * (BN / WN) + 32 * p + 8 * i) / 4 + (l >> 5);
          *reinterpret_cast<uint2*>(lds + r * (BN * 2) + (piece ^ (r & 31)) * 8) =
              make_uint2(bf16x2_rne(acc[p][q][4 * i + 0] * sc, acc[p][q][4 * i + 1] * sc),
                         bf16x2_rne(acc[p][q][4 * i + 2] * sc, acc[p][q][4 * i + 3] * sc));
        }
      }
    }
    __syncthreads();
    if (ldc % 8 == 0) {
      // 16-byte pieces: logical 8-byte pieces 2j and 2j+1 sit in the
      // physical pair j ^ (s >> 1) (s = r % 32), swapped when s is odd
      constexpr int kPairs = BN / 8;
      constexpr int kRows2 = C::kThreads / kPairs;
      static_assert(C::kThreads % kPairs == 0 && BM % kRows2 == 0, "wide store pass shape");
      const int j = tid % kPairs, r0 = tid / kPairs;
      if (m0 + BM <= M && n0 + BN <= N) {
        // whole tile (wave-uniform test): no per-row guard, the row address
        // advances by a scalar stride, and the LDS reads of a batch are all
        // issued before its stores (kRows2 is even, so r % 2 == r0 % 2)
        constexpr int kIters = BM / kRows2, kBatch = 8;
        static_assert(kRows2 % 2 == 0 && kIters % kBatch == 0, "store batch shape");
        // odd rows hold each pair's two 8-byte halves swapped: undone with a
        // per-lane bit mask (a select on the whole vector compiles to
        // exec-masked moves, each waiting for its LDS read)
        const uint32_t odd = (r0 & 1) ? 0xFFFFFFFFu : 0u;
        auto pick = [odd](uint32_t x, uint32_t y) { return (x & ~odd) | (y & odd); };
        uint16_t* crow = c + (m0 + r0) * ldc + n0 + 8 * j;
        const int64_t rstep = kRows2 * ldc;
#pragma unroll
        for (int b0 = 0; b0 < kIters; b0 += kBatch) {
          uint4 o[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int r = r0 + (b0 + u) * kRows2;
            const uint4 v = *reinterpret_cast<const uint4*>(lds + r * (BN * 2) + (j ^ ((r & 31) >> 1)) * 16);
            o[u] = make_uint4(pick(v.x, v.z), pick(v.y, v.w), pick(v.z, v.x), pick(v.w, v.y));
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u) st_stream16(reinterpret_cast<uint4*>(crow + (b0 + u) * rstep), o[u]);
        }
      } else {
        const bool n_ok = n0 + 8 * j < N;  // N % 16 == 0: a 16-byte piece is wholly inside or outside
#pragma unroll 4
        for (int r = r0; r < BM; r += kRows2) {
          const int s = r & 31;
          const uint4 v = *reinterpret_cast<const uint4*>(lds + r * (BN * 2) + (j ^ (s >> 1)) * 16);
          const uint4 o = (s & 1) ? make_uint4(v.z, v.w, v.x, v.y) : v;
          if (n_ok && m0 + r < M) st_stream16(reinterpret_cast<uint4*>(c + (m0 + r) * ldc + n0 + 8 * j), o);
        }
      }
    } else {
      const int j = tid % kPieces, r0 = tid / kPieces;
      const bool n_ok = n0 + 4 * j < N;  // N % 16 == 0: a piece is wholly inside or outside
#pragma unroll 4
      for (int r = r0; r < BM; r += kRowsPerPass) {
        const uint2 v = *reinterpret_cast<const uint2*>(lds + r * (BN * 2) + (j ^ (r & 31)) * 8);
        if (n_ok && m0 + r < M) st_stream8(reinterpret_cast<uint2*>(c + (m0 + r) * ldc + n0 + 4 * j), v.x, v.y);
      }
    }
  };
  // The tiles whose accumulators live in the accumulator registers (256x256,
  // and 128x128 as two waves of 64x128) stage fp32 instead: the VALU cannot
  // read those registers, so scaling and converting before the regroup
  // costs a register read, a multiply and half a conversion per value on
  // the VALU, one wave per SIMD, and the regroup is VALU-bound.  Here the
  // accumulators go to LDS as they are (16-byte writes straight from the
  // accumulator registers), 128 columns of the tile at a time (BM rows x 128
  // fp32: two passes of 128 KiB for 256x256, one of 64 KiB for 128x128), and
  // the store pass reads each row's values back, multiplies by the row's
  // scale, converts and stores: no register reads, no bf16 shuffling (bench
  // step with the 256x256 tile so: 2.903-2.912 -> 2.890-2.894 ms,
  // alternating the two builds on one box; bit-identical outputs).  Column
  // pass h holds, for wave column wn, the wave's kW-column slice h (kW = 64
  // for 256x256, 128 for 128x128) at LDS columns wn*kW ..; 16-byte chunk k
  // of a row sits at slot k ^ (row % 16), so the 16 rows of a write phase
  // and the 16 lanes of a read phase (one row, chunks tid16 and tid16 + 16)
  // each cover 16 distinct slots.  A lane stores two 4-column pieces (8
  // bytes each; 16 lanes write 128 contiguous bytes of a row).
  constexpr bool kF32Epi =
      (BM == 256 && BN == 256 && WM == 2 && WN == 2) || (BM == 128 && BN == 128 && WM == 2 && WN == 1);
  auto store_tile_f32 = [&]() {
    if constexpr (kF32Epi) {
      constexpr int kPassN = BN / 128;                 // column passes
      constexpr int kPP = C::kTN / kPassN;             // a wave's 32-column blocks per pass
      constexpr int kW = kPP * 32;                     // a wave's columns per pass
      static_assert(WN * kW == 128 && C::kTN % kPassN == 0, "128 staged columns per pass");
      static_assert(BM * 128 * 4 <= STAGES * C::kStage, "a column pass must fit the stage buffers");
      constexpr int kRowBytes = 128 * 4;
      constexpr int kRows = C::kThreads / 16;          // rows per store pass (16 lanes per row)
      constexpr int kPasses = BM / kRows, kBatch = 8;
      static_assert(kPasses % kBatch == 0, "store batch shape");
      // tile-column distance of LDS column 64 + x from LDS column x (x < 64)
      constexpr int kDelta = kW == 64 ? BN / WN : 64;
      const int tid16 = tid & 15, rsub = tid >> 4;
      const bool whole = m0 + BM <= M && n0 + BN <= N;
      wait_vm<0>();
#pragma unroll
      for (int h = 0; h < kPassN; ++h) {
        // every wave is done with the stage buffers (h = 0) / with pass h - 1
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int q = 0; q < C::kTM; ++q) {
          const int r = arow[q];
          uint8_t* rowp = lds + r * kRowBytes;
          const int x = r & 15;
#pragma unroll
          for (int pp = 0; pp < kPP; ++pp)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int k = wn * (kW / 4) + 8 * pp + 2 * j + (l >> 5);
              const v16f& av = acc[h * kPP + pp][q];
              *reinterpret_cast<float4*>(rowp + ((k ^ x) << 4)) =
                  make_float4(av[4 * j + 0], av[4 * j + 1], av[4 * j + 2], av[4 * j + 3]);
            }
        }
        __syncthreads();
        // LDS column 4 * tid16 is tile column 4 * tid16 + h * kW; LDS column
        // 64 + 4 * tid16 is kDelta further on
        const int ncol = 4 * tid16 + h * kW;
        auto row_out = [&](int pass) {
          const int r = pass * kRows + rsub, x = r & 15;
          const uint8_t* rp = lds + r * kRowBytes;
          const float4 u = *reinterpret_cast<const float4*>(rp + ((tid16 ^ x) << 4));
          const float4 v = *reinterpret_cast<const float4*>(rp + (((tid16 + 16) ^ x) << 4));
          const float sc = s_tok[r];
          return make_uint4(bf16x2_rne(u.x * sc, u.y * sc), bf16x2_rne(u.z * sc, u.w * sc),
                            bf16x2_rne(v.x * sc, v.y * sc), bf16x2_rne(v.z * sc, v.w * sc));
        };
        if (whole) {
          // scalar row stride; a batch's LDS reads are issued before its stores
          uint16_t* dst = c + static_cast<int64_t>(m0 + rsub) * ldc + n0 + ncol;
          const int64_t rstep = kRows * ldc;
#pragma unroll
          for (int b0 = 0; b0 < kPasses; b0 += kBatch) {
            uint4 o[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) o[i] = row_out(b0 + i);
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
              st_stream8(reinterpret_cast<uint2*>(dst + (b0 + i) * rstep), o[i].x, o[i].y);
              st_stream8(reinterpret_cast<uint2*>(dst + (b0 + i) * rstep + kDelta), o[i].z, o[i].w);
            }
          }
        } else {
          // N % 16 == 0: each 4-column piece is all inside or all outside
          const bool n_ok0 = n0 + ncol < N, n_ok1 = n0 + ncol + kDelta < N;
#pragma unroll 4
          for (int pass = 0; pass < kPasses; ++pass) {
            const int r = pass * kRows + rsub;
            const uint4 o = row_out(pass);
            if (m0 + r < M) {
              uint16_t* dst = c + static_cast<int64_t>(m0 + r) * ldc + n0 + ncol;
              if (n_ok0) st_stream8(reinterpret_cast<uint2*>(dst), o.x, o.y);
              if (n_ok1) st_stream8(reinterpret_cast<uint2*>(dst + kDelta), o.z, o.w);
            }
          }
        }
      }
    }
  };
  if (!SPLIT || S == 1) {
    if constexpr (kF32Epi) store_tile_f32();
    else store_tile();
    return;
  }
  // Split K: the fp32 partial tile in MFMA fragment order (element r of lane
  // l of sub-tile (p, q) of wave w at ((w*kTN + p)*kTM + q)*1024 + r*64 + l),
  // device-scope stores and loads, no cache maintenance -- the same hand-off
  // as the decode GEMMs.
  auto slot = [&](int b, int p, int q) {
    const size_t t = ((static_cast<size_t>(b) * gridDim.x + bx) * C::kWaves + wave) * C::kTN + p;
    return slab + (t * C::kTM + q) * 1024 + l;
  };
#pragma unroll
  for (int p = 0; p < C::kTN; ++p)
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) {
      float* dst = slot(sp, p, q);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __hip_atomic_store(dst + r * 64, acc[p][q][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(&counters[bx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last) return;
  {
    // value (p, q, r) of split b sits at slot(b, p, q) + 64 r = slot(0, 0, 0) + b * split stride + 64 v;
    // a split's 64 values per lane are one batch (two would not fit beside the tile in 256 registers)
    constexpr int kNV = C::kTN * C::kTM * 16;
    float tot[kNV];
    sum_partials<kNV, 64, 1>(tot, slot(0, 0, 0), static_cast<size_t>(gridDim.x) * (C::kWaves * kNV * 64), S);
#pragma unroll
    for (int p = 0; p < C::kTN; ++p)
#pragma unroll
      for (int q = 0; q < C::kTM; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[p][q][r] = tot[(p * C::kTM + q) * 16 + r];
  }
  if constexpr (kF32Epi) store_tile_f32();
  else store_tile();
  if (tid == 0) __hip_atomic_store(&counters[bx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per output tile, except that a large-tile grid of at least
// two whole rounds (one workgroup per CU, 256 per round) runs with fewer
// workgroups than tiles: workgroup b takes tile b and then tile b + G (G the
// grid size; the first workgroups of the grid get the second tiles, so no
// round is partial, and G is a multiple of 256, so both tiles belong to the
// same XCD's share of the tile order).  The second tile's first loads go
// out while the first one's stores are still draining (its first wait
// covers both), instead of after the workgroup has ended and a new one has
// been dispatched.  Split launches (grid (tiles, S)) always run one tile per
// workgroup.
template <int BM, int BN, int WM, int WN, int OCC, bool SPLIT, bool IL, bool AT = false>
__global__ __launch_bounds__(64 * WM * WN, OCC) void k_w4a8_prefill(
    const uint8_t* __restrict__ a, int lda, const float* __restrict__ as, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ wsc, uint16_t* __restrict__ c, int64_t ldc, int M, int N, int KS, int group_m,
    float* __restrict__ slab, int* __restrict__ counters) {
  prefill_tile<BM, BN, WM, WN, OCC, SPLIT, IL, AT>(blockIdx.x, a, lda, as, w, wsc, c, ldc, M, N, KS, group_m, slab,
                                                   counters);
  if constexpr (IL && !SPLIT) {
    // (two inlined copies rather than a loop: the loop kept state across
    // tiles and spilled)
    const int second = static_cast<int>(blockIdx.x + gridDim.x);
    if (second < ((M + BM - 1) / BM) * ((N + BN - 1) / BN)) {
      __syncthreads();  // every wave is done with the first tile's LDS
      prefill_tile<BM, BN, WM, WN, OCC, SPLIT, IL, AT>(second, a, lda, as, w, wsc, c, ldc, M, N, KS, group_m, slab,
                                                       counters);
    }
  }
}

template <int BM, int BN, int WM, int WN, int OCC, bool SPLIT, bool IL, bool AT>
int launch_cfg(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint8_t* wsc, uint16_t* c,
               int64_t ldc, int M, int N, int KS, int group_m, int S, void* ws, hipStream_t st) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  float* slab = nullptr;
  int* counters = nullptr;
  if (S > 1) {
    if (tiles > kWsMaxCounters) return BS_ERR_SHAPE;  // split only below 256 tiles (prefill_plan)
    counters = static_cast<int*>(ws);
    slab = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kWsCounterBytes);
  }
  // large tiles: the first (tiles / 512) * 256 workgroups take two tiles
  const int grid = IL && !SPLIT ? tiles - (tiles / 512) * 256 : tiles;
  k_w4a8_prefill<BM, BN, WM, WN, OCC, SPLIT, IL, AT><<<dim3(grid, S), 64 * WM * WN, 0, st>>>(
      a, static_cast<int>(lda), as, w, wsc, c, ldc, M, N, KS, group_m, slab, counters);
  return bs_launch_status();
}

// Tile and K-split choice.  256x256 tiles run one workgroup per CU, so a
// grid of T big tiles takes ceil(T / 256) rounds and a partial last round
// costs nearly a whole one (1088 tiles: 335 us against 4 x 67 us).  When
// there are at least 256 big tiles, the big-tile launch takes the widest
// column range [0, n_main) whose tile count is a whole number of rounds --
// n_main / 256 a multiple of 256 / gcd(m_tiles, 256) -- and the remaining
// column strip (less than one round of big tiles) runs as 128x128 tiles,
// two workgroups per CU.  Below 256 big tiles everything runs as small tiles
// (that way 320 tiles ran 20% faster than as big ones).  The small tiles
// have the same problem one level down: more than 512 of them (two per CU)
// with a partial last round are cut the same way, the widest column range
// [n_main, n_mid) that fills whole rounds runs unsplit, and only the
// remaining columns go to the split launch.  Small-tile grids under 256
// tiles split K so that about 256 workgroups run, keeping at least 8 K steps
// (1024 K) per split (measured with the batched split-K reduction: 80 tiles
// run fastest with 3 splits, 160 tiles unsplit -- 512 workgroups were 10-20%
// slower; 129 to 256 tiles, such as the column strips, run faster unsplit,
// over a long K too since split launches of more than 256 workgroups take
// the two-wave tile: M = 4096 N = 5120 K = 17408 243-253 -> 238-242 us,
// M = 1024 N = 2560 K = 17408 61-63 -> 56-59 us against two splits).
struct PrefillPlan {
  int n_main;   // columns [0, n_main) as 256x256 tiles (0: none)
  int n_mid;    // columns [n_main, n_mid) as unsplit 128x128 tiles, whole rounds of 512
  int s;        // K splits of the small-tile launch over columns [n_mid, N)
  int tiles;    // small tiles of that launch (0: none)
};
PrefillPlan prefill_plan(int M, int N, int K) {
  const int KS = K / 128;
  const int mt = (M + 255) / 256, nt = (N + 255) / 256;
  PrefillPlan p{0, 0, 1, 0};
  if (mt * nt >= 256) {
    p.n_main = N;
    if ((mt * nt) % 256 != 0) {
      const int g = 256 / std::gcd(mt, 256);   // n-tile multiple that fills whole rounds
      const int n1 = (nt - 1) / g * g;
      if (n1 >= 1 && mt * (nt - n1) < 256) p.n_main = n1 * 256;
    }
  }
  p.n_mid = p.n_main;
  const int mts = (M + 127) / 128;
  const int nts = (N - p.n_main + 127) / 128;
  if (mts * nts > 512 && (mts * nts) % 512 != 0) {
    const int g = 512 / std::gcd(mts, 512);
    const int n1 = (nts - 1) / g * g;
    if (n1 >= 1) p.n_mid = p.n_main + n1 * 128;
  }
  const int ns = N - p.n_mid;
  if (ns > 0) {
    p.tiles = mts * ((ns + 127) / 128);
    if (p.tiles < 256) p.s = std::max(1, std::min(256 / p.tiles, KS / 8));
    p.s = std::min(p.s, 0x7FFFFFFF / KS);  // the split bounds are computed as KS * index in 32 bits
  }
  return p;
}

}  // namespace

size_t bs_prefill_workspace(int M, int N, int K) {
  const PrefillPlan pl = prefill_plan(M, N, K);
  if (pl.tiles == 0 || pl.s <= 1) return 0;
  return kWsCounterBytes + static_cast<size_t>(pl.s) * pl.tiles * 128 * 128 * sizeof(float);
}

namespace {
// The tile plan's launches; a_tiled selects the activation-tiled input order.
template <bool AT>
int launch_plan(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc, uint16_t* c,
                int64_t ldc, int M, int N, int K, void* ws, hipStream_t st) {
  const int KS = K / 128;
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(wsc);
  const PrefillPlan pl = prefill_plan(M, N, K);
  if (pl.n_main > 0) {
    const int rc = launch_cfg<256, 256, 2, 2, 1, false, true, AT>(a, lda, as, w, sc, c, ldc, M, pl.n_main, KS, 4, 1,
                                                                   nullptr, st);
    if (rc != BS_OK || pl.tiles == 0) return rc;
  }
  // a small-tile launch over columns [n0, n1): the weight's n-tiles from
  // n0 / 16 on (codes KS KiB and scales ceil(KS/4) * 256 bytes per
  // 16-column tile), output columns from n0 on
  // More small-tile workgroups than CUs run two waves of 64 x 128 per tile:
  // two such workgroups share a CU with half the LDS fragment reads of four
  // 64 x 64 waves each, which held those launches back (M = 512 N = 10240
  // K = 5120: 39.6-41.1 -> 34.0-35.4 us, M = 1024 N = 5120 K = 17408
  // 105-110 -> 91-92 us, M = 256 N = 34816 60-66 -> 57-59 us).  With at most
  // one workgroup per CU, two waves would leave two SIMDs idle (M = 256
  // N = 10240: 23.4-23.8 -> 27.3-28.0 us), so those keep four.
  auto small = [&](int n0, int n1, int s, void* work) {
    const size_t nt_off = static_cast<size_t>(n0) / 16;
    const uint8_t* wn = w + nt_off * KS * 1024;
    const uint8_t* sn = sc + nt_off * ((KS + 3) / 4) * 256;
    const int wgs = ((M + 127) / 128) * ((n1 - n0 + 127) / 128) * s;
    if (wgs > 256)
      return launch_cfg<128, 128, 2, 1, 1, true, false, AT>(a, lda, as, wn, sn, c + n0, ldc, M, n1 - n0, KS, 4, s,
                                                            work, st);
    return launch_cfg<128, 128, 2, 2, 2, true, false, AT>(a, lda, as, wn, sn, c + n0, ldc, M, n1 - n0, KS, 4, s, work,
                                                          st);
  };
  if (pl.n_mid > pl.n_main) {
    const int rc = small(pl.n_main, pl.n_mid, 1, nullptr);
    if (rc != BS_OK || pl.tiles == 0) return rc;
  }
  return small(pl.n_mid, N, pl.s, ws);
}
}  // namespace

int bs_launch_w4a8_prefill(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                           uint16_t* c, int64_t ldc, int M, int N, int K, void* ws, bool a_tiled, hipStream_t st) {
  return a_tiled ? launch_plan<true>(a, lda, as, w, wsc, c, ldc, M, N, K, ws, st)
                 : launch_plan<false>(a, lda, as, w, wsc, c, ldc, M, N, K, ws, st);
}
