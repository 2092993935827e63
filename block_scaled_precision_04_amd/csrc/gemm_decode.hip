// Small-M (decode) block-scaled GEMMs: a weight stream through MFMA.
//
// Block-FP8 W8A8 (radiance_kernels.py page, block_scaled_mm: e4m3 weights with
// one scale per 128x128 block, e4m3 activations with one scale per token per
// 128-wide K group) and MXFP4 W4A8 at small M (radiance_mxfp4.py page: the
// decode band, the fragment-order weight that makes a wave's weight read
// contiguous, and split-K for shapes with too little N to fill the GPU; the
// decode split-K scratch whose last-arriving block reduces and resets it).
//
// At M <= 64 the weight bytes dominate: the arithmetic intensity is far below
// the MFMA ridge, so the kernel is built to keep HBM busy and to spend as few
// memory instructions as possible on anything but the weight:
//   * the weight was pre-laid-out in fragment order, so one (16-row tile,
//     128-K step) is one contiguous 2 KiB (fp8) / 1 KiB (fp4) block and each
//     lane issues 16-byte loads;
//   * a wave owns T 16-column tiles over the R K steps of its split and
//     issues all of its weight loads at once, straight into registers;
//   * the activation slice of a split (R steps x up to 16*MB rows) is copied
//     once per workgroup into LDS by direct-to-LDS loads in which every lane
//     fetches useful bytes, and the TW*T tiles of the workgroup read their
//     MFMA fragments from there -- per-wave activation loads (half of whose
//     lanes repeat rows when M < 16) cost as many memory instructions as the
//     weight itself;
//   * when K has more than one split, the last workgroup of a tile group to
//     finish (atomic counter) adds the S fp32 partials in split order, then
//     resets its counter -- deterministic, and the workspace stays ready;
//   * one rounding to bf16 at the end.
// Every load is unconditional: rows past M and steps past K re-read valid
// bytes and are masked afterwards, because loads inside data-dependent
// branches make the compiler wait for all outstanding loads at each branch.
// The MFMA puts the weight tile in the first operand (rows = n) and the
// activations in the second (rows = m), so D[n][m] and each lane holds four
// consecutive n of one m.
//
// Block-FP8: every 16x16x128 MFMA covers exactly one 128-wide scale group, so
// its result (fresh accumulator) is scaled by a_scale[m,g] * w_scale[n/128,g]
// and added into an fp32 accumulator.  MXFP4: the scaled MFMA applies the e8m0
// weight scales in hardware (activation scale byte 127 = 1.0) and accumulates;
// the per-token activation scale multiplies the sum at the end.  The fp8 x fp8
// fragments hold K offsets 32*(l/16) .. +32 on both sides; an 8-bit operand
// paired with a 4-bit one holds 16g.. and 64+16g.. (gfx950), while the 4-bit
// operand holds 32g..32g+31, so the activation fragment follows the hardware's
// 8-bit order and real K lines up with the weight.
#include <algorithm>

#include "common.h"

namespace {

BS_INLINE v8i pack8(uint4 x, uint4 y) {
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}
// 16-byte chunk swizzle of an activation row in LDS: the 16 rows of an MFMA
// fragment read the same chunk index, and this permutation spreads them over
// distinct bank groups whether the LDS serves 8 or 16 lanes of a 128-bit read
// per cycle.
BS_INLINE int a_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
BS_INLINE v4f mfma_fp8(v8i w, v8i a, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 0, 0, 0, 127, 0, 127);
}
BS_INLINE v4f mfma_fp4w_fp8a(v8i w, v8i a, v4f c, int wscale) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 4, 0, 0, wscale, 0, 127);
}

struct DecodeArgs {
  const uint8_t* a;
  int64_t lda;
  const float* as;      // fp8: a_scale base; mx: per-token scale [M]
  int64_t as_m, as_g;   // fp8 strides
  const uint8_t* w;     // pre-laid-out codes
  const float* wsf;     // fp8: w_scale [N/128, K/128]
  const uint32_t* wsx;  // mx: e8m0 section
  uint16_t* c;
  int64_t ldc;
  int M, N, KS;
  int rs;               // activation rows staged per workgroup: min(M, 16*MB)
  float* slab;          // fp32 partials in fragment order when gridDim.y > 1
  int* counters;        // [gridDim.z][gridDim.x]
};

// Vector loads of the weight side issued after the activation DMA (the DMA is
// complete once at most this many loads are outstanding).
template <bool MX, int T, int R>
constexpr int weight_loads() {
  return MX ? T * R + T * ((R + 3) / 4) : 2 * T * R + 1;
}

// grid (ceil(N/16 / (TW*T)), S, ceil(M / (16*MB))); TW*KW waves.
// Workgroup (x, y, z) covers n-tiles [x*TW*T, (x+1)*TW*T) over the K steps
// [y*KW*R, (y+1)*KW*R) for activation rows [16*MB*z, 16*MB*(z+1)).  Wave
// (tw, kw) owns T of the tiles over the kw-th run of R steps; the KW partial
// sums of a tile are added through LDS in kw order.
// LDS: the activation slice (KW*R steps x rs rows x 128 B, as 16-byte chunks)
// and, for block-FP8, its scales [KW*R][rs]; the cross-wave partials reuse the
// slice after the MFMAs.
// At most 256 threads per workgroup (one wave per SIMD) give the compiler a
// 512-register budget, and it then accumulates the 16x16x128 scaled MFMA in
// the accumulator registers (AGPRs).  The one decode configuration ever built
// that way (MXFP4, TW=2 KW=2 T=1 R=8) gave wrong results on the GPU although
// its indexing is exact and the compiler's wait states before reading the
// AGPRs follow the 8-pass rules; every configuration in use accumulates in
// ordinary VGPRs.  So that form is kept out of this kernel.
template <bool MX, int MB, int TW, int KW, int T, int R>
__global__ __launch_bounds__(TW * KW * 64) void k_decode(DecodeArgs p) {
  static_assert(TW * KW > 4, "<= 4 waves per workgroup puts the accumulators in AGPRs (see above)");
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int last;
  constexpr int kThreads = TW * KW * 64;
  constexpr int kSteps = KW * R;  // K steps per workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tw = wave % TW, kw = wave / TW;
  const int l = threadIdx.x & 63, g = l >> 4;
  const int split = blockIdx.y, S = gridDim.y;
  const int m0 = blockIdx.z * 16 * MB;
  const int KS = p.KS, RS = p.rs;
  const int wg_k0 = split * kSteps;
  const int wg_steps = min(kSteps, KS - wg_k0);
  const int ks0 = wg_k0 + kw * R;
  const int klast = min(ks0 + R, KS) - 1;  // >= 0; below ks0 for an idle wave
  const int nsteps = klast - ks0 + 1;      // <= 0 for an idle wave
  const int rows = min(RS, p.M - m0);
  const int ntiles = p.N >> 4;
  const int tile0 = (blockIdx.x * TW + tw) * T;
  const int KQ = (KS + 3) >> 2;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const int a_instr = (kSteps * RS * 8 + 63) >> 6;
  float* s_as = reinterpret_cast<float*>(lds + a_instr * 1024);
  float* s_red = reinterpret_cast<float*>(lds);  // reuses the slice once every wave is done with it

  // ---- 1. activation slice -> LDS (direct DMA, every lane useful).  Chunk c
  // (16 B) of row i of step r sits at position (r*RS + i)*8 + (c ^ a_swz(i)).
  // Positions past the slice, or rows past M in the last row block, re-read
  // valid bytes that are never used.
  {
    const uint8_t* abase = p.a + static_cast<int64_t>(m0) * p.lda + static_cast<int64_t>(wg_k0) * 128;
    for (int k = wave; k < a_instr; k += TW * KW) {
      const int q = k * 64 + l;
      const int r = min(q / (RS * 8), wg_steps - 1);
      const int ii = (q >> 3) % RS;
      const int i = min(ii, rows - 1);
      const int c = (q & 7) ^ a_swz(ii);
      dma16(lds0 + k * 1024, abase, static_cast<uint32_t>(i * p.lda + r * 128 + c * 16));
    }
  }
  // block-FP8 activation scales of the slice (written to LDS below)
  constexpr int kSPer = (kSteps * 16 * MB + kThreads - 1) / kThreads;
  float sv[kSPer];
  if constexpr (!MX) {
#pragma unroll
    for (int j = 0; j < kSPer; ++j) {
      const int e = min(static_cast<int>(threadIdx.x) + j * kThreads, kSteps * RS - 1);
      const int r = min(e / RS, wg_steps - 1), i = min(e % RS, rows - 1);
      sv[j] = p.as[(m0 + i) * p.as_m + (wg_k0 + r) * p.as_g];
    }
  }
  // block-FP8 weight scales of the wave's T tiles x R steps, one per lane
  // (read back per step with a lane broadcast)
  float wsv = 0.0f;
  if constexpr (!MX) {
    static_assert(T * R <= 64, "one weight scale per lane");
    const int j = min(l, T * R - 1);
    const int tj = min(tile0 + j / R, ntiles - 1);
    wsv = p.wsf[static_cast<size_t>(tj >> 3) * KS + min(ks0 + j % R, klast)];
  }
  // The scale loads stay ahead of the weight loads: the LDS store of the
  // activation scales below waits for them, and with the weight loads issued
  // first that wait would cover the whole weight stream too.
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. the wave's weight fragments (all R steps of its T tiles) ---------
  // Every weight byte is read by exactly one wave: streaming loads.
  v8i wf[T][R];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const size_t tile = static_cast<size_t>(min(tile0 + t, ntiles - 1)) * KS;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t ks = min(ks0 + r, klast);
      if constexpr (MX) {
        const uint4 x = ld_stream16(reinterpret_cast<const uint4*>(p.w + (tile + ks) * 1024 + l * 16));
        wf[t][r] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      } else {
        const uint8_t* src = p.w + (tile + ks) * 2048 + l * 16;
        wf[t][r] = pack8(ld_stream16(reinterpret_cast<const uint4*>(src)),
                         ld_stream16(reinterpret_cast<const uint4*>(src + 1024)));
      }
    }
  }
  // mx: one e8m0 dword per lane covers four steps (ks0 is a multiple of 4)
  uint32_t sd[T][(R + 3) / 4];
  if constexpr (MX) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int qd = 0; qd < (R + 3) / 4; ++qd)
        sd[t][qd] = p.wsx[(static_cast<size_t>(min(tile0 + t, ntiles - 1)) * KQ + min((ks0 >> 2) + qd, klast >> 2)) * 64 + l];
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!MX) {
#pragma unroll
    for (int j = 0; j < kSPer; ++j) {
      const int e = static_cast<int>(threadIdx.x) + j * kThreads;
      if (e < kSteps * RS) s_as[e] = sv[j];
    }
  }
  wait_vm<weight_loads<MX, T, R>()>();  // this wave's activation DMA has landed
  __syncthreads();

  // ---- 3. MFMA over the slice ---------------------------------------------
  v4f acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = v4f{0, 0, 0, 0};
  // Lanes whose row is past M compute garbage in their own output column only
  // (never stored), so only the steps past this wave's range need care.
  // Where two fragment sets fit in 128 VGPRs (four waves per SIMD), the
  // fragments of step r+1 are read from LDS before the MFMAs of step r, so
  // the LDS latency runs under them.  That form runs every step and zeroes
  // the products of those past the range (MXFP4: the weight fragment;
  // block-FP8: the step's scale), which meet clamped re-reads of this wave's
  // last step: an and-mask, because with a branch per step the compiler sinks
  // the MFMAs below the branches and the read-ahead is lost.  Otherwise each
  // step reads its own fragments just before its MFMAs and the loop ends at
  // the range's end (the mask-and-run form costs these registers: M = 64
  // block-FP8 with 8 tiles of 8 steps went from 123 to 129 VGPRs).
  constexpr bool kPipeA = T * R * (MX ? 4 : 8) + 2 * MB * (MX ? 8 : 9) + T * MB * 4 + 16 <= 128;
  constexpr int kSets = kPipeA ? 2 : 1;
  v8i af[kSets][MB];
  float sa[kSets][MB];
  auto read_a = [&](int r, v8i (&f)[MB], float (&sf)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int rc = min(16 * mb + (l & 15), RS - 1);
      const int c0 = MX ? g : 2 * g, c1 = MX ? 4 + g : 2 * g + 1;
      const uint8_t* rb = lds + ((kw * R + r) * RS + rc) * 128;
      const uint4 x = *reinterpret_cast<const uint4*>(rb + ((c0 ^ a_swz(rc)) << 4));
      const uint4 y = *reinterpret_cast<const uint4*>(rb + ((c1 ^ a_swz(rc)) << 4));
      f[mb] = pack8(x, y);
      if constexpr (!MX) sf[mb] = s_as[(kw * R + r) * RS + rc];
    }
  };
  if constexpr (kPipeA) read_a(0, af[0], sa[0]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int cur = kPipeA ? (r & 1) : 0;
    if constexpr (kPipeA) {
      if (r + 1 < R) read_a(r + 1, af[(r + 1) & 1], sa[(r + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (r >= nsteps) break;
      read_a(r, af[0], sa[0]);
    }
    const int live = kPipeA && r >= nsteps ? 0 : -1;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (MX) {
        const int sc = static_cast<int>(sd[t][r >> 2] >> (8 * (r & 3)));
        const v8i wm = wf[t][r] & live;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_fp4w_fp8a(wm, af[cur][mb], acc[t][mb], sc);
      } else {
        // (block-FP8 scales each product anyway: a zero scale drops the step)
        const float sw =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsv), t * R + r) & live);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const v4f tmp = mfma_fp8(wf[t][r], af[cur][mb], v4f{0, 0, 0, 0});
          acc[t][mb] += tmp * (sa[cur][mb] * sw);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 4. add the KW partials of each tile in kw order ----------------------
  if constexpr (KW > 1) {
    constexpr int kPer = T * MB * 4;  // floats per lane
    __syncthreads();  // the activation slice is dead from here on
    if (kw > 0) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s_red[(((kw - 1) * TW + tw) * kPer + (t * MB + mb) * 4 + j) * 64 + l] = acc[t][mb][j];
    }
    __syncthreads();
    if (kw == 0)
#pragma unroll
    for (int u = 1; u < KW; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[t][mb][j] += s_red[(((u - 1) * TW + tw) * kPer + (t * MB + mb) * 4 + j) * 64 + l];
  }

  // ---- 5. output: lane l holds C[m = l%16 (+16 mb)][n = 4(l/16) .. +3] -------
  auto store_bf16x4 = [&](int m, int n, v4f v) {
    const uint32_t lo = bf16x2_rne(v[0], v[1]);
    const uint32_t hi = bf16x2_rne(v[2], v[3]);
    *reinterpret_cast<uint2*>(p.c + m * p.ldc + n) = uint2{lo, hi};
  };
  // (waves with kw > 0 stay to the end: they take part in every barrier)
  const bool owner = kw == 0;
  if (S == 1) {
    if (owner)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = m0 + 16 * mb + (l & 15), n = (tile0 + t) * 16 + 4 * g;
          if (m < p.M && tile0 + t < ntiles) store_bf16x4(m, n, MX ? acc[t][mb] * p.as[m] : acc[t][mb]);
        }
    return;
  }
  // Split K: fp32 partials, then the last workgroup of this tile group adds
  // them in split order.  The partials keep the MFMA fragment order -- slot
  // (split, z, x, tw, t, mb) holds 4 x 64 floats, element j of lane l at
  // j*64 + l -- so every store and load instruction covers 256 contiguous
  // bytes.  They are device-scope stores (written through to the
  // device-coherent level) read back with device-scope loads, so the hand-off
  // needs no cache maintenance: each wave waits for its stores to be
  // acknowledged before the counter increment.  (A device-scope fence would
  // write back and invalidate the L2 of every XCD that runs a split --
  // microseconds per workgroup.)
  auto frag = [&](int sp, int t, int mb) {
    const size_t f = ((((static_cast<size_t>(sp) * gridDim.z + blockIdx.z) * gridDim.x + blockIdx.x) * TW + tw) * T + t) * MB + mb;
    return p.slab + f * 256 + l;
  };
  if (owner)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float* dst = frag(split, t, mb);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __hip_atomic_store(dst + j * 64, acc[t][mb][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  __syncthreads();
  const int cidx = blockIdx.z * gridDim.x + blockIdx.x;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&p.counters[cidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!last || !owner) return;
  // value (t, mb, j) of split b sits at frag(b, t, mb) + 64 j = frag(0, 0, 0) + b * split stride + 64 v
  constexpr int kNV = T * MB * 4;
  constexpr int kU = kNV >= 32 ? 2 : (kNV >= 16 ? 4 : 8);
  float tot[kNV];
  sum_partials<kNV, 64, kU>(tot, frag(0, 0, 0),
                            static_cast<size_t>(gridDim.z) * gridDim.x * (TW * T * MB * 256), S);
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int v = (t * MB + mb) * 4;
      const v4f sum = v4f{tot[v], tot[v + 1], tot[v + 2], tot[v + 3]};
      const int m = m0 + 16 * mb + (l & 15), n = (tile0 + t) * 16 + 4 * g;
      if (m < p.M && tile0 + t < ntiles) store_bf16x4(m, n, MX ? sum * p.as[m] : sum);
    }
  if (threadIdx.x == 0) __hip_atomic_store(&p.counters[cidx], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct DecodeCfg {
  int mb, tw, kw, t, r, s, groups, mblocks, rs;
};

// LDS the hardware grants one workgroup, less this kernel's static part.
constexpr size_t kMaxDecodeLds = 160 * 1024 - 256;

// Tile-waves (TW), K-waves (KW), n-tiles per wave (T) and K steps per wave
// (R) for a small-M shape; S workgroups split the rest of K.  Chosen from
// sweeps of the decode shapes on MI355X (graph-replayed, weights pooled past
// the Infinity Cache): for M <= 16 the activation slice is small, so one or
// two tiles per workgroup and many K-waves keep thousands of waves streaming;
// for larger M the slice (8 KiB per step at M = 64) is shared by 4-8 tiles
// over fewer steps.  Long K (>= 96 steps) and wide N (>= 512 tiles) run
// 8-wave workgroups with a 64 KiB slice, two per CU, which split K further
// now that the split-K reduction costs a few round trips (M = 32 / 64:
// K = 17408 8-15% and N = 10240 10-14% faster than the 16-wave workgroup,
// which stays best at N = K = 5120).  At M <= 16, block-FP8 with at most 20
// K steps runs 8-wave workgroups (M = 16 N = 512 K = 1024: 5.3 -> 4.2 us)
// and wide N one tile per workgroup (M = 8 N = 10240: 13.1 -> 11.9 us).
// MXFP4 needs R % 4 == 0 (one e8m0 dword per lane covers four steps).
DecodeCfg decode_cfg(int M, int N, int KS, bool mx) {
  DecodeCfg d{};
  d.mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  d.mblocks = (M + 16 * d.mb - 1) / (16 * d.mb);
  d.rs = std::min(M, 16 * d.mb);
  const bool long_k = KS >= 96, wide_n = N / 16 >= 512;
  auto set = [&](int tw, int kw, int t, int r) { d.tw = tw; d.kw = kw; d.t = t; d.r = r; };
  if (d.mb == 1 && mx) {
    // At 16 staged rows the 40-step slice (80 KiB) would leave one workgroup
    // per CU, so halve the K-waves and give each wave two tiles (M = 16:
    // N = 17408 20 -> 16 us, N = 34816 36 -> 26 us).  From 5 rows and 640
    // tiles on, three tiles per workgroup share the slice (M = 8: N = 17408
    // 12.7 -> 11.5 us, N = 34816 20.6 -> 17.7 us; slower at N = 5120 and
    // below 5 rows).
    const bool slice_halves_lds = static_cast<size_t>(d.rs) * 40 * 128 > kMaxDecodeLds / 2;
    // long K: 12 waves of 8 steps (re-swept: M = 8 N = 5120 K = 17408
    // 13.5 -> 12.4 us against TW=4 KW=2)
    if (long_k) set(4, 3, 1, 8);
    else if (slice_halves_lds) set(1, 5, 2, 4);
    else if (M >= 5 && N / 16 >= 640) set(3, 5, 1, 8);
    else set(1, 10, 1, 4);
  } else if (d.mb == 1) {
    // wide N whose 40-step slice takes more than half the LDS (16 rows):
    // 8 waves of 10 steps (M = 16, K = 5120: N = 10240 16.8 -> 15.4 us,
    // N = 17408 26.1 -> 22.7 us; up to 12 rows 10 waves of 4 stay faster)
    const bool slice_halves_lds = static_cast<size_t>(d.rs) * 40 * 128 > kMaxDecodeLds / 2;
    if (KS <= 20) set(2, 4, 1, 5);  // few K steps: fewer idle K-waves
    else if (wide_n && !long_k && !slice_halves_lds) set(1, 10, 1, 4);
    // 40 steps per workgroup as 8 waves of 10 rather than 16 of 5: half the
    // waves to launch for the same loads in flight (M = 8 N = 5120: K = 5120
    // 7.5 -> 7.3 us, K = 17408 24.0 -> 20.7 us; M = 8 N = 10240 K = 17408
    // 40.6 -> 35.3 us; M = 16 K = 17408 unchanged)
    else set(2, 4, 1, 10);
  } else if (mx) {
    set(8, 1, 1, 8);
  } else if (long_k) {
    // 33..64 rows: 8 tiles x 8 steps per workgroup (re-swept once the scale
    // loads stopped holding up the weight stream: M = 64 K = 17408 34.4 ->
    // 32.2 us against TW=4 KW=2 R=4)
    d.mb == 2 ? set(4, 2, 1, 8) : set(8, 1, 1, 8);
  } else if (wide_n) {
    set(8, 1, 1, 8);
  } else {
    // 33..64 rows: two K-waves of 8 steps (M = 48 / 64, N = K = 5120:
    // 12.84 / 13.27 -> 12.41 / 12.98 us against four K-waves of 4 steps)
    d.mb == 2 ? set(4, 2, 1, 4) : set(4, 2, 1, 8);
  }
  const int ntiles = N / 16;
  d.groups = (ntiles + d.tw * d.t - 1) / (d.tw * d.t);
  d.s = (KS + d.kw * d.r - 1) / (d.kw * d.r);
  return d;
}

size_t decode_lds_bytes(const DecodeCfg& d, bool mx) {
  const int steps = d.kw * d.r;
  const size_t a = static_cast<size_t>((steps * d.rs * 8 + 63) / 64) * 1024;
  const size_t sc = mx ? 0 : static_cast<size_t>(steps) * d.rs * sizeof(float);
  const size_t red = static_cast<size_t>(d.kw - 1) * d.tw * d.t * d.mb * 4 * 64 * sizeof(float);
  return std::max(a + sc, red + sc);
}

}  // namespace

// Rows per launch: larger M runs as consecutive 64-row launches that share the
// workspace (stream order keeps them apart), so the split-K slab stays small.
constexpr int kDecodeRows = 64;

namespace {
size_t slab_bytes(const DecodeCfg& d) {
  return static_cast<size_t>(d.s) * d.mblocks * d.groups * d.tw * d.t * d.mb * 256 * sizeof(float);
}

// Workspace: kWsCounterBytes of counters (one per tile group and row block
// of a launch), then the slab, sized for the largest of the call's row
// chunks (full 64-row chunks and the remainder can differ in configuration).
struct DecodeWs {
  size_t slab;      // bytes
  int max_counters;
};
DecodeWs decode_ws(int M, int N, int K, bool mx) {
  DecodeWs w{0, 0};
  for (int rows : {std::min(M, kDecodeRows), M > kDecodeRows ? M % kDecodeRows : 0}) {
    if (rows <= 0) continue;
    const DecodeCfg d = decode_cfg(rows, N, K / 128, mx);
    if (d.s <= 1) continue;
    w.slab = std::max(w.slab, slab_bytes(d));
    w.max_counters = std::max(w.max_counters, d.groups * d.mblocks);
  }
  return w;
}

}  // namespace

size_t bs_decode_workspace(int M, int N, int K, bool mx) {
  const DecodeWs w = decode_ws(M, N, K, mx);
  return w.slab ? kWsCounterBytes + w.slab : 0;
}

namespace {

int launch_decode(bool mx, DecodeArgs& p, void* ws, hipStream_t st) {
  const DecodeCfg d = decode_cfg(p.M, p.N, p.KS, mx);
  if (d.s > 1) {
    p.counters = static_cast<int*>(ws);
    p.slab = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kWsCounterBytes);
  }
  p.rs = d.rs;
  dim3 grid(d.groups, d.s, d.mblocks);
  dim3 block(64 * d.tw * d.kw);
  const size_t lds = decode_lds_bytes(d, mx);
  if (lds > kMaxDecodeLds) return BS_ERR_SHAPE;  // a dispatch beyond the LDS size aborts the queue
  // Each instantiation raises its dynamic-LDS limit once, before its first launch.
#define BS_DEC(MX_, MB_, TW_, KW_, T_, R_)                                                                 \
  do {                                                                                                     \
    auto* fn = &k_decode<MX_, MB_, TW_, KW_, T_, R_>;                                                      \
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                  \
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,         \
                                                       static_cast<int>(kMaxDecodeLds));                   \
    if (attr != hipSuccess) return BS_ERR_LAUNCH;                                                          \
    fn<<<grid, block, lds, st>>>(p);                                                                       \
  } while (0)
  // one instantiation per configuration decode_cfg can return
  const int key = ((d.tw * 100 + d.kw) * 10 + d.t) * 100 + d.r;  // TW, KW, R < 100, T < 10
  if (mx) {
    if (d.mb == 1 && key == 110104) BS_DEC(true, 1, 1, 10, 1, 4);
    else if (d.mb == 1 && key == 403108) BS_DEC(true, 1, 4, 3, 1, 8);
    else if (d.mb == 1 && key == 105204) BS_DEC(true, 1, 1, 5, 2, 4);
    else if (d.mb == 1 && key == 305108) BS_DEC(true, 1, 3, 5, 1, 8);
    else if (d.mb == 2 && key == 801108) BS_DEC(true, 2, 8, 1, 1, 8);
    else if (d.mb == 4 && key == 801108) BS_DEC(true, 4, 8, 1, 1, 8);
    else return BS_ERR_SHAPE;
  } else {
    if (d.mb == 1 && key == 204110) BS_DEC(false, 1, 2, 4, 1, 10);
    else if (d.mb == 1 && key == 204105) BS_DEC(false, 1, 2, 4, 1, 5);
    else if (d.mb == 1 && key == 110104) BS_DEC(false, 1, 1, 10, 1, 4);
    else if (d.mb == 2 && key == 402104) BS_DEC(false, 2, 4, 2, 1, 4);
    else if (d.mb == 2 && key == 402108) BS_DEC(false, 2, 4, 2, 1, 8);
    else if (d.mb == 2 && key == 801108) BS_DEC(false, 2, 8, 1, 1, 8);
    else if (d.mb == 4 && key == 402108) BS_DEC(false, 4, 4, 2, 1, 8);
    else if (d.mb == 4 && key == 801108) BS_DEC(false, 4, 8, 1, 1, 8);
    else return BS_ERR_SHAPE;
  }
#undef BS_DEC
  return bs_launch_status();
}

}  // namespace

// Internal entry points used by the ABI layer (gemm_abi.hip).
int bs_launch_fp8_block_decode(const uint8_t* a, int64_t lda, const float* as, int64_t asm_, int64_t asg,
                               const uint8_t* w, const float* ws, uint16_t* c, int64_t ldc, int M, int N, int K,
                               void* work, hipStream_t st) {
  if (decode_ws(M, N, K, false).max_counters > kWsMaxCounters) return BS_ERR_SHAPE;
  for (int r0 = 0; r0 < M; r0 += kDecodeRows) {
    DecodeArgs p{a + r0 * lda, lda, as + r0 * asm_, asm_, asg, w, ws, nullptr, c + r0 * ldc, ldc,
                 std::min(kDecodeRows, M - r0), N, K / 128, 0, nullptr, nullptr};
    const int st_ = launch_decode(false, p, work, st);
    if (st_ != BS_OK) return st_;
  }
  return BS_OK;
}

int bs_launch_w4a8_decode(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                          uint16_t* c, int64_t ldc, int M, int N, int K, void* work, hipStream_t st) {
  if (decode_ws(M, N, K, true).max_counters > kWsMaxCounters) return BS_ERR_SHAPE;
  DecodeArgs p{a, lda, as, 0, 0, w, nullptr, wsc, c, ldc, M, N, K / 128, 0, nullptr, nullptr};
  return launch_decode(true, p, work, st);
}
