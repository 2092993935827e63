// Large-M (prefill) MXFP4 W4A8 GEMM on gfx950 scaled MFMA.
//
// The radiance_mxfp4.py page (module docstring) explains why this path is
// hand-written: the compiler route upconverts e2m1 to 16 bits and never
// issues the low-precision matrix instruction, while the hardware's own
// 8-bit matrix instruction is about twice as fast.  On gfx950 the scaled
// MFMA V_MFMA_SCALE_F32_32X32X64_F8F6F4 takes the e2m1 weight and the e4m3
// activation directly and applies the MX e8m0 block scale (one per 32 K) in
// hardware, so the exact dequantised product of the page's _exact_ref is
// accumulated in fp32 with no software decode at all.
//
// Tiling: a workgroup computes a BM x BN output tile with WM x WN waves; each
// wave owns (BM/WM) x (BN/WN) as 32x32 MFMA sub-tiles with fp32 accumulators.
// K advances in 128-wide steps.  Each step's activation tile (BM x 128 bytes,
// row pitch padded to avoid LDS bank conflicts) and weight tile (BN/16
// fragment-order 1 KiB blocks, copied as they are) are staged through LDS,
// double buffered: the global loads of step k+1 are in flight while step k
// is computed.  The e8m0 scales are read straight from the pre-laid-out
// scale section (one dword per lane per 4 steps).  The per-token activation
// scale multiplies the accumulator in the epilogue, then bf16 RNE and store.
// The first MFMA operand is the weight (rows = n), the second the activation
// (rows = m), so each lane stores four consecutive n of one m (8 bytes).
#include "common.h"

namespace {

constexpr int kApitch = 144;  // bytes per staged activation row (128 + 16 pad)

template <int BM, int BN, int WM, int WN>
struct PrefillCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kTM = BM / WM / 32;  // 32-row sub-tiles per wave along m
  static constexpr int kTN = BN / WN / 32;  // along n
  static constexpr int kAChunks = BM * 8;   // 16-byte chunks of one activation tile
  static constexpr int kBChunks = BN * 4;   // of one weight tile (BN/16 x 64 lanes)
  static constexpr int kAPer = kAChunks / kThreads;
  static constexpr int kBPer = kBChunks / kThreads;
  static constexpr int kAStage = BM * kApitch;
  static constexpr int kBStage = BN * 64;
  static_assert(kAChunks % kThreads == 0 && kBChunks % kThreads == 0, "tile / thread mismatch");
  static_assert(kTM >= 1 && kTN >= 1, "wave tile too small");
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void k_w4a8_prefill(
    const uint8_t* __restrict__ a, int64_t lda, const float* __restrict__ as, const uint8_t* __restrict__ w,
    const uint32_t* __restrict__ wsc, uint16_t* __restrict__ c, int64_t ldc, int M, int N, int KS, int group_m) {
  using C = PrefillCfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][C::kAStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][C::kBStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, l = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int NT = N >> 4;
  const int KQ = (KS + 3) >> 2;

  // grouped raster: group_m m-tiles share one sweep over the n-tiles
  const int n_tiles = (N + BN - 1) / BN;
  const int m_tiles = (M + BM - 1) / BM;
  const int bid = blockIdx.x;
  const int per_group = group_m * n_tiles;
  const int grp = bid / per_group;
  const int first_m = grp * group_m;
  const int gsize = min(m_tiles - first_m, group_m);
  const int mt = first_m + (bid % per_group) % gsize;
  const int ntile = (bid % per_group) / gsize;
  const int m0 = mt * BM, n0 = ntile * BN;
  const int nt0 = n0 >> 4;

  // ---- global -> register prefetch of one K step
  uint4 ra[C::kAPer], rb[C::kBPer];
  auto gload = [&](int ks) {
#pragma unroll
    for (int i = 0; i < C::kAPer; ++i) {
      const int ch = i * C::kThreads + tid;
      const int row = ch >> 3, col = ch & 7;
      const int m = m0 + row;
      ra[i] = m < M ? *reinterpret_cast<const uint4*>(a + m * lda + ks * 128 + col * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kBPer; ++i) {
      const int ch = i * C::kThreads + tid;
      const int ntl = ch >> 6, ln = ch & 63;
      const int nt = nt0 + ntl;
      rb[i] = nt < NT ? *reinterpret_cast<const uint4*>(w + (static_cast<size_t>(nt) * KS + ks) * 1024 + ln * 16)
                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kAPer; ++i) {
      const int ch = i * C::kThreads + tid;
      *reinterpret_cast<uint4*>(&lds_a[buf][(ch >> 3) * kApitch + (ch & 7) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::kBPer; ++i) {
      const int ch = i * C::kThreads + tid;
      *reinterpret_cast<uint4*>(&lds_b[buf][ch * 16]) = rb[i];
    }
  };
  // ---- per-lane e8m0 scale dwords for one K step: [p][hh]
  uint32_t sd[C::kTN][2];
  auto sload = [&](int ks) {
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      const int n = n0 + wn * (BN / WN) + 32 * p + (l & 31);
      const int nt = n >> 4;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int lanep = (n & 15) + 16 * (2 * hh + (l >> 5));
        sd[p][hh] = nt < NT ? wsc[(static_cast<size_t>(nt) * KQ + (ks >> 2)) * 64 + lanep] : 0x7F7F7F7Fu;
      }
    }
  };

  v16f acc[C::kTN][C::kTM];
#pragma unroll
  for (int p = 0; p < C::kTN; ++p)
#pragma unroll
    for (int q = 0; q < C::kTM; ++q) acc[p][q] = v16f{};

  gload(0);
  sstore(0);
  sload(0);
  __syncthreads();

  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < KS;
    if (more) gload(ks + 1);
    uint32_t scur[C::kTN][2];
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
      scur[p][0] = sd[p][0] >> (8 * (ks & 3));
      scur[p][1] = sd[p][1] >> (8 * (ks & 3));
    }
    if (more && ((ks + 1) & 3) == 0) sload(ks + 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      v8i bf[C::kTN], af[C::kTM];
#pragma unroll
      for (int p = 0; p < C::kTN; ++p) {
        const int nl = wn * (BN / WN) + 32 * p + (l & 31);
        const int lanep = (nl & 15) + 16 * (2 * hh + (l >> 5));
        const uint4 x = *reinterpret_cast<const uint4*>(&lds_b[buf][(nl >> 4) * 1024 + lanep * 16]);
        bf[p] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int q = 0; q < C::kTM; ++q) {
        const int ml = wm * (BM / WM) + 32 * q + (l & 31);
        const uint8_t* row = &lds_a[buf][ml * kApitch + 64 * hh + 16 * (l >> 5)];
        const uint4 x = *reinterpret_cast<const uint4*>(row);
        const uint4 y = *reinterpret_cast<const uint4*>(row + 32);
        af[q] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
      }
#pragma unroll
      for (int p = 0; p < C::kTN; ++p)
#pragma unroll
        for (int q = 0; q < C::kTM; ++q)
          acc[p][q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[p], af[q], acc[p][q], 4, 0, 0,
                                                                      static_cast<int>(scur[p][hh]), 0, 127);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: x per-token scale, bf16 RNE, 8-byte stores
#pragma unroll
  for (int q = 0; q < C::kTM; ++q) {
    const int m = m0 + wm * (BM / WM) + 32 * q + (l & 31);
    if (m >= M) continue;
    const float s = as[m];
#pragma unroll
    for (int p = 0; p < C::kTN; ++p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * (BN / WN) + 32 * p + 8 * i + 4 * (l >> 5);
        if (n < N) {
          const uint32_t b0 = f32_to_bf16_rne(acc[p][q][4 * i + 0] * s);
          const uint32_t b1 = f32_to_bf16_rne(acc[p][q][4 * i + 1] * s);
          const uint32_t b2 = f32_to_bf16_rne(acc[p][q][4 * i + 2] * s);
          const uint32_t b3 = f32_to_bf16_rne(acc[p][q][4 * i + 3] * s);
          *reinterpret_cast<uint2*>(c + m * ldc + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        }
      }
    }
  }
}

}  // namespace

int bs_launch_w4a8_prefill(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                           uint16_t* c, int64_t ldc, int M, int N, int K, hipStream_t st) {
  const int KS = K / 128;
  constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
  const int n_tiles = (N + BN - 1) / BN, m_tiles = (M + BM - 1) / BM;
  const int group_m = 8;
  k_w4a8_prefill<BM, BN, WM, WN><<<n_tiles * m_tiles, 64 * WM * WN, 0, st>>>(a, lda, as, w, wsc, c, ldc, M, N, KS,
                                                                            group_m);
  return bs_launch_status();
}
