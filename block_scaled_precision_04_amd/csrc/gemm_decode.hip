// Small-M (decode) block-scaled GEMMs: a weight stream through MFMA.
//
// Block-FP8 W8A8 (radiance_kernels.py page, block_scaled_mm: e4m3 weights with
// one scale per 128x128 block, e4m3 activations with one scale per token per
// 128-wide K group) and MXFP4 W4A8 at small M (radiance_mxfp4.py page: the
// decode band, the fragment-order weight that makes a wave's weight read
// contiguous, and split-K for shapes with too little N to fill the GPU).
//
// At M <= 64 the weight bytes dominate: the arithmetic intensity is far below
// the MFMA ridge, so the kernel is built to keep HBM busy:
//   * the weight was pre-laid-out in fragment order, so one (16-row tile,
//     128-K step) is one contiguous 2 KiB (fp8) / 1 KiB (fp4) block and each
//     lane issues 16-byte loads;
//   * a workgroup owns one 16-column tile of the output and splits K across
//     its SK waves; each wave first issues the loads of S steps at once, then
//     consumes them, so many KiB per CU are in flight;
//   * partial sums are reduced across the waves through LDS in a fixed order
//     (deterministic), then rounded once to bf16.
// The MFMA puts the weight tile in the first operand (rows = n) and the
// activations in the second (rows = m), so D[n][m] and each lane holds four
// consecutive n of one m.
//
// Block-FP8: every 16x16x128 MFMA covers exactly one 128-wide scale group, so
// its result (fresh accumulator) is scaled by a_scale[m,g] * w_scale[n/128,g]
// and added into an fp32 accumulator.  MXFP4: the scaled MFMA applies the e8m0
// weight scales in hardware (activation scale byte 127 = 1.0) and accumulates;
// the per-token activation scale multiplies the sum at the end.
#include "common.h"

namespace {

// ---- fragment loads --------------------------------------------------------
// fp8 x fp8 MFMA: both operands hold, in lane l, 32 bytes for K offsets
// 32*(l/16) .. +32 of a 128-K step (the same order on both sides, so the
// pairing is exact).
BS_INLINE v8i load_a_fp8_contig(const uint8_t* a, int64_t lda, int m, int M, int k) {
  if (m >= M) return v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const uint4* p = reinterpret_cast<const uint4*>(a + m * lda + k);
  uint4 x = p[0], y = p[1];
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}
// fp8 operand paired with an fp4 operand: the 8-bit operand's bytes 0..15 of
// lane group g are K offsets 16g.., bytes 16..31 are 64+16g.. (gfx950), while
// the 4-bit operand holds 32g..32g+31; so the activation loads follow the
// hardware's 8-bit order and real K lines up with the weight.
BS_INLINE v8i load_a_fp8_split(const uint8_t* a, int64_t lda, int m, int M, int k0, int g) {
  if (m >= M) return v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const uint8_t* row = a + m * lda + k0;
  uint4 x = *reinterpret_cast<const uint4*>(row + 16 * g);
  uint4 y = *reinterpret_cast<const uint4*>(row + 64 + 16 * g);
  return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

BS_INLINE v4f mfma_fp8(v8i w, v8i a, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 0, 0, 0, 127, 0, 127);
}
BS_INLINE v4f mfma_fp4w_fp8a(v8i w, v8i a, v4f c, int wscale) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 4, 0, 0, wscale, 0, 127);
}

// ---- cross-wave reduction and store -----------------------------------------
// red: [SK][MB*4][64] floats.  Every thread of the workgroup sums some outputs
// over the waves in wave order, then stores bf16.
template <int MB>
BS_INLINE void reduce_store(const v4f (&acc)[MB], float* red, int nwaves, uint16_t* c, int64_t ldc, int M,
                            int n0, int m0, const float* a_scale_tok) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * MB * 4 + mb * 4 + r) * 64 + l] = acc[mb][r];
  __syncthreads();
  for (int o = threadIdx.x; o < MB * 4 * 64; o += blockDim.x) {
    float s = 0.0f;
    for (int w = 0; w < nwaves; ++w) s += red[w * MB * 4 * 64 + o];
    const int lane = o & 63, r = (o >> 6) & 3, mb = o >> 8;
    const int m = m0 + 16 * mb + (lane & 15);
    const int n = n0 + 4 * (lane >> 4) + r;
    if (m < M) {
      if (a_scale_tok) s *= a_scale_tok[m];
      c[m * ldc + n] = static_cast<uint16_t>(f32_to_bf16_rne(s));
    }
  }
}

// ---- block-FP8 --------------------------------------------------------------
// grid (N/16, ceil(M/(16*MB))), block 64*SK threads.  Wave w handles the K
// steps [w*per, min((w+1)*per, KS)) in chunks of S.
template <int MB, int S>
__global__ __launch_bounds__(512) void k_fp8_block_decode(
    const uint8_t* __restrict__ a, int64_t lda, const float* __restrict__ as, int64_t asm_, int64_t asg,
    const uint8_t* __restrict__ w, const float* __restrict__ ws, uint16_t* __restrict__ c, int64_t ldc, int M,
    int KS, int per) {
  extern __shared__ float red[];
  const int nt = blockIdx.x;
  const int m0 = blockIdx.y * 16 * MB;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int g = l >> 4;
  const uint8_t* wt = w + static_cast<size_t>(nt) * KS * 2048 + l * 16;
  const float* wsc = ws + static_cast<size_t>(nt >> 3) * KS;  // 8 16-row tiles per 128-row block
  v4f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4f{0, 0, 0, 0};
  const int kbeg = wave * per;
  const int kend = min(kbeg + per, KS);
  for (int base = kbeg; base < kend; base += S) {
    v8i wf[S];
    v8i af[S][MB];
    float sa[S][MB];
    float sw[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int ks = base + s;
      if (ks < kend) {
        const uint4 x = *reinterpret_cast<const uint4*>(wt + static_cast<size_t>(ks) * 2048);
        const uint4 y = *reinterpret_cast<const uint4*>(wt + static_cast<size_t>(ks) * 2048 + 1024);
        wf[s] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        sw[s] = wsc[ks];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = m0 + 16 * mb + (l & 15);
          af[s][mb] = load_a_fp8_contig(a, lda, m, M, ks * 128 + 32 * g);
          sa[s][mb] = m < M ? as[m * asm_ + ks * asg] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (base + s < kend) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const v4f t = mfma_fp8(wf[s], af[s][mb], v4f{0, 0, 0, 0});
          const float f = sa[s][mb] * sw[s];
          acc[mb] += t * f;
        }
      }
    }
  }
  reduce_store<MB>(acc, red, nwaves, c, ldc, M, nt * 16, m0, nullptr);
}

// ---- MXFP4 W4A8 -------------------------------------------------------------
// Same decomposition; K steps are handed out in groups of four so that a
// wave's scale dword (four steps) is loaded once.  S is a multiple of 4.
template <int MB, int S>
__global__ __launch_bounds__(512) void k_w4a8_decode(const uint8_t* __restrict__ a, int64_t lda,
                                                      const float* __restrict__ as, const uint8_t* __restrict__ w,
                                                      const uint32_t* __restrict__ wsc, uint16_t* __restrict__ c,
                                                      int64_t ldc, int M, int KS, int per) {
  extern __shared__ float red[];
  const int nt = blockIdx.x;
  const int m0 = blockIdx.y * 16 * MB;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int g = l >> 4;
  const int KQ = (KS + 3) >> 2;
  const uint8_t* wt = w + static_cast<size_t>(nt) * KS * 1024 + l * 16;
  const uint32_t* st = wsc + static_cast<size_t>(nt) * KQ * 64 + l;
  v4f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4f{0, 0, 0, 0};
  const int kbeg = wave * per;  // per is a multiple of 4
  const int kend = min(kbeg + per, KS);
  for (int base = kbeg; base < kend; base += S) {
    v8i wf[S];
    v8i af[S][MB];
    uint32_t sd[S / 4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int ks = base + s;
      if (ks < kend) {
        const uint4 x = *reinterpret_cast<const uint4*>(wt + static_cast<size_t>(ks) * 1024);
        wf[s] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        if ((s & 3) == 0) sd[s >> 2] = st[static_cast<size_t>(ks >> 2) * 64];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[s][mb] = load_a_fp8_split(a, lda, m0 + 16 * mb + (l & 15), M, ks * 128, g);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (base + s < kend) {
        const int sc = static_cast<int>(sd[s >> 2] >> (8 * (s & 3)));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_fp4w_fp8a(wf[s], af[s][mb], acc[mb], sc);
      }
    }
  }
  reduce_store<MB>(acc, red, nwaves, c, ldc, M, nt * 16, m0, as);
}

constexpr int kMaxWaves = 8;  // 512 threads: leaves 256 VGPRs per lane

struct DecodeCfg {
  int mb, s, sk, per;
};

// Choose the m-tiles per workgroup, the steps per load batch and the number of
// waves per workgroup (K split) for a small-M shape.
DecodeCfg decode_cfg(int M, int KS, bool mx) {
  DecodeCfg d{};
  d.mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  d.s = d.mb == 1 ? 8 : 4;
  int sk = (KS + d.s - 1) / d.s;
  if (sk > kMaxWaves) sk = kMaxWaves;
  if (sk < 1) sk = 1;
  int per = (KS + sk - 1) / sk;
  if (mx) per = (per + 3) / 4 * 4;
  sk = (KS + per - 1) / per;
  d.sk = sk;
  d.per = per;
  return d;
}

}  // namespace

// Internal entry points used by the ABI layer (gemm_abi.cpp).
int bs_launch_fp8_block_decode(const uint8_t* a, int64_t lda, const float* as, int64_t asm_, int64_t asg,
                               const uint8_t* w, const float* ws, uint16_t* c, int64_t ldc, int M, int N, int K,
                               hipStream_t st) {
  const int KS = K / 128;
  const DecodeCfg d = decode_cfg(M, KS, false);
  dim3 grid(N / 16, (M + 16 * d.mb - 1) / (16 * d.mb));
  dim3 block(64 * d.sk);
  const size_t lds = static_cast<size_t>(d.sk) * d.mb * 4 * 64 * sizeof(float);
#define BS_FP8D(MB_, S_) \
  k_fp8_block_decode<MB_, S_><<<grid, block, lds, st>>>(a, lda, as, asm_, asg, w, ws, c, ldc, M, KS, d.per)
  if (d.mb == 1) BS_FP8D(1, 8);
  else if (d.mb == 2) BS_FP8D(2, 4);
  else BS_FP8D(4, 4);
#undef BS_FP8D
  return bs_launch_status();
}

int bs_launch_w4a8_decode(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                          uint16_t* c, int64_t ldc, int M, int N, int K, hipStream_t st) {
  const int KS = K / 128;
  const DecodeCfg d = decode_cfg(M, KS, true);
  dim3 grid(N / 16, (M + 16 * d.mb - 1) / (16 * d.mb));
  dim3 block(64 * d.sk);
  const size_t lds = static_cast<size_t>(d.sk) * d.mb * 4 * 64 * sizeof(float);
#define BS_W4D(MB_, S_) k_w4a8_decode<MB_, S_><<<grid, block, lds, st>>>(a, lda, as, w, wsc, c, ldc, M, KS, d.per)
  if (d.mb == 1) BS_W4D(1, 8);
  else if (d.mb == 2) BS_W4D(2, 4);
  else BS_W4D(4, 4);
#undef BS_W4D
  return bs_launch_status();
}
