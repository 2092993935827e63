// Producers of e4m3 activations / weights for the block-scaled GEMMs.
//
// add_rms_quant_fp8: residual add -> Gemma RMSNorm -> per-token e4m3 quant in
// one pass over HBM (radiance_arnq.py page: ar_add_rms_quant and the fp8
// residual-stream contract; the quant rule is the radiance_mxfp4.py page's
// _traced_quant: scale = max(rowamax/448, 1/(448*512)), fp32 math, clamp,
// round-to-nearest cast).
//
// One workgroup of T threads per row (256, or 128 for many short rows).
// Each thread owns NC chunks of 8 bf16
// (16-byte loads), keeps them in registers between the two row reductions
// (sum of squares, then absolute maximum) and writes the e4m3 codes, so every
// byte is read once and written once: 7 bytes per element plus 2 per column
// of gamma (shared by all rows, cache-resident).  The stores carry the
// streaming hint; the loads do not (measured: the hint on the loads costs
// about 4% here, on the stores it saves about 7%).
//
// Precision: r = bf16(y + residual) is exact (an fp32 add of two bf16 values
// is exact or below half a bf16 ulp, so one more rounding to bf16 equals a
// single rounding of the exact sum).  The sum of r^2 and the normalisation
// are carried in fp64 and h is rounded once to fp32, so h, the row maximum
// and the scale agree with a correctly rounded evaluation; the code decision
// h/scale is an IEEE fp32 division followed by the hardware's round-to-
// nearest-even e4m3 convert, as the page's traced quant takes it in fp32.
#include "common.h"

namespace {

constexpr int kThreads = 256;

// Workgroup reductions over W waves (wave partials through LDS, added in wave
// order).  Each LDS array serves one reduction per kernel, so no barrier
// follows the reads.
template <int W = kThreads / 64>
BS_INLINE float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < W; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int W = kThreads / 64>
BS_INLINE double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  double r;
  if constexpr (W == 4) {
    r = (red[0] + red[1]) + (red[2] + red[3]);
  } else {
    r = red[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r += red[i];
  }
  return r;
}

BS_INLINE uint2 quant8(const float* h, float s) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    float a = fminf(fmaxf(h[j] / s, -kFp8Max), kFp8Max);
    float b = fminf(fmaxf(h[j + 1] / s, -kFp8Max), kFp8Max);
    lo |= f32x2_to_e4m3(a, b) << (8 * j);
  }
#pragma unroll
  for (int j = 4; j < 8; j += 2) {
    float a = fminf(fmaxf(h[j] / s, -kFp8Max), kFp8Max);
    float b = fminf(fmaxf(h[j + 1] / s, -kFp8Max), kFp8Max);
    hi |= f32x2_to_e4m3(a, b) << (8 * (j - 4));
  }
  return make_uint2(lo, hi);
}

// Activation-tiled order (the radiance_mxfp4.py page's fragment-tiled
// producer output, A_TILED_MIN_M comment, laid out for gfx950): the operand
// order of the 32x32x64 MFMA with an 8-bit operand, rows in blocks of 32.
// A (32-row block, 128-K step) is 4 KiB, two 2 KiB halves of 64 K; in a half,
// lane l holds row l % 32 and 32 bytes: K = 16*(l/32) .. +15, then
// 32 + 16*(l/32) .. +15.  Byte offset of codes (m, k .. k+7), k % 8 == 0:
BS_INLINE size_t tiled_offset(int m, int k, int KS) {
  const int kp = k & 63;
  const int lane = (m & 31) + 32 * ((kp >> 4) & 1);
  return ((static_cast<size_t>(m >> 5) * KS + (k >> 7)) * 2 + ((k >> 6) & 1)) * 2048 + lane * 32 + (kp >> 5) * 16 +
         (kp & 15);
}

BS_INLINE void unpack8(uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// NORM = true: add + RMSNorm + quant.  NORM = false: per-token quant of y.
// GROUP = true: one scale per 128-wide group of the row instead of one per
// row; chunk idx = c*256 + t belongs to group idx/16, so the 16 consecutive
// threads holding a group reduce its maximum with four shuffles.
// TILED = true: the codes go out in the activation-tiled order (below)
// instead of row-major [M, K].
// res and rout may be the same buffer (the residual updated in place), so
// neither is declared __restrict__; every thread reads its chunks of a row
// before it writes them.
template <int NC, bool NORM, bool GROUP = false, int T = kThreads, bool TILED = false>
__global__ __launch_bounds__(T) void k_row_quant(const uint4* __restrict__ y,
                                                 const uint4* res,
                                                 const uint4* __restrict__ gamma, float eps,
                                                 uint2* __restrict__ q, float* __restrict__ scale,
                                                 uint4* rout, int K) {
  static_assert(T % 64 == 0, "whole waves");
  constexpr int kThreads = T;  // threads per row (shadows the file-wide default)
  __shared__ double red_d[T / 64];
  __shared__ float red_f[T / 64];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int nch = K >> 3;
  const size_t base = static_cast<size_t>(row) * nch;
  // Every load of the row -- y, the residual and gamma -- is issued before
  // any arithmetic (clamped chunk index, masked afterwards), so the row costs
  // one memory round trip before the reductions.
  uint4 yv[NC], rv[NC], gv[NC];
  bool live[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = c * kThreads + t;
    live[c] = idx < nch;
    const int ci = min(idx, nch - 1);
    yv[c] = y[base + ci];
    if constexpr (NORM) {
      rv[c] = res[base + ci];
      gv[c] = gamma[ci];
    }
  }
  float h[NC][8];
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float a[8];
    unpack8(yv[c], a);
    if constexpr (NORM) {
      float b[8];
      unpack8(rv[c], b);
      uint32_t rb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rb[j] = f32_to_bf16_rne(a[j] + b[j]);
        h[c][j] = live[c] ? __uint_as_float(rb[j] << 16) : 0.0f;
        ss += static_cast<double>(h[c][j]) * static_cast<double>(h[c][j]);
      }
      if (live[c])
        st_stream16(rout + base + c * kThreads + t, make_uint4(rb[0] | (rb[1] << 16), rb[2] | (rb[3] << 16),
                                                               rb[4] | (rb[5] << 16), rb[6] | (rb[7] << 16)));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[c][j] = live[c] ? a[j] : 0.0f;
    }
  }
  if constexpr (NORM) {
    const double tot = block_sum_f64<T / 64>(ss, red_d);
    const double inv = 1.0 / sqrt(tot / static_cast<double>(K) + static_cast<double>(eps));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float g[8];
      unpack8(gv[c], g);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        h[c][j] = static_cast<float>(static_cast<double>(h[c][j]) * inv * (1.0 + static_cast<double>(g[j])));
    }
  }
  if constexpr (GROUP) {
    const int ngroups = nch >> 4;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[c][j]));
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
      const int idx = c * kThreads + t;
      if (idx < nch) {   // K % 128 == 0: a group's 16 threads are all live or all idle
        if ((t & 15) == 0) scale[static_cast<size_t>(row) * ngroups + (idx >> 4)] = s;
        const uint2 v = quant8(h[c], s);
        st_stream8(q + base + idx, v.x, v.y);
      }
    }
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[c][j]));
    amax = block_max<T / 64>(amax, red_f);
    const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
    if (t == 0) scale[row] = s;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = c * kThreads + t;
      if (idx < nch) {
        const uint2 v = quant8(h[c], s);
        if constexpr (TILED)
          st_stream8(reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(q) + tiled_offset(row, idx * 8, K >> 7)),
                     v.x, v.y);
        else
          st_stream8(q + base + idx, v.x, v.y);
      }
    }
  }
}

// The norm producer writing the activation-tiled order: four consecutive
// rows per workgroup (T threads each, as k_row_quant), their codes gathered
// in LDS, then written as whole 128-byte lines.  In the tiled order a row
// owns 32-byte lane slots, never a whole line: four consecutive rows (4r ..
// 4r+3, lanes 4r%32 .. +3 of one half step) fill one line, so a workgroup
// holding them stores full lines instead of scattering 16-byte pieces
// (measured: one row per workgroup took 43 us at M = 4096, K = 5120, against
// 33 us for the row-major codes).  Per row the arithmetic is k_row_quant's
// with NORM: residual add, fp64 sum of squares, h rounded once to fp32,
// per-token scale, IEEE h / scale and the e4m3 convert.
template <int NC, int T>
__global__ __launch_bounds__(4 * T) void k_row_quant_tiled(const uint4* __restrict__ y, const uint4* res,
                                                           const uint4* __restrict__ gamma, float eps,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale,
                                                           uint4* rout, int M, int K) {
  static_assert(T % 64 == 0, "whole waves");
  constexpr int kW = T / 64;  // waves per row
  __shared__ double red_d[4][kW];
  __shared__ float red_f[4][kW];
  extern __shared__ __align__(16) uint8_t codes[];  // [4][K] e4m3, row-major
  const int rr = threadIdx.x / T;                    // row within the workgroup
  const int t = threadIdx.x % T;
  const int wv = t >> 6, l = t & 63;
  const int row0 = blockIdx.x * 4;
  const int row = min(row0 + rr, M - 1);            // rows past M redo row M-1 (never stored)
  const int nch = K >> 3;
  const size_t base = static_cast<size_t>(row) * nch;
  uint4 yv[NC], rv[NC], gv[NC];
  bool live[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = c * T + t;
    live[c] = idx < nch;
    const int ci = min(idx, nch - 1);
    yv[c] = y[base + ci];
    rv[c] = res[base + ci];
    gv[c] = gamma[ci];
  }
  float h[NC][8];
  double ss = 0.0;
  const bool own = row0 + rr < M;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float a[8], b[8];
    unpack8(yv[c], a);
    unpack8(rv[c], b);
    uint32_t rb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      rb[j] = f32_to_bf16_rne(a[j] + b[j]);
      h[c][j] = live[c] ? __uint_as_float(rb[j] << 16) : 0.0f;
      ss += static_cast<double>(h[c][j]) * static_cast<double>(h[c][j]);
    }
    if (live[c] && own)
      st_stream16(rout + base + c * T + t, make_uint4(rb[0] | (rb[1] << 16), rb[2] | (rb[3] << 16),
                                                      rb[4] | (rb[5] << 16), rb[6] | (rb[7] << 16)));
  }
  // per-row reductions: the row's kW waves through LDS slots of their own
  ss = wave_sum_f64(ss);
  if (l == 0) red_d[rr][wv] = ss;
  __syncthreads();
  double tot = red_d[rr][0];
#pragma unroll
  for (int i = 1; i < kW; ++i) tot += red_d[rr][i];
  const double inv = 1.0 / sqrt(tot / static_cast<double>(K) + static_cast<double>(eps));
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float g[8];
    unpack8(gv[c], g);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[c][j] = static_cast<float>(static_cast<double>(h[c][j]) * inv * (1.0 + static_cast<double>(g[j])));
      amax = fmaxf(amax, fabsf(h[c][j]));
    }
  }
  amax = wave_max(amax);
  if (l == 0) red_f[rr][wv] = amax;
  __syncthreads();
  amax = red_f[rr][0];
#pragma unroll
  for (int i = 1; i < kW; ++i) amax = fmaxf(amax, red_f[rr][i]);
  const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
  if (t == 0 && own) scale[row] = s;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = c * T + t;
    if (idx < nch) *reinterpret_cast<uint2*>(codes + rr * K + idx * 8) = quant8(h[c], s);
  }
  __syncthreads();
  // whole lines: line (ks, h, g) of this row quad is 4 rows x 32 bytes; its
  // 16-byte unit u holds row u/2, bytes 16c .. +15 (c = u%2) of the row's
  // lane slot = K offsets 128ks + 64h + 32c + 16g .. +15
  const int rows = min(4, M - row0);
  const int KS = K >> 7;
  const int lines = KS * 4;
  uint8_t* qb = q + ((static_cast<size_t>(row0 >> 5) * KS) * 2) * 2048 + (row0 & 31) * 32;
  for (int v = threadIdx.x; v < lines * 8; v += 4 * T) {
    const int line = v >> 3, u = v & 7;
    const int r = u >> 1, c = u & 1;
    const int ks = line >> 2, hh = (line >> 1) & 1, g = line & 1;
    if (r < rows) {
      const uint4 val = *reinterpret_cast<const uint4*>(codes + r * K + ks * 128 + hh * 64 + 32 * c + 16 * g);
      st_stream16(reinterpret_cast<uint4*>(qb + ((static_cast<size_t>(ks) * 2 + hh) * 2048) + g * 1024 + u * 16), val);
    }
  }
}

// One scale per 128-wide group of each row.  Block = 256 threads = 16 groups
// of 16 threads, each thread one 8-element chunk.  grid = (ceil(K/2048), M).
__global__ __launch_bounds__(kThreads) void k_group_quant(const uint4* __restrict__ x, uint2* __restrict__ q,
                                                          float* __restrict__ scale, int K) {
  const int row = blockIdx.y;
  const int nch = K >> 3;
  const int idx = blockIdx.x * kThreads + threadIdx.x;
  const bool live = idx < nch;  // K % 128 == 0: whole 16-thread groups are live or not
  float h[8];
  if (live) {
    unpack8(x[static_cast<size_t>(row) * nch + idx], h);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[j]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
  if (live) {
    if ((threadIdx.x & 15) == 0) scale[static_cast<size_t>(row) * (K >> 7) + (idx >> 4)] = s;
    q[static_cast<size_t>(row) * nch + idx] = quant8(h, s);
  }
}

// One scale per 128x128 block of a weight.  One workgroup per block; thread t
// handles row (t >> 1) of the block, chunks 8*(t&1) .. +8.
__global__ __launch_bounds__(kThreads) void k_block_quant(const uint4* __restrict__ w, uint2* __restrict__ q,
                                                          float* __restrict__ scale, int K) {
  __shared__ float red_f[4];
  const int bk = blockIdx.x, bn = blockIdx.y;
  const int nch = K >> 3;
  const int r = bn * 128 + (threadIdx.x >> 1);
  const int c0 = bk * 16 + (threadIdx.x & 1) * 8;
  float h[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    unpack8(w[static_cast<size_t>(r) * nch + c0 + c], h[c]);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[c][j]));
  }
  amax = block_max(amax, red_f);
  const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
  if (threadIdx.x == 0) scale[static_cast<size_t>(bn) * (K >> 7) + bk] = s;
#pragma unroll
  for (int c = 0; c < 8; ++c) q[static_cast<size_t>(r) * nch + c0 + c] = quant8(h[c], s);
}

// SiLU(gate) * up -> per-token e4m3 quant (radiance_arnq.py page, the
// silu_mul_quant op that stands in for the MLP's SiluAndMul ahead of the down
// projection).  gu is [M, 2N] bf16: columns 0..N-1 are the gate (the SiLU's
// input), N..2N-1 the up half.  One T-thread workgroup per row; each thread
// owns NC chunks of 8 columns, issues both halves' loads for all of them
// before any arithmetic, keeps h in registers through the row maximum and
// writes the codes: 4 bytes read and 1 written per output column, all with
// the streaming hint (nothing here is read twice).
//
// Arithmetic is budgeted for the HBM stream (at N = 17408, M = 4096 the IEEE
// exp and two IEEE divisions per element would outlast the 357 MB pass):
// sigmoid(g) = 1 / (1 + 2^(-g log2 e)) with the hardware exp2 and reciprocal,
// h = g * sigmoid(g) * up in fp32 (a few fp32 ulps from the correctly rounded
// value), and the codes take h * (1/scale) with the reciprocal correctly
// rounded once per row.  The scale itself is the exact quotient rule,
// max(amax/448, 1/(448*512)) with an IEEE fp32 division.
template <int NC, int T>
__global__ __launch_bounds__(T) void k_silu_quant(const uint4* __restrict__ gu, uint2* __restrict__ q,
                                                  float* __restrict__ scale, int N) {
  __shared__ float red[T / 64];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int nch = N >> 3;
  const uint4* g_row = gu + static_cast<size_t>(row) * (2 * nch);
  const uint4* u_row = g_row + nch;
  uint4 gv[NC], uv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ci = min(c * T + t, nch - 1);
    gv[c] = ld_stream16(g_row + ci);
    uv[c] = ld_stream16(u_row + ci);
  }
  constexpr float kLog2e = 1.4426950408889634f;
  float h[NC][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float g[8], u[8];
    unpack8(gv[c], g);
    unpack8(uv[c], u);
    const bool live = c * T + t < nch;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = __builtin_amdgcn_exp2f(-g[j] * kLog2e);
      const float v = g[j] * __builtin_amdgcn_rcpf(1.0f + e) * u[j];
      h[c][j] = live ? v : 0.0f;
      amax = fmaxf(amax, fabsf(h[c][j]));
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < T / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = fmaxf(amax / kFp8Max, static_cast<float>(kMinScale));
  const float inv = 1.0f / s;
  if (t == 0) scale[row] = s;
  uint2* q_row = q + static_cast<size_t>(row) * nch;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = c * T + t;
    if (idx < nch) {
      uint32_t w2[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float a = fminf(fmaxf(h[c][j] * inv, -kFp8Max), kFp8Max);
        const float b = fminf(fmaxf(h[c][j + 1] * inv, -kFp8Max), kFp8Max);
        w2[j >> 2] |= f32x2_to_e4m3(a, b) << (8 * (j & 3));
      }
      st_stream8(q_row + idx, w2[0], w2[1]);
    }
  }
}

int launch_silu_quant(const void* gu, void* q, float* scale, int M, int N, hipStream_t st) {
  // 768 threads (12 waves) per row: three 8-column chunks per thread cover
  // N = 17408 with 6% idle slots; measured best from 256 to 8192 rows.
  const int nc = (N / 8 + 767) / 768;
#define BS_SILU(N_)                                                                                        \
  k_silu_quant<N_, 768><<<dim3(M), dim3(768), 0, st>>>(static_cast<const uint4*>(gu), static_cast<uint2*>(q), \
                                                       scale, N)
  if (nc <= 1) BS_SILU(1);
  else if (nc <= 2) BS_SILU(2);
  else if (nc <= 3) BS_SILU(3);
  else if (nc <= 4) BS_SILU(4);
  else BS_SILU(6);
#undef BS_SILU
  return bs_launch_status();
}

// Threads per row: 256 in general; with many rows (M >= 2048) and K <= 5120,
// 128-thread rows of up to five chunks per thread, which keep more rows in
// flight per CU (M = 8192, K = 5120: 63 -> 56 us, graph-replayed over inputs
// pooled past the Infinity Cache).
template <bool NORM, bool GROUP = false, bool TILED = false>
int launch_row_quant(const void* y, const void* res, const void* gamma, float eps, void* q, float* scale,
                     void* rout, int M, int K, hipStream_t st) {
  if (M >= 2048 && K <= 5120) {
    const int nc = (K / 8 + 127) / 128;
#define BS_ROWQ128(N_)                                                                                  \
  k_row_quant<N_, NORM, GROUP, 128, TILED><<<dim3(M), dim3(128), 0, st>>>(                             \
      static_cast<const uint4*>(y), static_cast<const uint4*>(res), static_cast<const uint4*>(gamma), eps, \
      static_cast<uint2*>(q), scale, static_cast<uint4*>(rout), K)
    if (nc <= 1) BS_ROWQ128(1);
    else if (nc <= 2) BS_ROWQ128(2);
    else if (nc <= 3) BS_ROWQ128(3);
    else if (nc <= 4) BS_ROWQ128(4);
    else BS_ROWQ128(5);
#undef BS_ROWQ128
    return bs_launch_status();
  }
  if (GROUP && M < 256 && K / 8 > kThreads) {
    // group scales, fewer rows than CUs: 1024 threads per row, so each thread
    // carries at most a few chunks through the serial per-element arithmetic
    // (M = 8, K = 5120: 4.34 -> 4.18 us; the per-row-scale form, whose block
    // maximum then spans 16 waves, went from 4.24 to 4.75 us)
    const int nc = (K / 8 + 1023) / 1024;
#define BS_ROWQ1K(N_)                                                                                   \
  k_row_quant<N_, NORM, GROUP, 1024, TILED><<<dim3(M), dim3(1024), 0, st>>>(                           \
      static_cast<const uint4*>(y), static_cast<const uint4*>(res), static_cast<const uint4*>(gamma), eps, \
      static_cast<uint2*>(q), scale, static_cast<uint4*>(rout), K)
    if (nc <= 1) BS_ROWQ1K(1);
    else if (nc <= 2) BS_ROWQ1K(2);
    else BS_ROWQ1K(4);
#undef BS_ROWQ1K
    return bs_launch_status();
  }
  const int nc = (K / 8 + kThreads - 1) / kThreads;
  dim3 grid(M), block(kThreads);
#define BS_ROWQ(N_)                                                                                    \
  k_row_quant<N_, NORM, GROUP, kThreads, TILED><<<grid, block, 0, st>>>(                                \
      static_cast<const uint4*>(y), static_cast<const uint4*>(res), static_cast<const uint4*>(gamma), eps, \
      static_cast<uint2*>(q), scale, static_cast<uint4*>(rout), K)
  if (nc <= 1) BS_ROWQ(1);
  else if (nc <= 2) BS_ROWQ(2);
  else if (nc <= 3) BS_ROWQ(3);
  else if (nc <= 4) BS_ROWQ(4);
  else if (nc <= 6) BS_ROWQ(6);
  else if (nc <= 8) BS_ROWQ(8);
  else if (nc <= 12) BS_ROWQ(12);
  else BS_ROWQ(16);
#undef BS_ROWQ
  return bs_launch_status();
}

constexpr int kMaxRowK = 32768;  // 16 chunks of 8 per thread

}  // namespace

extern "C" {

BS_API int add_rms_quant_fp8(const void* y, const void* residual, const void* gamma, float eps, void* q,
                             float* scale, void* residual_out, int M, int K, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(y && residual && gamma && q && scale && residual_out, BS_ERR_NULL);
  BS_CHECK(M >= 1 && K >= 8 && K % 8 == 0 && K <= kMaxRowK, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(y, 16) && bs_aligned(residual, 16) && bs_aligned(gamma, 16) && bs_aligned(q, 8) &&
               bs_aligned(scale, 4) && bs_aligned(residual_out, 16),
           BS_ERR_ALIGN);
  BS_CHECK(eps >= 0.0f, BS_ERR_ARG);
  return launch_row_quant<true>(y, residual, gamma, eps, q, scale, residual_out, M, K,
                                static_cast<hipStream_t>(stream));
}

BS_API int add_rms_quant_fp8_tiled(const void* y, const void* residual, const void* gamma, float eps, void* q_tiled,
                                   float* scale, void* residual_out, int M, int K, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(y && residual && gamma && q_tiled && scale && residual_out, BS_ERR_NULL);
  BS_CHECK(M >= 1 && K >= 128 && K % 128 == 0 && K <= kMaxRowK, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(y, 16) && bs_aligned(residual, 16) && bs_aligned(gamma, 16) && bs_aligned(q_tiled, 16) &&
               bs_aligned(scale, 4) && bs_aligned(residual_out, 16),
           BS_ERR_ALIGN);
  BS_CHECK(eps >= 0.0f, BS_ERR_ARG);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t lds = static_cast<size_t>(4) * K;   // the row quad's codes
  const dim3 grid((M + 3) / 4);
#define BS_ROWQT(N_, T_)                                                                                     \
  do {                                                                                                       \
    auto* fn = &k_row_quant_tiled<N_, T_>;                                                                   \
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                    \
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 4 * 5120);       \
    if (attr != hipSuccess) return BS_ERR_LAUNCH;                                                            \
    fn<<<grid, dim3(4 * T_), lds, st>>>(static_cast<const uint4*>(y), static_cast<const uint4*>(residual),   \
                                        static_cast<const uint4*>(gamma), eps, static_cast<uint8_t*>(q_tiled), \
                                        scale, static_cast<uint4*>(residual_out), M, K);                     \
  } while (0)
  // row quads of 128-thread rows, up to five chunks per thread (K <= 5120:
  // 512 threads per workgroup, two waves per SIMD); longer rows would need
  // more registers than four rows per workgroup leave, and keep one row per
  // workgroup with scattered 8-byte stores
  const int nc128 = (K / 8 + 127) / 128;
  if (nc128 > 5)
    return launch_row_quant<true, false, true>(y, residual, gamma, eps, q_tiled, scale, residual_out, M, K, st);
  if (nc128 <= 1) BS_ROWQT(1, 128);
  else if (nc128 <= 2) BS_ROWQT(2, 128);
  else if (nc128 <= 3) BS_ROWQT(3, 128);
  else if (nc128 <= 4) BS_ROWQT(4, 128);
  else BS_ROWQT(5, 128);
#undef BS_ROWQT
  return bs_launch_status();
}

BS_API int add_rms_quant_fp8_group128(const void* y, const void* residual, const void* gamma, float eps, void* q,
                                      float* scale, void* residual_out, int M, int K, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(y && residual && gamma && q && scale && residual_out, BS_ERR_NULL);
  BS_CHECK(M >= 1 && K >= 128 && K % 128 == 0 && K <= kMaxRowK, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(y, 16) && bs_aligned(residual, 16) && bs_aligned(gamma, 16) && bs_aligned(q, 8) &&
               bs_aligned(scale, 4) && bs_aligned(residual_out, 16),
           BS_ERR_ALIGN);
  BS_CHECK(eps >= 0.0f, BS_ERR_ARG);
  return launch_row_quant<true, true>(y, residual, gamma, eps, q, scale, residual_out, M, K,
                                      static_cast<hipStream_t>(stream));
}

BS_API int silu_mul_quant_fp8(const void* gu, void* q, float* scale, int M, int N, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(gu && q && scale, BS_ERR_NULL);
  BS_CHECK(M >= 1 && N >= 8 && N % 8 == 0 && N <= kMaxRowK, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(gu, 16) && bs_aligned(q, 8) && bs_aligned(scale, 4), BS_ERR_ALIGN);
  return launch_silu_quant(gu, q, scale, M, N, static_cast<hipStream_t>(stream));
}

BS_API int quant_fp8_per_token(const void* x, void* q, float* scale, int M, int K, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(x && q && scale, BS_ERR_NULL);
  BS_CHECK(M >= 1 && K >= 8 && K % 8 == 0 && K <= kMaxRowK, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(x, 16) && bs_aligned(q, 8) && bs_aligned(scale, 4), BS_ERR_ALIGN);
  return launch_row_quant<false>(x, nullptr, nullptr, 0.0f, q, scale, nullptr, M, K,
                                 static_cast<hipStream_t>(stream));
}

BS_API int quant_fp8_group128(const void* x, void* q, float* scale, int M, int K, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(x && q && scale, BS_ERR_NULL);
  BS_CHECK(M >= 1 && M <= 65535 && K >= 128 && K % 128 == 0, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(x, 16) && bs_aligned(q, 8) && bs_aligned(scale, 4), BS_ERR_ALIGN);
  dim3 grid((K / 8 + kThreads - 1) / kThreads, M);
  k_group_quant<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(x), static_cast<uint2*>(q), scale, K);
  return bs_launch_status();
}

BS_API int quant_fp8_block128(const void* w, void* q, float* scale, int N, int K, bs_stream_t stream) {
  BS_CHECK(w && q && scale, BS_ERR_NULL);
  BS_CHECK(N >= 128 && N % 128 == 0 && N / 128 <= 65535 && K >= 128 && K % 128 == 0, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(w, 16) && bs_aligned(q, 8) && bs_aligned(scale, 4), BS_ERR_ALIGN);
  dim3 grid(K / 128, N / 128);
  k_block_quant<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(w), static_cast<uint2*>(q), scale, K);
  return bs_launch_status();
}

}  // extern "C"
