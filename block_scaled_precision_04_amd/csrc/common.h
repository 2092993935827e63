// Internal helpers shared by the HIP sources of libbsgemm (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "bsgemm.h"

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define BS_INLINE __device__ __forceinline__

// Host-side argument checks: return the status from the enclosing function.
#define BS_CHECK(cond, status) \
  do {                         \
    if (!(cond)) return (status); \
  } while (0)

static inline bool bs_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static inline int bs_launch_status() {
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

// ------------------------------------------------------------ device helpers
// fp32 -> bf16 bit pattern, round to nearest even (inputs are finite here).
BS_INLINE uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two fp32 values -> two bf16 bit patterns packed low/high, with gfx950's
// packed convert (v_cvt_pk_bf16_f32: round to nearest even under the default
// rounding mode; the kernels keep fp32 denormals, so it equals
// f32_to_bf16_rne on every finite input -- one instruction instead of about
// five per value).
typedef __bf16 bs_bf16x2 __attribute__((ext_vector_type(2)));
BS_INLINE uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bs_bf16x2{static_cast<__bf16>(lo), static_cast<__bf16>(hi)});
}
BS_INLINE float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
BS_INLINE float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values -> two e4m3 codes in the low 16 bits (hardware convert:
// round to nearest even, exact for |x| <= 448; callers clamp first).
BS_INLINE uint32_t f32x2_to_e4m3(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

template <typename T>
BS_INLINE T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
BS_INLINE double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Streaming (non-temporal) 16-byte loads and 8/16-byte stores, for data that
// one kernel touches once: the accesses carry the non-temporal hint, so they
// do not displace cache lines that other workgroups still reuse.  Whether it
// pays is measured per kernel: it lifts the SiLU producer's sustained HBM
// rate by about a seventh and the decode weight stream by 3-8%.
typedef unsigned int bs_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bs_u32x2 __attribute__((ext_vector_type(2)));
BS_INLINE uint4 ld_stream16(const uint4* p) {
  const bs_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const bs_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
BS_INLINE void st_stream8(uint2* p, uint32_t lo, uint32_t hi) {
  bs_u32x2 v;
  v.x = lo;
  v.y = hi;
  __builtin_nontemporal_store(v, reinterpret_cast<bs_u32x2*>(p));
}
BS_INLINE void st_stream16(uint4* p, uint4 w) {
  bs_u32x4 v;
  v.x = w.x;
  v.y = w.y;
  v.z = w.z;
  v.w = w.w;
  __builtin_nontemporal_store(v, reinterpret_cast<bs_u32x4*>(p));
}

// Direct-to-LDS 16-byte load: lane i's 16 bytes from sbase + voff land at LDS
// byte address lds_addr + 16*i.  Issued from inline assembly so that the
// compiler does not serialise it against the LDS reads of other stages; the
// kernel waits for these loads itself (vmcnt) before the barrier that
// publishes a stage.
BS_INLINE void dma16(uint32_t lds_addr, const void* sbase, uint32_t voff) {
  // one wait state between the M0 write and the LDS-DMA that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// The 4-byte form: lane i's dword from sbase + voff lands at lds_addr + 4*i.
BS_INLINE void dma4(uint32_t lds_addr, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_addr), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}

// An empty statement that takes x in VGPRs: x stays live, in the registers it
// already has, up to this point of the program.
BS_INLINE void keep_vgprs(v4i x) { asm volatile("" ::"v"(x)); }
BS_INLINE void keep_vgprs(v8i x) { asm volatile("" ::"v"(x)); }
BS_INLINE void keep_vgprs(uint32_t x) { asm volatile("" ::"v"(x)); }

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory loads outstanding
template <int N>
BS_INLINE void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Output-tile order of the LDS-tiled GEMMs.  gfx950 hands workgroup b to XCD
// b % 8, and each XCD has its own L2: the tile sequence is cut into eight
// contiguous chunks, one per XCD, and inside a chunk the tiles follow a
// grouped raster (group_m m-tiles sweep the n-tiles together), so the
// workgroups resident on one XCD at any moment share a few activation and
// weight tiles in that XCD's L2.  One workgroup per tile: b < m_tiles*n_tiles.
constexpr int kXcds = 8;
BS_INLINE void xcd_tile(int b, int m_tiles, int n_tiles, int group_m, int& mt, int& nt) {
  const int T = m_tiles * n_tiles;
  const int x = b % kXcds, jj = b / kXcds;
  const int t = x * (T / kXcds) + min(x, T % kXcds) + jj;
  const int per_group = group_m * n_tiles;
  const int grp = t / per_group;
  const int first_m = grp * group_m;
  const int gsize = min(m_tiles - first_m, group_m);
  const int loc = t - grp * per_group;
  mt = first_m + loc % gsize;
  nt = loc / gsize;
}

// Split-K workspaces (every GEMM that splits K across workgroups): the first
// kWsCounterBytes hold the int32 tile counters, the fp32 slab of partials
// starts right after them.  Counters are zero between launches (the last
// workgroup of a tile resets its own), and no launch writes partials into the
// counter region, so any sequence of calls -- of any shapes -- can share one
// workspace that is large enough for each of them.
constexpr size_t kWsCounterBytes = 64 * 1024;
constexpr int kWsMaxCounters = static_cast<int>(kWsCounterBytes / sizeof(int));

// Split-K reduction of the last-arriving workgroup: sum[v] = the S fp32
// partials base[b * stride + v * VSTRIDE] added in split order b = 0, 1, ...
// (deterministic).  The partials were written with device-scope stores, so
// they are read with device-scope loads, which are served past the XCD's L2:
// a round trip costs about a microsecond.  The loads of U splits are all
// issued before any of them is added, so the reduction waits ceil(S / U)
// round trips rather than one per split and value group.  Splits past S
// re-read split S - 1 (valid memory) and are not added.
template <int NV, int VSTRIDE, int U>
BS_INLINE void sum_partials(float (&sum)[NV], const float* base, size_t stride, int S) {
#pragma unroll
  for (int v = 0; v < NV; ++v) sum[v] = 0.0f;
  for (int b0 = 0; b0 < S; b0 += U) {
    float x[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* src = base + static_cast<size_t>(min(b0 + u, S - 1)) * stride;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        x[u][v] = __hip_atomic_load(src + v * VSTRIDE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = b0 + u < S;
#pragma unroll
      for (int v = 0; v < NV; ++v) sum[v] = live ? sum[v] + x[u][v] : sum[v];
    }
  }
}

constexpr float kFp8Max = 448.0f;
constexpr double kMinScale = 1.0 / (448.0 * 512.0);
