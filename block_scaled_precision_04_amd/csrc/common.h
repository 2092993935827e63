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

constexpr float kFp8Max = 448.0f;
constexpr double kMinScale = 1.0 / (448.0 * 512.0);
