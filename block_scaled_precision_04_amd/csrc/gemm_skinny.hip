// Skinny bf16 NT GEMM C[M,N] = x[M,K] . W[N,K]^T for sub-megabyte weights at
// M <= 64 (radiance_gemm.py page: gemm_bf16_nt_m64).  The page's diagnosis:
// a weight under 1 MB gives a library GEMM only a handful of workgroups, each
// walking all of K, so the GPU idles; its fix is heavy split-K (the measured
// best MoE-gate config splits each column tile 16 ways) with a flat cost in M,
// and its fallback splits K across workgroups through an fp32 partial slab and
// per-tile counters.
//
// Here: grid = (N/16 column tiles, KSPLIT), four waves per workgroup, one
// 128-wide K chunk per wave.  Each lane loads 64 contiguous bytes of a weight
// row and of each activation row (four 16x16x32 bf16 MFMAs' worth; both
// operands use the same K order so the products pair exactly), the four waves
// reduce through LDS, and when K is split over several workgroups the partial
// tile goes to the workspace slab in MFMA fragment order (every store and load
// covers 256 contiguous bytes); the last workgroup to finish a tile (an atomic
// counter) sums the KSPLIT partials in index order (deterministic), writes
// bf16 and resets the counter to zero for the next call.  The hand-off uses
// device-scope stores and loads of the partials and no device-scope fence (a
// fence writes back and invalidates the L2 of the XCD on every workgroup).
// Rows past M load row M-1 (unconditional loads) and only ever reach output
// columns that are not stored.
#include <mutex>

#include "common.h"

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 128;  // K per wave

BS_INLINE v8bf as_bf(uint4 x) {
  v4i t{(int)x.x, (int)x.y, (int)x.z, (int)x.w};
  return __builtin_bit_cast(v8bf, t);
}
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
BS_INLINE v2bf as_bf2(uint32_t x) { return __builtin_bit_cast(v2bf, x); }

template <int MB>
__global__ __launch_bounds__(256) void k_skinny(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                uint16_t* __restrict__ c, int M, int N, int K,
                                                float* __restrict__ slab, int* __restrict__ counters) {
  __shared__ float red[kWaves][MB * 4][64];
  __shared__ int last;
  const int nt = blockIdx.x, kb = blockIdx.y, ksplit = gridDim.y;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int chunk = kb * kWaves + wave;
  v4f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4f{0, 0, 0, 0};
  if (chunk * kChunk < K) {
    // K % 32 == 0: a lane's 32 K values are wholly inside or past K.  A lane
    // past K (in a last, partial chunk) re-reads the row's last 32 values
    // and zeroes its weight, so it adds nothing.
    const int k0 = chunk * kChunk + 32 * (l >> 4);
    const bool k_in = k0 < K;
    const int kl = k_in ? k0 : K - 32;
    // (an and-mask rather than a select, which the compiler turns into a
    // conditional load and then cannot hoist the activation loads past)
    const uint32_t keep = k_in ? 0xFFFFFFFFu : 0u;
    const uint4* wr = reinterpret_cast<const uint4*>(w + static_cast<size_t>(nt * 16 + (l & 15)) * K + kl);
    uint4 wv[4], xv[MB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = wr[j];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = min(16 * mb + (l & 15), M - 1);
      const uint4* xr = reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + kl);
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[mb][j] = xr[j];
    }
    // every load of the chunk is issued before the first MFMA waits on one
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = make_uint4(wv[j].x & keep, wv[j].y & keep, wv[j].z & keep, wv[j].w & keep);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(wv[j]), as_bf(xv[mb][j]), acc[mb], 0, 0, 0);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][mb * 4 + r][l] = acc[mb][r];
  __syncthreads();
  // Thread o of the workgroup owns output o = (mb, r, lane): m = 16mb + lane%16, n = 4(lane/16) + r.
  const int ntiles = gridDim.x;
  for (int o = threadIdx.x; o < MB * 256; o += 256) {
    const int lane = o & 63, rr = (o >> 6) & 3, mb = o >> 8;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) s += red[v][mb * 4 + rr][lane];
    const int m = 16 * mb + (lane & 15), n = nt * 16 + 4 * (lane >> 4) + rr;
    if (ksplit == 1) {
      if (m < M) c[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(bf16x2_rne(s, 0.0f));
    } else {
      __hip_atomic_store(&slab[(static_cast<size_t>(kb) * ntiles + nt) * (MB * 256) + o], s, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (ksplit == 1) return;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partials are acknowledged
  asm volatile("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&counters[nt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ksplit - 1;
  __syncthreads();
  if (!last) return;
  // output o = threadIdx.x + 256 i of split b sits at slab[(b * ntiles + nt) * MB * 256 + o]
  float tot[MB];
  sum_partials<MB, 256, 8>(tot, slab + static_cast<size_t>(nt) * (MB * 256) + threadIdx.x,
                           static_cast<size_t>(ntiles) * (MB * 256), ksplit);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int o = threadIdx.x + 256 * i;
    const int lane = o & 63, rr = (o >> 6) & 3, mb = o >> 8;
    const int m = 16 * mb + (lane & 15), n = nt * 16 + 4 * (lane >> 4) + rr;
    if (m < M) c[static_cast<size_t>(m) * N + n] = static_cast<uint16_t>(bf16x2_rne(tot[i], 0.0f));
  }
  if (threadIdx.x == 0) __hip_atomic_store(&counters[nt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Up to 32 rows and K <= 2048: one output column and up to 8 rows per
// workgroup (grid (N, ceil(M/8))) over the whole of K, dot products on the
// VALU (v_dot2 over packed bf16 pairs, fp32 sums), so there is no split-K
// hand-off (graph-replayed over pooled weights, W[256, 2048]: M = 6 / 8
// 4.46-4.64 -> 3.98-4.01 us, M = 16 5.04-5.10 -> 4.37-4.44, M = 32 5.77 ->
// 5.21-5.25).  Past that each workgroup streams too much of the activation
// (M * K * 2 bytes over the row groups): M = 64 went from 7.2 to 7.7 us, and
// W[96, 5120] at 8 rows ran 0.2-0.4 us slower inside the bench step (3%
// faster alone), so those keep the split MFMA form.  Thread t takes the 16-byte chunks t, t + T, ... of
// the weight row and of each activation row; all NCH chunks' loads are
// issued before any arithmetic (chunk indices past K re-read the last chunk
// and are zeroed afterwards), then each row's sum goes through a wave
// reduction and the T/64 wave partials are added in wave order.
template <int MR, int T, int NCH>
__global__ __launch_bounds__(T) void k_skinny_dot(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                  uint16_t* __restrict__ c, int M, int N, int K) {
  constexpr int kW = T / 64;
  __shared__ float red[kW][MR];
  const int n = blockIdx.x;
  // blockIdx.y takes rows 8y .. 8y + 7 (at most MR)
  x += static_cast<size_t>(blockIdx.y) * MR * K;
  c += static_cast<size_t>(blockIdx.y) * MR * N;
  M -= blockIdx.y * MR;
  const int t = threadIdx.x, wave = t >> 6, l = t & 63;
  const int nch = K >> 3;
  const uint4* wr = reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * K);
  uint4 wv[NCH], xv[NCH][MR];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ch = min(t + j * T, nch - 1);
    wv[j] = wr[ch];
#pragma unroll
    for (int m = 0; m < MR; ++m)
      xv[j][m] = reinterpret_cast<const uint4*>(x + static_cast<size_t>(min(m, M - 1)) * K)[ch];
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint32_t keep = t + j * T < nch ? 0xFFFFFFFFu : 0u;
    const uint4 wk = make_uint4(wv[j].x & keep, wv[j].y & keep, wv[j].z & keep, wv[j].w & keep);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wk.x), as_bf2(xv[j][m].x), acc[m], false);
      acc[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wk.y), as_bf2(xv[j][m].y), acc[m], false);
      acc[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wk.z), as_bf2(xv[j][m].z), acc[m], false);
      acc[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wk.w), as_bf2(xv[j][m].w), acc[m], false);
    }
  }
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (l == 0) red[wave][m] = v;
  }
  __syncthreads();
  if (t < MR && t < M) {
    float s = red[0][t];
#pragma unroll
    for (int i = 1; i < kW; ++i) s += red[i][t];
    c[static_cast<size_t>(t) * N + n] = static_cast<uint16_t>(bf16x2_rne(s, 0.0f));
  }
}

}  // namespace

int bs_skinny_ksplit(int K) { return ((K + kChunk - 1) / kChunk + kWaves - 1) / kWaves; }

namespace {
// whether the VALU form (one column per workgroup, no split) takes the call
bool skinny_dot(int M, int K) { return M <= 32 && K <= 2048; }
}  // namespace

namespace {
int skinny_mb(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
size_t skinny_slab_bytes(int M, int N, int ks) {
  return static_cast<size_t>(ks) * (N / 16) * skinny_mb(M) * 256 * sizeof(float);
}
}  // namespace

size_t bs_skinny_workspace(int M, int N, int K) {
  const int ks = bs_skinny_ksplit(K);
  if (ks <= 1 || skinny_dot(M, K)) return 0;
  return kWsCounterBytes + skinny_slab_bytes(M, N, ks);
}

int bs_launch_skinny(const uint16_t* x, const uint16_t* w, uint16_t* c, int M, int N, int K, void* ws,
                     hipStream_t st) {
  if (skinny_dot(M, K)) {
    // K <= 2048: at most 256 16-byte chunks per row, one per thread
    k_skinny_dot<8, 256, 1><<<dim3(N, (M + 7) / 8), dim3(256), 0, st>>>(x, w, c, M, N, K);
    return bs_launch_status();
  }
  const int ks = bs_skinny_ksplit(K);
  float* slab = nullptr;
  int* counters = nullptr;
  if (ks > 1) {
    if (N / 16 > kWsMaxCounters) return BS_ERR_SHAPE;  // one counter per 16-column tile
    counters = static_cast<int*>(ws);
    slab = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kWsCounterBytes);
  }
  dim3 grid(N / 16, ks);
  if (M <= 16) k_skinny<1><<<grid, 256, 0, st>>>(x, w, c, M, N, K, slab, counters);
  else if (M <= 32) k_skinny<2><<<grid, 256, 0, st>>>(x, w, c, M, N, K, slab, counters);
  else k_skinny<4><<<grid, 256, 0, st>>>(x, w, c, M, N, K, slab, counters);
  return bs_launch_status();
}

// ---------------------------------------------------------------------------
// The same GEMM for callers that cannot allocate: its split-K scratch is a
// static device array instead of a caller workspace.  Each GPU the library
// runs on holds its own copy of the array (zero-filled when the code object
// is loaded) until the process ends.  In host code `scratch` names a host-side
// stand-in, not a device address: the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that
// pointer is handed to kernels.
namespace {
constexpr size_t kScratchBytes = BS_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kWsCounterBytes && kScratchBytes % 256 == 0, "scratch layout");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void k_zero_words(int* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// The device address of `scratch` on the device of stream st (which must be
// the current device).  The first call on a device looks it up and clears
// the counter region with a kernel on st (a kernel rather than a memset, so
// that the clear is also valid if it lands inside a captured graph).
int scratch_for(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BS_ERR_DEVICE;
  if (st != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(st, &sdev) != hipSuccess || sdev != dev) return BS_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return BS_ERR_LAUNCH;
    constexpr int kWords = static_cast<int>(kWsCounterBytes / sizeof(int));
    k_zero_words<<<(kWords + 255) / 256, 256, 0, st>>>(static_cast<int*>(ptr), kWords);
    if (hipGetLastError() != hipSuccess) return BS_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BS_OK;
}
}  // namespace

extern "C" BS_API int gemm_bf16_skinny_noalloc(const void* x, const void* w, void* c, int M, int N, int K,
                                               bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(x && w && c, BS_ERR_NULL);
  BS_CHECK(M >= 1 && M <= 64 && N >= 16 && N % 16 == 0 && K >= 32 && K % 32 == 0, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(x, 16) && bs_aligned(w, 16) && bs_aligned(c, 4), BS_ERR_ALIGN);
  const size_t need = bs_skinny_workspace(M, N, K);
  BS_CHECK(need <= kScratchBytes, BS_ERR_SCRATCH);
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_for(st, &ws);
    if (rc != BS_OK) return rc;
  }
  return bs_launch_skinny(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                          static_cast<uint16_t*>(c), M, N, K, ws, st);
}
