// One-time weight re-layout into gfx950 MFMA fragment order, and its exact
// inverse (radiance_kernels.py page, install_load_hook: the weight is shuffled
// once at load; radiance_mxfp4.py page, the WPERM comment and permute_w /
// unpermute_w: a byte permutation that makes a wave's weight read contiguous,
// never a re-quantisation).
//
// Fragment order (gfx950 16x16x128 8/4-bit MFMA operand): weight rows are cut
// into 16-row tiles and K into 128-wide steps; in each (tile nt, step ks),
// lane l owns row 16*nt + l%16 and the 32 K values starting at 32*(l/16).
//   FP8 block  2 KiB per (nt, ks): half h (1 KiB) holds 16 bytes per lane,
//              K offsets 32*(l/16) + 16*h .. +16.
//   MXFP4      1 KiB per (nt, ks): 16 packed bytes per lane (its 32 values);
//              then e8m0 scales, one dword per lane per (nt, group of four
//              steps), byte ks%4, pad 0x7F.
// Every kernel moves 16-byte chunks except the scale gather (4 bytes).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// chunk index i over the pre-laid-out FP8 buffer (16 bytes each):
// i = ((nt*KS + ks)*2 + h)*64 + lane
BS_INLINE size_t fp8_src_chunk(size_t i, int KS, int K) {
  const int lane = static_cast<int>(i & 63);
  const size_t t = i >> 6;
  const int h = static_cast<int>(t & 1);
  const size_t u = t >> 1;
  const int ks = static_cast<int>(u % KS);
  const size_t nt = u / KS;
  const size_t n = nt * 16 + (lane & 15);
  const size_t k = static_cast<size_t>(ks) * 128 + 32 * (lane >> 4) + 16 * h;
  return (n * K + k) >> 4;
}

__global__ __launch_bounds__(kThreads) void k_fp8_pre(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                      size_t nchunks, int KS, int K, bool inverse) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  const size_t s = fp8_src_chunk(i, KS, K);
  if (inverse) dst[s] = src[i];
  else dst[i] = src[s];
}

// MXFP4 codes: chunk i = (nt*KS + ks)*64 + lane -> row n, packed byte offset
// 64*ks + 16*(lane/16) of a [N, K/2] row.
BS_INLINE size_t mx_src_chunk(size_t i, int KS, int Kh) {
  const int lane = static_cast<int>(i & 63);
  const size_t t = i >> 6;
  const int ks = static_cast<int>(t % KS);
  const size_t nt = t / KS;
  const size_t n = nt * 16 + (lane & 15);
  const size_t p = static_cast<size_t>(ks) * 64 + 16 * (lane >> 4);
  return (n * Kh + p) >> 4;
}

__global__ __launch_bounds__(kThreads) void k_mx_codes(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                       size_t nchunks, int KS, int Kh, bool inverse) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  const size_t s = mx_src_chunk(i, KS, Kh);
  if (inverse) dst[s] = src[i];
  else dst[i] = src[s];
}

// MXFP4 scales: dword i = (nt*KQ + kq)*64 + lane holds E[n][4*(4kq + r) + lane/16]
// in byte r, for the steps 4kq + r < KS; other bytes are 0x7F.
__global__ __launch_bounds__(kThreads) void k_mx_scales(const uint8_t* __restrict__ e, uint32_t* __restrict__ dst,
                                                        size_t ndwords, int KS, int KQ, int K32) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= ndwords) return;
  const int lane = static_cast<int>(i & 63);
  const size_t t = i >> 6;
  const int kq = static_cast<int>(t % KQ);
  const size_t nt = t / KQ;
  const size_t n = nt * 16 + (lane & 15);
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ks = 4 * kq + r;
    const uint32_t b = ks < KS ? e[n * K32 + 4 * ks + (lane >> 4)] : 0x7Fu;
    v |= b << (8 * r);
  }
  dst[i] = v;
}

__global__ __launch_bounds__(kThreads) void k_mx_scales_inv(const uint32_t* __restrict__ src, uint8_t* __restrict__ e,
                                                            size_t ndwords, int KS, int KQ, int K32) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= ndwords) return;
  const int lane = static_cast<int>(i & 63);
  const size_t t = i >> 6;
  const int kq = static_cast<int>(t % KQ);
  const size_t nt = t / KQ;
  const size_t n = nt * 16 + (lane & 15);
  const uint32_t v = src[i];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ks = 4 * kq + r;
    if (ks < KS) e[n * K32 + 4 * ks + (lane >> 4)] = static_cast<uint8_t>(v >> (8 * r));
  }
}

inline unsigned blocks_for(size_t n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }

bool shape_ok(int N, int K) { return N >= 16 && N % 16 == 0 && K >= 128 && K % 128 == 0; }

uint64_t mx_codes_bytes(int N, int K) { return static_cast<uint64_t>(N) * K / 2; }
uint64_t mx_scale_bytes(int N, int K) { return static_cast<uint64_t>(N / 16) * ((K / 128 + 3) / 4) * 256; }
uint64_t mx_scale_off(int N, int K) { return (mx_codes_bytes(N, K) + 255) / 256 * 256; }

}  // namespace

extern "C" {

BS_API size_t bs_prelayout_fp8_block_bytes(int N, int K) {
  return shape_ok(N, K) ? static_cast<size_t>(N) * K : 0;
}

BS_API int bs_prelayout_fp8_block(const void* w, void* out, size_t out_bytes, int N, int K, bs_wdesc* desc,
                                  bs_stream_t stream) {
  BS_CHECK(w && out && desc, BS_ERR_NULL);
  BS_CHECK(shape_ok(N, K), BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(w, 16) && bs_aligned(out, 16), BS_ERR_ALIGN);
  const size_t bytes = static_cast<size_t>(N) * K;
  BS_CHECK(out_bytes >= bytes, BS_ERR_ARG);
  const size_t nchunks = bytes / 16;
  k_fp8_pre<<<blocks_for(nchunks), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(w), static_cast<uint4*>(out), nchunks, K / 128, K, false);
  const int st = bs_launch_status();
  if (st != BS_OK) return st;
  *desc = bs_wdesc{BS_WDESC_MAGIC, BS_LAYOUT_FP8_BLOCK, N, K, bytes, 0, 0, bytes};
  return BS_OK;
}

BS_API int bs_unprelayout_fp8_block(const bs_wdesc* d, const void* pre, void* w, bs_stream_t stream) {
  BS_CHECK(d && pre && w, BS_ERR_NULL);
  BS_CHECK(d->magic == BS_WDESC_MAGIC && d->layout == BS_LAYOUT_FP8_BLOCK && shape_ok(d->N, d->K), BS_ERR_LAYOUT);
  BS_CHECK(bs_aligned(w, 16) && bs_aligned(pre, 16), BS_ERR_ALIGN);
  const size_t nchunks = static_cast<size_t>(d->N) * d->K / 16;
  k_fp8_pre<<<blocks_for(nchunks), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(pre), static_cast<uint4*>(w), nchunks, d->K / 128, d->K, true);
  return bs_launch_status();
}

BS_API size_t bs_prelayout_mxfp4_bytes(int N, int K) {
  return shape_ok(N, K) ? static_cast<size_t>(mx_scale_off(N, K) + mx_scale_bytes(N, K)) : 0;
}

BS_API int bs_prelayout_mxfp4(const void* wp, const void* e8, void* out, size_t out_bytes, int N, int K,
                              bs_wdesc* desc, bs_stream_t stream) {
  BS_CHECK(wp && e8 && out && desc, BS_ERR_NULL);
  BS_CHECK(shape_ok(N, K), BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(wp, 16) && bs_aligned(out, 256), BS_ERR_ALIGN);
  const uint64_t total = mx_scale_off(N, K) + mx_scale_bytes(N, K);
  BS_CHECK(out_bytes >= total, BS_ERR_ARG);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t nchunks = mx_codes_bytes(N, K) / 16;
  k_mx_codes<<<blocks_for(nchunks), kThreads, 0, st>>>(static_cast<const uint4*>(wp), static_cast<uint4*>(out),
                                                        nchunks, K / 128, K / 2, false);
  int s = bs_launch_status();
  if (s != BS_OK) return s;
  const size_t ndw = mx_scale_bytes(N, K) / 4;
  k_mx_scales<<<blocks_for(ndw), kThreads, 0, st>>>(
      static_cast<const uint8_t*>(e8),
      reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + mx_scale_off(N, K)), ndw, K / 128,
      (K / 128 + 3) / 4, K / 32);
  s = bs_launch_status();
  if (s != BS_OK) return s;
  *desc = bs_wdesc{BS_WDESC_MAGIC, BS_LAYOUT_MXFP4, N, K, mx_codes_bytes(N, K), mx_scale_off(N, K),
                   mx_scale_bytes(N, K), total};
  return BS_OK;
}

BS_API int bs_unprelayout_mxfp4(const bs_wdesc* d, const void* pre, void* wp, void* e8, bs_stream_t stream) {
  BS_CHECK(d && pre && wp && e8, BS_ERR_NULL);
  BS_CHECK(d->magic == BS_WDESC_MAGIC && d->layout == BS_LAYOUT_MXFP4 && shape_ok(d->N, d->K) &&
               d->scales_offset == mx_scale_off(d->N, d->K),
           BS_ERR_LAYOUT);
  BS_CHECK(bs_aligned(wp, 16) && bs_aligned(pre, 256), BS_ERR_ALIGN);
  const int N = d->N, K = d->K;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t nchunks = mx_codes_bytes(N, K) / 16;
  k_mx_codes<<<blocks_for(nchunks), kThreads, 0, st>>>(static_cast<const uint4*>(pre), static_cast<uint4*>(wp),
                                                        nchunks, K / 128, K / 2, true);
  int s = bs_launch_status();
  if (s != BS_OK) return s;
  const size_t ndw = mx_scale_bytes(N, K) / 4;
  k_mx_scales_inv<<<blocks_for(ndw), kThreads, 0, st>>>(
      reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(pre) + d->scales_offset),
      static_cast<uint8_t*>(e8), ndw, K / 128, (K / 128 + 3) / 4, K / 32);
  return bs_launch_status();
}

}  // extern "C"
