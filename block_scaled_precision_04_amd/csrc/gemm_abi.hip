// C-ABI entry points of the GEMMs: host-side validation, then dispatch on the
// M regime (small M: weight-streaming decode kernels; large M: LDS-tiled
// scaled-MFMA kernel).  Nothing here touches device memory from the host.
#include "common.h"

int bs_launch_fp8_block_decode(const uint8_t* a, int64_t lda, const float* as, int64_t asm_, int64_t asg,
                               const uint8_t* w, const float* ws, uint16_t* c, int64_t ldc, int M, int N, int K,
                               void* work, hipStream_t st);
int bs_launch_w4a8_decode(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                          uint16_t* c, int64_t ldc, int M, int N, int K, void* work, hipStream_t st);
size_t bs_decode_workspace(int M, int N, int K, bool mx);
int bs_launch_fp8_block_prefill(const uint8_t* a, int64_t lda, const float* as, int64_t as_m, int64_t as_g,
                                const uint8_t* w, const float* ws, uint16_t* c, int64_t ldc, int M, int N, int K,
                                hipStream_t st);
bool bs_fp8_use_tiled(int M, int N, int K);
int bs_launch_w4a8_prefill(const uint8_t* a, int64_t lda, const float* as, const uint8_t* w, const uint32_t* wsc,
                           uint16_t* c, int64_t ldc, int M, int N, int K, void* ws, bool a_tiled, hipStream_t st);
size_t bs_prefill_workspace(int M, int N, int K);
int bs_launch_skinny(const uint16_t* x, const uint16_t* w, uint16_t* c, int M, int N, int K, void* ws,
                     hipStream_t st);
size_t bs_skinny_workspace(int M, int N, int K);

namespace {
constexpr int kW4A8DecodeMaxM = 64;  // above this the compute-bound tiled kernel runs
constexpr int kSkinnyMaxM = 64;
constexpr int kFp8MaxM = 1 << 20;

// A split-K launch needs a workspace of at least `need` bytes, 256-aligned.
int check_workspace(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return BS_OK;
  if (ws == nullptr || ws_bytes < need) return BS_ERR_WORKSPACE;
  if (!bs_aligned(ws, 256)) return BS_ERR_ALIGN;
  return BS_OK;
}
}  // namespace

extern "C" {

BS_API const char* bs_status_string(int status) {
  switch (status) {
    case BS_OK: return "ok";
    case BS_ERR_NULL: return "null pointer";
    case BS_ERR_SHAPE: return "unsupported shape";
    case BS_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case BS_ERR_LAYOUT: return "weight descriptor does not match";
    case BS_ERR_WORKSPACE: return "workspace missing or too small";
    case BS_ERR_LAUNCH: return "kernel launch failed";
    case BS_ERR_ARG: return "invalid argument";
    case BS_ERR_DEVICE: return "no usable device, or the stream belongs to another device";
    case BS_ERR_SCRATCH: return "shape needs more than the static scratch array";
    default: return "unknown status";
  }
}

BS_API int bs_version(void) { return 100; }

namespace {
// A weight descriptor is accepted only when every field is what the
// pre-layout of this shape writes (bs_prelayout_fp8_block /
// bs_prelayout_mxfp4): one filled by hand, or for another shape or layout,
// is refused with BS_ERR_LAYOUT before anything is read through it.
bool fp8_desc_ok(const bs_wdesc* d, int N, int K) {
  const uint64_t codes = static_cast<uint64_t>(N) * static_cast<uint64_t>(K);
  return d->magic == BS_WDESC_MAGIC && d->layout == BS_LAYOUT_FP8_BLOCK && d->N == N && d->K == K &&
         d->codes_bytes == codes && d->scales_offset == 0 && d->scales_bytes == 0 && d->total_bytes == codes;
}
bool mx_desc_ok(const bs_wdesc* d, int N, int K) {
  const uint64_t codes = static_cast<uint64_t>(N) * static_cast<uint64_t>(K) / 2;
  const uint64_t off = (codes + 255) / 256 * 256;
  const uint64_t scales = static_cast<uint64_t>(N / 16) * static_cast<uint64_t>((K / 128 + 3) / 4) * 256;
  return d->magic == BS_WDESC_MAGIC && d->layout == BS_LAYOUT_MXFP4 && d->N == N && d->K == K &&
         d->codes_bytes == codes && d->scales_offset == off && d->scales_bytes == scales &&
         d->total_bytes == off + scales;
}
}  // namespace

BS_API size_t bs_workspace_bytes(int op, int M, int N, int K) {
  if (op == BS_OP_BF16_SKINNY) {
    if (M < 1 || M > kSkinnyMaxM || N < 16 || N % 16 || K < 32 || K % 32) return 0;
    return bs_skinny_workspace(M, N, K);
  }
  if (op == BS_OP_FP8_BLOCK) {
    if (M < 1 || M > kFp8MaxM || N < 128 || N % 128 || K < 128 || K % 128) return 0;
    return bs_fp8_use_tiled(M, N, K) ? 0 : bs_decode_workspace(M, N, K, false);
  }
  if (op == BS_OP_W4A8_MXFP4) {
    if (M < 1 || M > (1 << 22) || N < 16 || N % 16 || K < 128 || K % 128) return 0;
    return M <= kW4A8DecodeMaxM ? bs_decode_workspace(M, N, K, true) : bs_prefill_workspace(M, N, K);
  }
  return 0;
}

BS_API int bsgemm_fp8_block(const void* a, int64_t lda, const float* a_scale, int64_t as_stride_m,
                            int64_t as_stride_g, const bs_wdesc* wd, const void* w_pre, const float* w_scale,
                            void* c, int64_t ldc, int M, int N, int K, void* ws, size_t ws_bytes,
                            bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(a && a_scale && wd && w_pre && w_scale && c, BS_ERR_NULL);
  BS_CHECK(M >= 1 && M <= kFp8MaxM && N >= 128 && N % 128 == 0 && K >= 128 && K % 128 == 0, BS_ERR_SHAPE);
  BS_CHECK(fp8_desc_ok(wd, N, K), BS_ERR_LAYOUT);
  BS_CHECK(lda >= K && lda % 16 == 0 && ldc >= N && ldc % 4 == 0, BS_ERR_ALIGN);
  BS_CHECK(lda < (1 << 25), BS_ERR_SHAPE);  // activation rows are addressed with 32-bit offsets
  BS_CHECK(bs_aligned(a, 16) && bs_aligned(w_pre, 16) && bs_aligned(c, 16) && bs_aligned(a_scale, 4) &&
               bs_aligned(w_scale, 4),
           BS_ERR_ALIGN);
  BS_CHECK(as_stride_m >= 0 && as_stride_g >= 0, BS_ERR_ARG);
  BS_CHECK(K < (1 << 24), BS_ERR_SHAPE);  // weight tiles are addressed with 32-bit offsets
  // the tiled kernel addresses a tile's activation rows (256 * lda), activation
  // scales (256 * as_stride_m floats) and weight scales ((N/128) * (K/128)
  // floats) with unsigned 32-bit offsets
  BS_CHECK(as_stride_m < (1 << 22), BS_ERR_SHAPE);
  if (bs_fp8_use_tiled(M, N, K)) {
    BS_CHECK(lda < (1 << 24) && static_cast<uint64_t>(N / 128) * (K / 128) < (1ull << 30), BS_ERR_SHAPE);
    return bs_launch_fp8_block_prefill(static_cast<const uint8_t*>(a), lda, a_scale, as_stride_m, as_stride_g,
                                       static_cast<const uint8_t*>(w_pre), w_scale, static_cast<uint16_t*>(c), ldc,
                                       M, N, K, static_cast<hipStream_t>(stream));
  }
  const int wst = check_workspace(bs_decode_workspace(M, N, K, false), ws, ws_bytes);
  if (wst != BS_OK) return wst;
  return bs_launch_fp8_block_decode(static_cast<const uint8_t*>(a), lda, a_scale, as_stride_m, as_stride_g,
                                    static_cast<const uint8_t*>(w_pre), w_scale, static_cast<uint16_t*>(c), ldc,
                                    M, N, K, ws, static_cast<hipStream_t>(stream));
}

BS_API int bsgemm_w4a8_mxfp4(const void* a, int64_t lda, const float* a_scale, const bs_wdesc* wd,
                             const void* w_pre, void* c, int64_t ldc, int M, int N, int K, void* ws,
                             size_t ws_bytes, bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(a && a_scale && wd && w_pre && c, BS_ERR_NULL);
  BS_CHECK(M >= 1 && M <= (1 << 22) && N >= 16 && N % 16 == 0 && K >= 128 && K % 128 == 0, BS_ERR_SHAPE);
  BS_CHECK(mx_desc_ok(wd, N, K), BS_ERR_LAYOUT);
  BS_CHECK(lda >= K && lda % 16 == 0 && ldc >= N && ldc % 4 == 0, BS_ERR_ALIGN);
  BS_CHECK(bs_aligned(a, 16) && bs_aligned(w_pre, 256) && bs_aligned(c, 16) && bs_aligned(a_scale, 4),
           BS_ERR_ALIGN);
  // both kernels address the activation, and the tiled kernel the weight
  // codes (N * K / 2 bytes), with unsigned 32-bit offsets
  BS_CHECK(static_cast<uint64_t>(M) * static_cast<uint64_t>(lda) < (1ull << 32) && lda < (1 << 25), BS_ERR_SHAPE);
  BS_CHECK(static_cast<uint64_t>(N) * static_cast<uint64_t>(K) / 2 < (1ull << 32), BS_ERR_SHAPE);
  const uint8_t* w = static_cast<const uint8_t*>(w_pre);
  const uint32_t* wsc = reinterpret_cast<const uint32_t*>(w + wd->scales_offset);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M <= kW4A8DecodeMaxM) {
    const int wst = check_workspace(bs_decode_workspace(M, N, K, true), ws, ws_bytes);
    if (wst != BS_OK) return wst;
    return bs_launch_w4a8_decode(static_cast<const uint8_t*>(a), lda, a_scale, w, wsc, static_cast<uint16_t*>(c),
                                 ldc, M, N, K, ws, st);
  }
  const int wst = check_workspace(bs_prefill_workspace(M, N, K), ws, ws_bytes);
  if (wst != BS_OK) return wst;
  return bs_launch_w4a8_prefill(static_cast<const uint8_t*>(a), lda, a_scale, w, wsc, static_cast<uint16_t*>(c),
                                ldc, M, N, K, ws, false, st);
}

BS_API int bsgemm_w4a8_mxfp4_atiled(const void* a_tiled, const float* a_scale, const bs_wdesc* wd, const void* w_pre,
                                    void* c, int64_t ldc, int M, int N, int K, void* ws, size_t ws_bytes,
                                    bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(a_tiled && a_scale && wd && w_pre && c, BS_ERR_NULL);
  BS_CHECK(M > kW4A8DecodeMaxM && M <= (1 << 22) && N >= 16 && N % 16 == 0 && K >= 128 && K % 128 == 0,
           BS_ERR_SHAPE);
  BS_CHECK(mx_desc_ok(wd, N, K), BS_ERR_LAYOUT);
  BS_CHECK(ldc >= N && ldc % 4 == 0, BS_ERR_ALIGN);
  BS_CHECK(bs_aligned(a_tiled, 16) && bs_aligned(w_pre, 256) && bs_aligned(c, 16) && bs_aligned(a_scale, 4),
           BS_ERR_ALIGN);
  // the tiled activation (rows padded to 32) and the weight codes are
  // addressed with unsigned 32-bit offsets
  BS_CHECK(static_cast<uint64_t>((M + 31) / 32) * 32 * static_cast<uint64_t>(K) < (1ull << 32), BS_ERR_SHAPE);
  BS_CHECK(static_cast<uint64_t>(N) * static_cast<uint64_t>(K) / 2 < (1ull << 32), BS_ERR_SHAPE);
  const int wst = check_workspace(bs_prefill_workspace(M, N, K), ws, ws_bytes);
  if (wst != BS_OK) return wst;
  const uint8_t* w = static_cast<const uint8_t*>(w_pre);
  return bs_launch_w4a8_prefill(static_cast<const uint8_t*>(a_tiled), K, a_scale, w,
                                reinterpret_cast<const uint32_t*>(w + wd->scales_offset), static_cast<uint16_t*>(c),
                                ldc, M, N, K, ws, true, static_cast<hipStream_t>(stream));
}

BS_API int gemm_bf16_skinny(const void* x, const void* w, void* c, int M, int N, int K, void* ws, size_t ws_bytes,
                            bs_stream_t stream) {
  if (M == 0) return BS_OK;  // an empty batch: nothing is read or launched
  BS_CHECK(x && w && c, BS_ERR_NULL);
  BS_CHECK(M >= 1 && M <= kSkinnyMaxM && N >= 16 && N % 16 == 0 && K >= 32 && K % 32 == 0, BS_ERR_SHAPE);
  BS_CHECK(bs_aligned(x, 16) && bs_aligned(w, 16) && bs_aligned(c, 4), BS_ERR_ALIGN);
  const int wst = check_workspace(bs_skinny_workspace(M, N, K), ws, ws_bytes);
  if (wst != BS_OK) return wst;
  return bs_launch_skinny(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w),
                          static_cast<uint16_t*>(c), M, N, K, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"
