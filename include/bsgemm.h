/*
 * bsgemm: block-scaled low-precision linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a DEVICE pointer owned by the caller; the
 * library never allocates, frees or synchronizes, and never reads device
 * memory from the host.  Work is enqueued on the given stream (a hipStream_t;
 * NULL means the default stream) and the call returns without waiting.
 * Arguments are validated on the host before anything is launched: on a
 * failed check the call returns a negative status and enqueues nothing.  A
 * launch failure returns BS_ERR_LAUNCH.  No C++ exception crosses this ABI.
 * A call with zero rows (M == 0 for the GEMMs, producers and activation
 * quantizers) is an empty batch: it returns BS_OK before reading any other
 * argument (pointers may be NULL) and launches nothing.
 * The library keeps no state between calls and is safe to call from several
 * host threads.
 *
 * The operations follow the "vllm-sly-radiance" pages:
 *   radiance_kernels.py  block-FP8 W8A8 GEMM routing (block_scaled_mm), the
 *                        one-time weight re-layout at load (install_load_hook),
 *                        activation scales passed by strides, not copied;
 *   radiance_gemm.py     the skinny bf16 NT GEMM for sub-megabyte weights
 *                        (gemm_bf16_nt_m64, maybe_gemm / config_for);
 *   radiance_mxfp4.py    the MXFP4 W4A8 linear (module docstring, _exact_ref,
 *                        permute_w, the per-token quant _traced_quant, the
 *                        decode split-K scratch);
 *   radiance_arnq.py     the fused residual add + Gemma RMSNorm + per-token
 *                        fp8 quant (ar_add_rms_quant, launch_add_rms_quant) and
 *                        the SiLU * up + quant producer (silu_mul_quant).
 *
 * Formats: e4m3 is OCP FP8 e4m3fn (max 448, no infinities); e2m1 is OCP FP4
 * packed two per byte, the even element in the low nibble; e8m0 is an MX
 * scale 2^(e-127); bf16 is stored as uint16_t bit patterns.  Matrices are
 * row-major unless stated.
 */
#ifndef BSGEMM_H
#define BSGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BS_API __attribute__((visibility("default")))

typedef void* bs_stream_t; /* hipStream_t; NULL = default stream */

/* ---------------------------------------------------------------- status */
enum {
  BS_OK = 0,
  BS_ERR_NULL = -1,      /* a required pointer is NULL                         */
  BS_ERR_SHAPE = -2,     /* a size is out of range or not a required multiple  */
  BS_ERR_ALIGN = -3,     /* a pointer or leading dimension breaks alignment    */
  BS_ERR_LAYOUT = -4,    /* weight descriptor does not match the call          */
  BS_ERR_WORKSPACE = -5, /* workspace missing or smaller than required         */
  BS_ERR_LAUNCH = -6,    /* the HIP runtime refused a launch                   */
  BS_ERR_DEVICE = -7,    /* no usable current device, or the stream is on      */
                         /* another device                                     */
  BS_ERR_SCRATCH = -8,   /* the shape needs more than the static scratch array */
  BS_ERR_ARG = -9        /* any other invalid argument                         */
};

/* Human-readable name of a status code (static string). */
BS_API const char* bs_status_string(int status);
/* Library version as major*10000 + minor*100 + patch. */
BS_API int bs_version(void);

/* ------------------------------------------------------- weight layouts
 * One-time re-layout of a weight into gfx950 MFMA fragment order, done at
 * load time (radiance_kernels.py page, install_load_hook; radiance_mxfp4.py
 * page, the WPERM comment and permute_w).  It is a byte permutation, not a
 * re-quantisation, and has an exact inverse.  The layout is recorded in a
 * HOST-side descriptor that every GEMM call checks field by field against
 * what the pre-layout of its (N, K) writes, so a weight in the wrong layout,
 * or a descriptor of another shape, is an error (BS_ERR_LAYOUT), never
 * silently misread.
 *
 * Order: the weight is cut into 16-row tiles and 128-wide K steps.  In each
 * (tile nt, step ks), lane l of a 64-lane wave owns row 16*nt + l%16 and the
 * 32 K values starting at 128*ks + 32*(l/16).
 *   FP8 block:  per (nt, ks) 2 KiB: two 1 KiB halves; half h holds, for lane l,
 *               16 bytes W[n][128ks + 32(l/16) + 16h .. +16] at offset 16*l.
 *   MXFP4:      codes, per (nt, ks) 1 KiB: lane l holds the 16 packed bytes of
 *               its 32 K values at offset 16*l.  Then the e8m0 scales, per
 *               (nt, 4 consecutive ks) 256 B: lane l's dword holds the scales
 *               of its row and K-block l/16 for those four steps (byte = ks%4;
 *               unused bytes of a final partial dword are 0x7F).
 */
enum {
  BS_LAYOUT_FP8_BLOCK = 0x38423631, /* e4m3 codes, 16x128 fragment order   */
  BS_LAYOUT_MXFP4 = 0x34584D31      /* e2m1 codes + e8m0, fragment order   */
};
#define BS_WDESC_MAGIC 0x42534744u

typedef struct bs_wdesc {
  uint32_t magic;         /* BS_WDESC_MAGIC once filled                        */
  uint32_t layout;        /* BS_LAYOUT_*                                       */
  int32_t N, K;           /* logical weight shape [N, K]                       */
  uint64_t codes_bytes;   /* bytes of the code section (at offset 0)           */
  uint64_t scales_offset; /* MXFP4: byte offset of the e8m0 section (256-aligned) */
  uint64_t scales_bytes;  /* MXFP4: bytes of the e8m0 section; 0 for FP8 block */
  uint64_t total_bytes;   /* bytes the pre-laid-out buffer must hold           */
} bs_wdesc;

/* Bytes needed for a pre-laid-out block-FP8 weight (N*K), 0 on bad shape. */
BS_API size_t bs_prelayout_fp8_block_bytes(int N, int K);
/* w_e4m3: [N, K] e4m3 codes, row-major.  N % 16 == 0, K % 128 == 0 (the GEMM
 * itself needs N % 128 == 0).  out: out_bytes >= the size above, 16-byte
 * aligned.  Fills *desc (host memory).  The per-128x128-block fp32 scales are
 * not moved: they are passed to the GEMM as they are. */
BS_API int bs_prelayout_fp8_block(const void* w_e4m3, void* out, size_t out_bytes, int N, int K,
                                  bs_wdesc* desc, bs_stream_t stream);
/* Exact inverse: pre-laid-out bytes back to [N, K] row-major codes. */
BS_API int bs_unprelayout_fp8_block(const bs_wdesc* desc, const void* pre, void* w_e4m3,
                                    bs_stream_t stream);

/* Bytes needed for a pre-laid-out MXFP4 weight (codes + scales), 0 on bad shape. */
BS_API size_t bs_prelayout_mxfp4_bytes(int N, int K);
/* w_packed: [N, K/2] packed e2m1 (even k in the low nibble); w_e8m0: [N, K/32]
 * (the checkpoint order; the pages' kernel reads it transposed, here it is
 * re-laid-out with the codes).  N % 16 == 0, K % 128 == 0. */
BS_API int bs_prelayout_mxfp4(const void* w_packed, const void* w_e8m0, void* out, size_t out_bytes,
                              int N, int K, bs_wdesc* desc, bs_stream_t stream);
/* Exact inverse: back to [N, K/2] codes and [N, K/32] scales. */
BS_API int bs_unprelayout_mxfp4(const bs_wdesc* desc, const void* pre, void* w_packed, void* w_e8m0,
                                bs_stream_t stream);

/* ---------------------------------------------------------- workspaces
 * Some shapes split K across workgroups and reduce through a caller-provided
 * workspace (int32 counters + fp32 partial slab, as the pages' decode split-K
 * scratch: allocated once outside graph capture, zeroed once; the last
 * workgroup to finish a tile reduces it in a fixed order and resets its
 * counter, so the workspace is left zeroed-ready for the next call).  The
 * caller zero-fills it ONCE after allocation.  Layout: the first 64 KiB hold
 * the counters, the partials follow; no call writes partials into the counter
 * region, so one workspace may serve any sequence of calls, of any ops and
 * shapes, whose bs_workspace_bytes it covers.  Calls that share a workspace
 * must be ordered (same stream); 0 means no workspace is needed.  A split
 * that would need more than 16384 counters (one per 16-column tile group)
 * is refused with BS_ERR_SHAPE.
 * Memory kind: ordinary device memory of the GPU the call runs on (hipMalloc,
 * coarse-grained).  The workgroups of one tile may run on different XCDs,
 * whose L2 caches are not coherent with each other; the hand-off works
 * because the partials are written and read with device-scope (sc1) memory
 * instructions and each workgroup waits for its partial stores to be
 * acknowledged before it bumps the counter with a device-scope atomic.  The
 * test suite pins that encoding in the compiled kernels. */
enum { BS_OP_FP8_BLOCK = 1, BS_OP_W4A8_MXFP4 = 2, BS_OP_BF16_SKINNY = 3 };
BS_API size_t bs_workspace_bytes(int op, int M, int N, int K);

/* ------------------------------------------------------------- GEMMs */

/* Block-FP8 W8A8 GEMM (radiance_kernels.py page, block_scaled_mm):
 *   C[m,n] = bf16( sum_g a_scale[m,g] * w_scale[n/128, g] * sum_{k in group g} A[m,k] W[n,k] )
 * a:       e4m3 [M, K], leading dimension lda (bytes, multiple of 16).
 * a_scale: fp32, element (m, g) at a_scale[m*as_stride_m + g*as_stride_g]
 *          (g = k/128); strides describe row- or column-major storage, so a
 *          column-major scale needs no transpose copy.
 * w_pre:   the weight pre-laid-out by bs_prelayout_fp8_block (desc wd).
 * w_scale: fp32 [N/128, K/128] row-major, one multiplicative scale per block.
 * c:       bf16 [M, N], leading dimension ldc (elements, multiple of 4).
 * ws:      bs_workspace_bytes(BS_OP_FP8_BLOCK, M, N, K) bytes (256-byte
 *          aligned, zeroed once) when that is non-zero: K split across
 *          workgroups; otherwise may be NULL.
 * Regimes: small M streams the weight (64 < M runs as consecutive 64-row
 * launches on the stream, all sharing ws); M >= 512, and 64 < M < 512 where
 * a timing model puts the repeated weight stream above the tiled kernel's K
 * sweep (about 4 + 1.6 * K/128 us per round of 256 tiles against
 * ceil(M/64) * (2 + 0.38 * N*K/1e6) us), run the LDS-tiled kernel (256x256
 * tiles), which needs no workspace; bs_workspace_bytes returns 0 exactly
 * when the tiled kernel takes the call.
 * Needs M >= 1, N % 128 == 0, K % 128 == 0, K < 2^24, lda < 2^25,
 * 0 <= as_stride_m < 2^22, as_stride_g >= 0 (and, in the tiled regime,
 * lda < 2^24 and (N/128)*(K/128) < 2^30); a, c and w_pre 16-byte aligned,
 * the scales 4-byte aligned. */
BS_API int bsgemm_fp8_block(const void* a, int64_t lda, const float* a_scale, int64_t as_stride_m,
                            int64_t as_stride_g, const bs_wdesc* wd, const void* w_pre,
                            const float* w_scale, void* c, int64_t ldc, int M, int N, int K,
                            void* ws, size_t ws_bytes, bs_stream_t stream);

/* MXFP4 W4A8 GEMM (radiance_mxfp4.py page: W4A8 with per-token fp8
 * activations; _exact_ref):
 *   C[m,n] = bf16( a_scale[m] * sum_k A[m,k] * e2m1(W[n,k]) * 2^(E[n,k/32]-127) )
 * a: e4m3 [M, K] (lda bytes, multiple of 16); a_scale: fp32 [M];
 * w_pre: pre-laid-out by bs_prelayout_mxfp4 (desc wd); c: bf16 [M, N] (ldc
 * elements, multiple of 4).  Needs M >= 1, N % 16 == 0, K % 128 == 0.
 * Small M (<= 64) streams the weight (bandwidth-bound); large M runs the
 * LDS-tiled scaled-MFMA kernel (compute-bound; a grid whose large tiles end
 * in a partial round runs its last columns as small tiles, and a small-tile
 * grid that ends in a partial round runs its last columns as a separate
 * split launch; every launch is on the given stream, in order).  Whenever either
 * splits K across workgroups (small grids, column strips) the call needs ws
 * of bs_workspace_bytes(BS_OP_W4A8_MXFP4, M, N, K) bytes (256-byte aligned,
 * zeroed once); when that is 0, ws may be NULL.
 * Needs M * lda < 2^32, lda < 2^25 and N * K / 2 < 2^32 (32-bit activation
 * and weight offsets). */
BS_API int bsgemm_w4a8_mxfp4(const void* a, int64_t lda, const float* a_scale, const bs_wdesc* wd,
                             const void* w_pre, void* c, int64_t ldc, int M, int N, int K, void* ws,
                             size_t ws_bytes, bs_stream_t stream);

/* The same GEMM on an activation in the activation-tiled order written by
 * add_rms_quant_fp8_tiled (radiance_mxfp4.py page, the A_TILED_MIN_M comment:
 * at large M the producer emits fragment-tiled activations and the consumer
 * takes them without re-laying them out).  The order is that of gfx950's
 * 32x32x64 MFMA operand with 8-bit data, rows in blocks of 32: a (32-row
 * block rb, 128-K step ks) is the 4 KiB at byte ((rb*K/128 + ks)*4096); in
 * its half h (2 KiB at +2048h), lane l's 32 bytes (at +32l) hold row
 * 32rb + l%32, K = 128ks + 64h + 16(l/32) .. +15, then 128ks + 64h + 32 +
 * 16(l/32) .. +15.  a_tiled holds ceil(M/32)*32*K bytes; the codes of the pad
 * rows are never used.  Prefill regime only: M > 64 (smaller M is the decode
 * kernel's row-major input).  Other arguments, the workspace and the result
 * as bsgemm_w4a8_mxfp4; needs ceil(M/32)*32*K < 2^32. */
BS_API int bsgemm_w4a8_mxfp4_atiled(const void* a_tiled, const float* a_scale, const bs_wdesc* wd,
                                    const void* w_pre, void* c, int64_t ldc, int M, int N, int K, void* ws,
                                    size_t ws_bytes, bs_stream_t stream);

/* Skinny bf16 NT GEMM (radiance_gemm.py page, gemm_bf16_nt_m64):
 *   C[m,n] = bf16( sum_k x[m,k] * w[n,k] ), fp32 accumulation.
 * x: bf16 [M, K]; w: bf16 [N, K]; c: bf16 [M, N]; all contiguous row-major,
 * 16-byte aligned.  1 <= M <= 64, N % 16 == 0, K >= 32, K % 32 == 0 (K past
 * the last multiple of 128 runs as a partial chunk).  Up to 32 rows with
 * K <= 2048, one workgroup per output column and group of 8 rows walks all
 * of K and no workspace is used; otherwise K is split across workgroups and
 * ws must hold
 * bs_workspace_bytes(BS_OP_BF16_SKINNY, ...) (0 in the first case). */
BS_API int gemm_bf16_skinny(const void* x, const void* w, void* c, int M, int N, int K, void* ws,
                            size_t ws_bytes, bs_stream_t stream);

/* The skinny GEMM for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and result as gemm_bf16_skinny, without a workspace.  Its split-K
 * scratch (counters and partials) is a static device array of
 * BS_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends; the call itself allocates and frees nothing.
 *   - A shape whose split-K scratch, bs_workspace_bytes(BS_OP_BF16_SKINNY,
 *     M, N, K), exceeds BS_NOALLOC_SCRATCH_BYTES returns BS_ERR_SCRATCH and
 *     launches nothing (e.g. at M = 64: N <= 1600 for K = 5120, N <= 4032 for
 *     K = 2048).
 *   - The stream must belong to the current device (else BS_ERR_DEVICE).
 *   - The first call on a device looks up the array's address on that device
 *     and clears its counters with a kernel on the stream; make it outside
 *     graph capture.  After that every call leaves the counters zeroed.
 *   - All calls on one GPU share that GPU's array: calls ordered on one stream
 *     are safe, calls that may overlap in time on one GPU (several streams,
 *     several host threads) race and give undefined results. */
#define BS_NOALLOC_SCRATCH_BYTES (4u << 20)
BS_API int gemm_bf16_skinny_noalloc(const void* x, const void* w, void* c, int M, int N, int K,
                                    bs_stream_t stream);

/* ----------------------------------------------------------- producers */

/* Fused residual add + Gemma RMSNorm + per-token e4m3 quant (radiance_arnq.py
 * page, ar_add_rms_quant without the all-reduce; the quant is the
 * radiance_mxfp4.py page's per-token quant):
 *   r = bf16(y + residual)                    -> residual_out (bf16 [M, K])
 *   h = r / sqrt(mean_k r^2 + eps) * (1 + gamma)
 *   scale[m] = max(max_k |h| / 448, 1/(448*512))  (fp32)
 *   q = e4m3(clamp(h / scale, +-448))         (round to nearest even)
 * y, residual, residual_out: bf16 [M, K]; gamma: bf16 [K]; q: e4m3 [M, K];
 * scale: fp32 [M].  residual_out may equal residual (in place); no other
 * overlap.  K % 8 == 0, 8 <= K <= 32768; pointers 16-byte aligned. */
BS_API int add_rms_quant_fp8(const void* y, const void* residual, const void* gamma, float eps,
                             void* q, float* scale, void* residual_out, int M, int K,
                             bs_stream_t stream);

/* The same producer writing the codes in the activation-tiled order that
 * bsgemm_w4a8_mxfp4_atiled reads (see there); residual_out and scale as
 * above.  q_tiled holds ceil(M/32)*32*K bytes, 16-byte aligned; the pad rows
 * of the last 32-row block are not written.  K % 128 == 0, 128 <= K <= 32768. */
BS_API int add_rms_quant_fp8_tiled(const void* y, const void* residual, const void* gamma, float eps,
                                   void* q_tiled, float* scale, void* residual_out, int M, int K,
                                   bs_stream_t stream);

/* The same producer for the block-FP8 consumer: one scale per token per
 * 128-wide K group (the block-FP8 activation format of the radiance_kernels.py
 * page, block_scaled_mm with per-token-per-128 activation scales) instead of
 * one per token:
 *   r, h as in add_rms_quant_fp8
 *   scale[m, g] = max(max_{k in group g} |h| / 448, 1/(448*512))  (fp32)
 *   q[m, k] = e4m3(clamp(h / scale[m, k/128], +-448))
 * scale: fp32 [M, K/128] row-major.  K % 128 == 0, 128 <= K <= 32768; other
 * arguments, aliasing and alignment as add_rms_quant_fp8. */
BS_API int add_rms_quant_fp8_group128(const void* y, const void* residual, const void* gamma, float eps,
                                      void* q, float* scale, void* residual_out, int M, int K,
                                      bs_stream_t stream);

/* SiLU(gate) * up + per-token e4m3 quant (radiance_arnq.py page, the
 * silu_mul_quant op that replaces the MLP's SiluAndMul ahead of the down
 * projection; the quant is the per-token rule above):
 *   h = g / (1 + exp(-g)) * u,   g = gu[m, k], u = gu[m, N + k]
 *   scale[m] = max(max_k |h| / 448, 1/(448*512))  (fp32)
 *   q = e4m3(clamp(h / scale, +-448))
 * gu: bf16 [M, 2N] contiguous (gate half first); q: e4m3 [M, N]; scale: fp32
 * [M].  h is held in fp32 from the hardware exp2 and reciprocal and the codes
 * use h * (1/scale): h is within a few fp32 ulps of the correctly rounded
 * value, so a code may differ by one step where h/scale lies that close to a
 * rounding midpoint.  N % 8 == 0, 8 <= N <= 32768; gu 16-byte aligned, q
 * 8-byte aligned.  No overlap between gu and the outputs. */
BS_API int silu_mul_quant_fp8(const void* gu, void* q, float* scale, int M, int N, bs_stream_t stream);

/* Per-token e4m3 quant of bf16 rows (radiance_mxfp4.py page, _traced_quant):
 * scale[m] = max(max_k |x| / 448, 1/(448*512)); q = e4m3(clamp(x/scale)).
 * x: bf16 [M, K]; q: e4m3 [M, K]; scale: fp32 [M].  K % 8 == 0, K <= 32768. */
BS_API int quant_fp8_per_token(const void* x, void* q, float* scale, int M, int K, bs_stream_t stream);

/* The same rule per 128-wide K group of each row: the block-FP8 activation
 * format (one scale per token per 128 K).  scale: fp32 [M, K/128] row-major.
 * K % 128 == 0. */
BS_API int quant_fp8_group128(const void* x, void* q, float* scale, int M, int K, bs_stream_t stream);

/* The same rule per 128x128 block of a weight: the block-FP8 weight format.
 * w: bf16 [N, K]; q: e4m3 [N, K]; scale: fp32 [N/128, K/128].
 * N % 128 == 0, K % 128 == 0. */
BS_API int quant_fp8_block128(const void* w, void* q, float* scale, int N, int K, bs_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BSGEMM_H */
