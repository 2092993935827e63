"""Per-token e4m3 quantization and the block / group fixture quantizers.

Test infrastructure (see the package docstring); never used by the product path.

The pages' per-token quant (radiance_mxfp4.py page, ``_traced_quant`` and the
``TRACED_QUANT`` comment above it, which says it matches vLLM's dynamic
per-token fp8 quant):
    scale = max(rowamax / 448, 1 / (448 * 512))        fp32 math
    q     = e4m3(clamp(x / scale, -448, 448))          round-to-nearest cast
Readings taken here:
  * the scale is the exact quotient amax/448 rounded once to fp32, then
    clamped below by 1/(448*512) (the page multiplies by a rounded 1/448;
    the two differ by at most one fp32 ulp);
  * the quotient x/scale is an IEEE fp32 division of the fp32 input by the
    fp32 scale, i.e. the integer code decision is taken in fp32 as on the
    page, then clamped and rounded to nearest-even e4m3.

The block-FP8 GEMM's inputs (one scale per token per 128-wide K group for
activations, one per 128x128 block for weights, scale = amax/448) are made by
the same rule applied per group / per block; those two are fixtures that turn
seeded bf16 draws into the GEMM's quantized inputs.
"""
import numpy as np

from .codecs import round_to_e4m3, decode_bf16

FP8_MAX = 448.0
MIN_SCALE = 1.0 / (448.0 * 512.0)


def scale_from_amax(amax):
    """fp32 scale for a group with the given absolute maximum (fp64 in)."""
    s = np.asarray(amax, np.float64) / FP8_MAX
    return np.maximum(s, MIN_SCALE).astype(np.float32)


def quant_with_scale(x32, s32):
    """e4m3 codes of x/s: fp32 division, clamp to +-448, RNE to e4m3."""
    x32 = np.asarray(x32, np.float32)
    s32 = np.asarray(s32, np.float32)
    with np.errstate(over="ignore"):
        v = x32 / s32                                  # IEEE fp32 division
    v = np.clip(v, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return round_to_e4m3(v.astype(np.float64))


def quant_per_token(x32):
    """Per-token (per-row) dynamic quant of fp32 rows [M, K] -> (codes uint8
    [M, K], scale fp32 [M])."""
    x32 = np.asarray(x32, np.float32)
    amax = np.abs(x32).astype(np.float64).max(axis=1)
    s = scale_from_amax(amax)
    return quant_with_scale(x32, s[:, None]), s


def quant_per_token_bf16(x_bits):
    """quant_per_token of bf16 rows (the page converts the input to fp32 first)."""
    return quant_per_token(decode_bf16(x_bits).astype(np.float32))


def quant_group128_bf16(x_bits, group=128):
    """Activation fixture: one scale per row per 128-wide K group.
    bf16 [M, K] -> (codes uint8 [M, K], scale fp32 [M, K/128])."""
    x = decode_bf16(x_bits).astype(np.float32)
    M, K = x.shape
    xg = x.reshape(M, K // group, group)
    s = scale_from_amax(np.abs(xg).astype(np.float64).max(axis=2))       # [M, G]
    q = quant_with_scale(xg, s[:, :, None]).reshape(M, K)
    return q, s


def quant_block128_bf16(w_bits, block=128):
    """Weight fixture: one scale per 128x128 block.
    bf16 [N, K] -> (codes uint8 [N, K], scale fp32 [N/128, K/128])."""
    w = decode_bf16(w_bits).astype(np.float32)
    N, K = w.shape
    wb = w.reshape(N // block, block, K // block, block)
    s = scale_from_amax(np.abs(wb).astype(np.float64).max(axis=(1, 3)))  # [N/128, K/128]
    q = quant_with_scale(wb, s[:, None, :, None]).reshape(N, K)
    return q, s
