"""The fused producers: residual add -> Gemma RMSNorm -> per-token e4m3 quant,
and SiLU(gate) * up -> per-token e4m3 quant.

Test infrastructure (see the package docstring); never used by the product path.

Source: radiance_arnq.py page (module docstring and ``ar_add_rms_quant``): each
row-parallel output is finished by one kernel that adds the residual, applies
the Gemma RMSNorm of the next layer's input norm and quantizes per token to
e4m3, returning (q [M,K] e4m3, scale [M] fp32, residual_out [M,K]).  The norm
is x * rsqrt(mean(x^2) + eps) * (1 + w) (Gemma's offset weight).  The quant
step is the radiance_mxfp4.py page's per-token quant (see quant.py).

Steps, in the pages' order, with the readings this oracle takes:
  1. r = bf16(y + residual): the exact sum rounded once to bf16 (round to
     nearest even); r is the residual-stream value both consumers see and is
     returned bit for bit.
  2. ms = mean_k r[k]^2, in fp64 over the bf16-rounded r.
  3. inv = 1 / sqrt(ms + eps).
  4. h = r * inv * (1 + w), fp64, w decoded from bf16.  No intermediate
     rounding of h to bf16 (the fused op emits no bf16 hidden tensor).
  5. the quant takes h as fp32, as the page's traced quant takes its input:
     h32 = fp32(h); amax = max_k |h32|; scale = fp32(max(amax/448, 1/(448*512)))
     (one rounding of the exact quotient).
  6. q = e4m3(clamp(h32 / scale, +-448)), the division in fp32 as on the
     page's traced quant, rounded to nearest even.
A row of zeros gives h = 0, scale = 1/(448*512) and q = 0.  NaN/Inf inputs
propagate (they are never generated).
"""
import numpy as np

from .codecs import decode_bf16, round_to_bf16
from .quant import scale_from_amax, quant_with_scale


def _add_rms(y_bits, res_bits, w_bits, eps):
    """Steps 1-4: (residual_out bf16 bits, h fp64)."""
    y = decode_bf16(y_bits)
    res = decode_bf16(res_bits)
    w = decode_bf16(w_bits)
    r_bits = round_to_bf16(y + res)                               # step 1
    r = decode_bf16(r_bits)
    ms = np.mean(r * r, axis=1, keepdims=True)                    # step 2
    inv = 1.0 / np.sqrt(ms + eps)                                 # step 3
    h = r * inv * (1.0 + w)[None, :]                              # step 4
    return r_bits, h


def add_rms_quant(y_bits, res_bits, w_bits, eps=1e-6, return_h=False):
    """y, residual bf16 [M, K]; w bf16 [K] -> (q uint8 [M,K], scale fp32 [M],
    residual_out bf16 [M,K]) and, on request, h fp64 [M,K]."""
    r_bits, h = _add_rms(y_bits, res_bits, w_bits, eps)
    h32 = h.astype(np.float32)
    s = scale_from_amax(np.abs(h32).astype(np.float64).max(axis=1))   # step 5
    q = quant_with_scale(h32, s[:, None])                         # step 6
    if return_h:
        return q, s, r_bits, h
    return q, s, r_bits


def add_rms_quant_group128(y_bits, res_bits, w_bits, eps=1e-6, return_h=False):
    """The norm producer for the block-FP8 consumer: steps 1-4 as above, then
    the same quant rule per 128-wide group of each row instead of per row --
    the activation format of the block-FP8 GEMM (radiance_kernels.py page:
    one scale per token per 128 K, the ``_ps_cfg`` comment and
    ``block_scaled_mm``).
      5'. h32 = fp32(h); for each group g of columns 128g .. 128g+127:
          scale[m, g] = fp32(max(amax_g/448, 1/(448*512)));
      6'. q = e4m3(clamp(h32 / scale[m, g], +-448)).
    Returns (q uint8 [M,K], scale fp32 [M, K/128], residual_out bf16 [M,K]).
    """
    r_bits, h = _add_rms(y_bits, res_bits, w_bits, eps)
    M, K = h.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    hg = h.astype(np.float32).reshape(M, K // 128, 128)
    s = scale_from_amax(np.abs(hg).astype(np.float64).max(axis=2))    # step 5'
    q = quant_with_scale(hg, s[:, :, None]).reshape(M, K)             # step 6'
    if return_h:
        return q, s, r_bits, h
    return q, s, r_bits


def silu_mul_quant(gu_bits, return_h=False):
    """The activation producer: SiLU(gate) * up, then the per-token e4m3 quant.

    Source: radiance_arnq.py page, the ``silu_mul_quant`` custom op and the
    ``_SiluMulQuant`` module that replaces the MLP's SiluAndMul ahead of the
    down projection: input gu bf16 [M, 2N], outputs (q e4m3 [M, N], scale fp32
    [M]) under the same per-token quant contract as the norm producer.

    Steps, with the readings this oracle takes:
      1. gate = gu[:, :N], up = gu[:, N:] (the first half is the activation's
         input, as in the SiluAndMul convention the op replaces).
      2. h = gate / (1 + exp(-gate)) * up in fp64 (SiLU(x) = x * sigmoid(x)),
         from the bf16-decoded inputs.  No rounding of h to bf16: the fused
         op emits no bf16 hidden tensor.
      3. h32 = fp32(h), then the per-token quant of quant.py on h32:
         scale = fp32(max(amax/448, 1/(448*512))), q = e4m3(clamp(h32/scale)).
    A gate of 0 gives h = 0; a row of zeros gives scale 1/(448*512), q = 0.
    """
    gu = decode_bf16(gu_bits)
    M, N2 = gu.shape
    if N2 % 2:
        raise ValueError("gu must have an even number of columns")
    N = N2 // 2
    gate, up = gu[:, :N], gu[:, N:]                               # step 1
    with np.errstate(over="ignore"):
        h = gate / (1.0 + np.exp(-gate)) * up                     # step 2
    h32 = h.astype(np.float32)
    s = scale_from_amax(np.abs(h32).astype(np.float64).max(axis=1))   # step 3
    q = quant_with_scale(h32, s[:, None])
    if return_h:
        return q, s, h
    return q, s
