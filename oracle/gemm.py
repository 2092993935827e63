"""The three GEMM definitions, C[M,N] (bf16) = dequant(A) . dequant(W)^T.

Test infrastructure (see the package docstring); never used by the product path.

Each function returns (c_bits, c_exact, abs_sum):
  c_exact  the fp64 value of the definition (decode exactly, apply the scales,
           accumulate in fp64);
  c_bits   c_exact rounded once to bf16 (round to nearest even);
  abs_sum  sum_k |a_k * w_k| over the dequantized operands, the quantity the
           parity tolerance is proportional to.
A fp64 matrix product (numpy.matmul) is used as a library step.
"""
import numpy as np

from .codecs import decode_e4m3, decode_e2m1, decode_e8m0, decode_bf16, unpack_fp4, round_to_bf16

GROUP = 128     # block-FP8 scale group along K and along N (radiance_kernels.py page)
MX_BLOCK = 32   # one e8m0 scale per 32 weights along K (radiance_mxfp4.py page)


def fp8_block_gemm(a_codes, a_scale, w_codes, w_scale):
    """Block-FP8 W8A8 GEMM (radiance_kernels.py page, ``block_scaled_mm``: the
    per-128-block scaled e4m3 GEMM; weight guard in ``install_load_hook``).

    a_codes  uint8 e4m3 [M, K]          a_scale fp32 [M, K/128]  (one per token per K group)
    w_codes  uint8 e4m3 [N, K]          w_scale fp32 [N/128, K/128] (one per 128x128 block)

    C[m,n] = sum_g a_scale[m,g] * w_scale[n//128, g] * sum_{k in g} A[m,k] W[n,k].
    The scales multiply (the page calls the weight scale a "deepseek-style"
    scale even though the attribute is named ``weight_scale_inv``).  Each
    inner group sum is exact in fp64 (e4m3 products are multiples of 2**-18
    below 2**18 and 128 of them need at most 43 bits).
    """
    a_codes = np.asarray(a_codes, np.uint8)
    w_codes = np.asarray(w_codes, np.uint8)
    M, K = a_codes.shape
    N, K2 = w_codes.shape
    assert K == K2 and K % GROUP == 0 and N % GROUP == 0
    G = K // GROUP
    a_scale = np.asarray(a_scale, np.float32).astype(np.float64).reshape(M, G)
    w_scale = np.asarray(w_scale, np.float32).astype(np.float64).reshape(N // GROUP, G)
    A = decode_e4m3(a_codes)
    W = decode_e4m3(w_codes)
    n_block = np.arange(N) // GROUP
    c = np.zeros((M, N))
    abs_sum = np.zeros((M, N))
    for g in range(G):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        part = A[:, ks] @ W[:, ks].T
        abs_part = np.abs(A[:, ks]) @ np.abs(W[:, ks]).T
        sc = a_scale[:, g][:, None] * w_scale[n_block, g][None, :]
        c += sc * part
        abs_sum += np.abs(sc) * abs_part
    return round_to_bf16(c), c, abs_sum


def dequant_mxfp4(w_packed, w_e8m0):
    """[N, K/2] packed e2m1 + [N, K/32] e8m0 -> fp64 [N, K]: code value times
    2**(e-127), the scale repeated along its 32 weights (radiance_mxfp4.py
    page, ``_exact_ref``)."""
    codes = unpack_fp4(w_packed)
    N, K = codes.shape
    scale = decode_e8m0(np.asarray(w_e8m0, np.uint8)).reshape(N, K // MX_BLOCK)
    return decode_e2m1(codes) * np.repeat(scale, MX_BLOCK, axis=1)


def w4a8_mxfp4_gemm(a_codes, a_scale, w_packed, w_e8m0):
    """MXFP4 W4A8 GEMM (radiance_mxfp4.py page, ``_exact_ref`` and the
    ``REFLINEAR`` dequantised linear): activations are per-token e4m3 with an
    fp32 scale per row, weights e2m1 with one e8m0 scale per 32 along K.

    a_codes uint8 e4m3 [M, K]; a_scale fp32 [M]; w_packed uint8 [N, K/2]
    (low nibble = even k); w_e8m0 uint8 [N, K/32].

    C[m,n] = a_scale[m] * sum_k A[m,k] * e2m1(W[n,k]) * 2**(E[n,k//32]-127).
    """
    a_codes = np.asarray(a_codes, np.uint8)
    M, K = a_codes.shape
    A = decode_e4m3(a_codes)
    W = dequant_mxfp4(w_packed, w_e8m0)
    assert W.shape[1] == K
    s = np.asarray(a_scale, np.float32).astype(np.float64).reshape(M, 1)
    c = s * (A @ W.T)
    abs_sum = np.abs(s) * (np.abs(A) @ np.abs(W).T)
    return round_to_bf16(c), c, abs_sum


def bf16_gemm(x_bits, w_bits):
    """Skinny bf16 NT GEMM C = x . W^T with exact products and fp64 sums
    (radiance_gemm.py page: ``gemm_bf16_nt_m64`` computes C[M,N] = x[M,K] @ W[N,K]^T)."""
    X = decode_bf16(x_bits)
    W = decode_bf16(w_bits)
    c = X @ W.T
    abs_sum = np.abs(X) @ np.abs(W).T
    return round_to_bf16(c), c, abs_sum


# ------------------------------------------------ single-element forms (sampled parity)
def fp8_block_gemm_at(a_codes, a_scale, w_codes, w_scale, rows, cols):
    """C at the listed (row, col) pairs only; same definition as fp8_block_gemm."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = decode_e4m3(np.asarray(a_codes, np.uint8)[rows])          # [S, K]
    W = decode_e4m3(np.asarray(w_codes, np.uint8)[cols])          # [S, K]
    S, K = A.shape
    G = K // GROUP
    asc = np.asarray(a_scale, np.float32).astype(np.float64)[rows].reshape(S, G)
    wsc = np.asarray(w_scale, np.float32).astype(np.float64)[cols // GROUP].reshape(S, G)
    prod = (A * W).reshape(S, G, GROUP)
    c = np.sum(asc * wsc * prod.sum(axis=2), axis=1)
    abs_sum = np.sum(np.abs(asc * wsc) * np.abs(prod).sum(axis=2), axis=1)
    return round_to_bf16(c), c, abs_sum


def w4a8_mxfp4_gemm_at(a_codes, a_scale, w_packed, w_e8m0, rows, cols):
    """C at the listed (row, col) pairs only; same definition as w4a8_mxfp4_gemm."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = decode_e4m3(np.asarray(a_codes, np.uint8)[rows])
    W = dequant_mxfp4(np.asarray(w_packed, np.uint8)[cols], np.asarray(w_e8m0, np.uint8)[cols])
    s = np.asarray(a_scale, np.float32).astype(np.float64)[rows]
    prod = A * W
    c = s * prod.sum(axis=1)
    abs_sum = np.abs(s) * np.abs(prod).sum(axis=1)
    return round_to_bf16(c), c, abs_sum
