"""Seeded random shapes for every GEMM path, full oracle comparison.

The shapes are drawn across the regime boundaries of each entry point --
block-FP8 below and above the tiled-kernel threshold (M = 512), W4A8 below
and above M = 64 (decode / tiled), the skinny GEMM over its whole M range --
with ragged M, N at and between tile edges, and K from one 128-wide step up,
so that split and unsplit launches, row tails and column tails all occur.
Sizes are bounded so the fp64 oracle finishes each case in about a second.
A second set draws larger shapes per regime (wide N, long K, 64-row chunks
with a remainder, the tiled kernels) and compares 400+ sampled outputs per
shape with the oracle evaluated at just those elements."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from oracle import gemm, checks
from tests.gpu_util import dev_u8, dev_f32, dev_bf16, host_bits16, fp8_block_inputs, w4a8_inputs
from block_scaled_precision_04_amd import synth

pytestmark = pytest.mark.gpu


def _shapes(seed, n, m_lo, m_hi, n_step, n_hi, k_hi):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(g.integers(m_lo, m_hi + 1))
        N = int(g.integers(1, n_hi // n_step + 1)) * n_step
        K = int(g.integers(1, k_hi // 128 + 1)) * 128
        out.append((M, N, K))
    return out


FP8_SHAPES = _shapes(41, 5, 1, 500, 128, 1280, 2560) + _shapes(42, 4, 512, 900, 128, 1152, 1536)
W4_SHAPES = _shapes(43, 5, 1, 64, 16, 1600, 3072) + _shapes(44, 4, 65, 700, 16, 1200, 1536)
SKINNY_SHAPES = _shapes(45, 6, 1, 64, 16, 512, 4096)


@pytest.mark.parametrize("M,N,K", FP8_SHAPES)
def test_fp8_block_random_shape(M, N, K):
    aq, asc, wq, wsc = fp8_block_inputs(10, M * 7 + N + K, M, N, K, outliers=True)
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    ws = bs.alloc_workspace(bs.BS_OP_FP8_BLOCK, M, N, K)
    c = bs.bsgemm_fp8_block(dev_u8(aq), dev_f32(asc), desc, pre, dev_f32(wsc), ws=ws)
    torch.cuda.synchronize()
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(host_bits16(c), ce, asum, f"fp8 block random M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_w4a8_random_shape(M, N, K):
    aq, asc, wp, e = w4a8_inputs(10, M * 7 + N + K, M, N, K)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    ws = bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, N, K)
    c = bs.bsgemm_w4a8_mxfp4(dev_u8(aq), dev_f32(asc), desc, pre, ws=ws)
    torch.cuda.synchronize()
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(c), ce, asum, f"w4a8 random M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_skinny_random_shape(M, N, K):
    g = synth.rng(M * 7 + N + K)
    x = synth.bf16_normal(g, (M, K), 1.0)
    w = synth.bf16_normal(g, (N, K), 0.02)
    ws = bs.alloc_workspace(bs.BS_OP_BF16_SKINNY, M, N, K)
    c = bs.gemm_bf16_skinny(dev_bf16(x), dev_bf16(w), ws=ws)
    torch.cuda.synchronize()
    _, ce, asum = gemm.bf16_gemm(x, w)
    checks.assert_gemm_close(host_bits16(c), ce, asum, f"skinny random M={M} N={N} K={K}")


# ---- larger seeded shapes across the decode / tiled regimes, sampled oracle.
# Regimes: general, wide N (>= 512 16-column tiles), long K (>= 96 K steps);
# M drawn from the row-block classes (1..16, 17..32 / 33..64, 65..511 as
# 64-row launches with a remainder chunk, >= 512 tiled for block-FP8).
def _regime_shapes(seed, n, fp8):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        regime = i % 3
        lo, hi = [(1, 17), (17, 65), (65, 512), (512, 700) if fp8 else (65, 600)][i % 4]
        M = int(g.integers(lo, hi))
        step = 128 if fp8 else 16
        if regime == 1:
            N = int(g.integers(8192 // step, 9216 // step)) * step
            K = int(g.integers(1, 17)) * 128
        elif regime == 2:
            N = int(g.integers(1, 1025 // step + 1)) * step
            K = int(g.integers(96, 137)) * 128
        else:
            N = int(g.integers(1, 5121 // step + 1)) * step
            K = int(g.integers(1, 41)) * 128
        out.append((M, N, K))
    return out


def _pairs(M, N, seed):
    g = np.random.default_rng(seed)
    r = np.concatenate([g.integers(0, M, 400), [0, M - 1, M - 1, 0, min(M - 1, 64), min(M - 1, 63)]])
    c = np.concatenate([g.integers(0, N, 400), [0, N - 1, 0, N - 1, min(N - 1, 16), min(N - 1, 127)]])
    return r, c


@pytest.mark.parametrize("M,N,K", _regime_shapes(51, 12, fp8=True))
def test_fp8_block_regime_shape_sampled(M, N, K):
    aq, asc, wq, wsc = fp8_block_inputs(15, M + N + K, M, N, K, outliers=True)
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    ws = bs.alloc_workspace(bs.BS_OP_FP8_BLOCK, M, N, K)
    c = host_bits16(bs.bsgemm_fp8_block(dev_u8(aq), dev_f32(asc), desc, pre, dev_f32(wsc), ws=ws))
    r, cc = _pairs(M, N, M + K)
    _, ce, asum = gemm.fp8_block_gemm_at(aq, asc, wq, wsc, r, cc)
    checks.assert_gemm_close(c[r, cc], ce, asum, f"fp8 block regime M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", _regime_shapes(52, 12, fp8=False))
def test_w4a8_regime_shape_sampled(M, N, K):
    aq, asc, wp, e = w4a8_inputs(16, M + N + K, M, N, K)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    ws = bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, N, K)
    c = host_bits16(bs.bsgemm_w4a8_mxfp4(dev_u8(aq), dev_f32(asc), desc, pre, ws=ws))
    r, cc = _pairs(M, N, M + K)
    _, ce, asum = gemm.w4a8_mxfp4_gemm_at(aq, asc, wp, e, r, cc)
    checks.assert_gemm_close(c[r, cc], ce, asum, f"w4a8 regime M={M} N={N} K={K}")
