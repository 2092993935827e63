"""Seeded random shapes for every GEMM path, full oracle comparison.

The shapes are drawn across the regime boundaries of each entry point --
block-FP8 below and above the tiled-kernel threshold (M = 512), W4A8 below
and above M = 64 (decode / tiled), the skinny GEMM over its whole M range --
with ragged M, N at and between tile edges, and K from one 128-wide step up,
so that split and unsplit launches, row tails and column tails all occur.
Sizes are bounded so the fp64 oracle finishes each case in about a second."""
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
