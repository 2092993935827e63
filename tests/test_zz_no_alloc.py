"""The skinny GEMM entry point that allocates nothing (its split-K scratch is
a static per-GPU array) against the workspace entry point, through the C ABI:
bit-identical outputs on two calls in a row, the second with a smaller input,
so the second call runs on scratch the first one left behind."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from block_scaled_precision_04_amd import synth
from oracle import gemm, checks
from tests.gpu_util import dev_bf16, host_bits16

pytestmark = pytest.mark.gpu


def _inputs(seed, M, N, K):
    g = synth.rng(seed)
    return synth.bf16_normal(g, (M, K), 1.0), synth.bf16_normal(g, (N, K), 0.02)


def _both(x, w):
    M, K = x.shape
    N = w.shape[0]
    xd, wd = dev_bf16(x), dev_bf16(w)
    ref = bs.gemm_bf16_skinny(xd, wd, ws=bs.alloc_workspace(bs.BS_OP_BF16_SKINNY, M, N, K))
    out = torch.full((M, N), -3.0, dtype=torch.bfloat16, device="cuda")
    got = bs.gemm_bf16_skinny_noalloc(xd, wd, out=out)
    torch.cuda.synchronize()
    return host_bits16(got), host_bits16(ref)


@pytest.mark.parametrize("first,second", [((64, 256, 5120), (12, 96, 2048)),    # split K both times
                                          ((32, 1600, 5120), (10, 256, 2048)),  # near the scratch limit first
                                          ((16, 96, 5120), (3, 16, 128)),       # then up to 8 rows (no scratch)
                                          ((33, 96, 5216), (9, 48, 2080))])     # K % 128 != 0: partial chunks
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        x, w = _inputs(100 * M + N + K + i, M, N, K)
        got, ref = _both(x, w)
        assert np.array_equal(got, ref), f"call {i}: M={M} N={N} K={K}"
        _, ce, asum = gemm.bf16_gemm(x, w)
        checks.assert_gemm_close(got, ce, asum, f"noalloc call {i} M={M} N={N} K={K}")


def test_noalloc_refuses_shapes_beyond_the_scratch():
    M, N, K = 64, 1616, 5120          # needs 64 KiB + 10 * 101 * 4 KiB > 4 MiB
    assert bs.workspace_bytes(bs.BS_OP_BF16_SKINNY, M, N, K) > (4 << 20)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bs.BsError, match="static scratch"):
        bs.gemm_bf16_skinny_noalloc(x, w)
    # a shape at the limit is accepted
    assert bs.workspace_bytes(bs.BS_OP_BF16_SKINNY, 64, 1600, 5120) <= (4 << 20)
