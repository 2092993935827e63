"""GPU parity of the one-time weight pre-layout: bytes equal to the oracle's
index maps (bit-exact) and exact inverses."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from oracle import layout
from tests.gpu_util import dev_u8, host_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (512, 1024), (5120, 5120)])
def test_fp8_block_prelayout(N, K):
    g = np.random.default_rng(N + K)
    w = g.integers(0, 256, (N, K), dtype=np.uint8)
    pre, desc = bs.prelayout_fp8_block(dev_u8(w))
    assert desc.N == N and desc.K == K and desc.total_bytes == N * K
    assert np.array_equal(host_u8(pre), layout.prelayout_fp8_block(w))
    back = bs.unprelayout_fp8_block(desc, pre)
    assert np.array_equal(host_u8(back), w)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (32, 640), (17408, 5120)])
def test_mxfp4_prelayout(N, K):
    g = np.random.default_rng(N * 3 + K)
    wp = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    e = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    host = host_u8(pre)
    assert np.array_equal(host[:desc.codes_bytes], layout.prelayout_mxfp4_codes(wp))
    sc = host[desc.scales_offset:desc.scales_offset + desc.scales_bytes]
    assert np.array_equal(sc, layout.prelayout_mxfp4_scales(e))
    wp2, e2 = bs.unprelayout_mxfp4(desc, pre)
    assert np.array_equal(host_u8(wp2), wp) and np.array_equal(host_u8(e2), e)
