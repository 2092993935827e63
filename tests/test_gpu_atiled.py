"""The activation-tiled path: the norm producer writing its codes in the
32x32x64 MFMA A-fragment order (rows padded to 32) and the W4A8 prefill
consumer reading that order without re-laying it out (radiance_mxfp4.py
page, the A_TILED_MIN_M comment).

* producer: the tiled buffer, put back in row-major order by the oracle's
  own index map, is bit-identical to the row-major producer's codes and
  within the producer tolerance of the oracle;
* consumer: the oracle tiles row-major codes, and the tiled GEMM on them is
  bit-identical to the row-major GEMM (same MFMAs in the same order) and
  within the GEMM tolerance of the oracle -- through the 256x256 launch, the
  column strips, the split small tiles and ragged M;
* chain: tiled producer -> tiled GEMM against oracle producer -> oracle GEMM."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from block_scaled_precision_04_amd import synth
from oracle import gemm, checks, layout, producer
from tests.gpu_util import (dev_u8, dev_bf16, dev_f32, host_bits16, w4a8_inputs, sample_grid, block_samples,
                            oracle_at)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K", [(65, 128), (100, 384), (333, 5120), (4096, 5120), (70, 8192), (37, 1024)])
def test_tiled_producer_matches_row_major_and_oracle(M, K):
    y, r, w = synth.producer_raw(M % 7, M, K)
    q, s, ro = bs.add_rms_quant_fp8(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
    qt, st, rot = bs.add_rms_quant_fp8_tiled(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
    torch.cuda.synchronize()
    assert qt.numel() == layout.tiled_activation_bytes(M, K)
    back = layout.untile_activation(qt.cpu().numpy(), M, K)
    assert np.array_equal(back, q.cpu().numpy())
    assert torch.equal(s, st) and torch.equal(ro.view(torch.int16), rot.view(torch.int16))
    rows = np.arange(M) if M <= 400 else np.r_[np.arange(64), np.arange(M - 64, M)]
    qo, so, ro_ref = producer.add_rms_quant(y[rows], r[rows], w, 1e-6)
    checks.assert_producer_close(back[rows], st.cpu().numpy()[rows], host_bits16(rot)[rows], qo, so, ro_ref,
                                 f"tiled producer M={M} K={K}")


def _tiled_vs_row_major(M, N, K, seed):
    aq, asc, wp, e = w4a8_inputs(15, seed, M, N, K)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    ws = bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, N, K)
    c_row = bs.bsgemm_w4a8_mxfp4(dev_u8(aq), dev_f32(asc), desc, pre, ws=ws)
    at = dev_u8(layout.tile_activation(aq))
    c_til = bs.bsgemm_w4a8_mxfp4_atiled(at, dev_f32(asc), desc, pre, M, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(c_row.view(torch.int16), c_til.view(torch.int16)), f"M={M} N={N} K={K}"
    return aq, asc, wp, e, host_bits16(c_til)


@pytest.mark.parametrize("M,N,K", [(65, 48, 384), (100, 176, 640), (300, 1280, 1024), (777, 2064, 2048)])
def test_tiled_gemm_full_oracle(M, N, K):
    aq, asc, wp, e, got = _tiled_vs_row_major(M, N, K, M + N)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(got, ce, asum, f"tiled w4a8 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 5120),      # one round of 256x256 tiles
                                   (2048, 13392, 1024),     # large tiles + unsplit small round + split strip
                                   (500, 17456, 2048),      # small tiles, split remainder, ragged M
                                   (4000, 4240, 2048)])     # ragged last row block inside a large tile
def test_tiled_gemm_every_tile_sampled(M, N, K):
    aq, asc, wp, e, got = _tiled_vs_row_major(M, N, K, M + K)
    rows, cols = sample_grid(M, N, 12, 24, seed=M)
    br, bc = block_samples(M, N, 128, seed=N)
    rows, cols = np.r_[rows, br], np.r_[cols, bc]
    ce, asum = oracle_at(gemm.w4a8_mxfp4_gemm_at, rows, cols, aq, asc, wp, e)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"tiled w4a8 sampled M={M} N={N} K={K}")


def test_tiled_chain():
    """add + RMSNorm + quant into the tiled order, then the tiled GEMM, at the
    fused chain's prefill size (M=4096, K=5120, N=17408)."""
    K, N, M = 5120, 17408, 4096
    wp, e = synth.mxfp4_weight_raw(4, 0, N, K)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    y, r, w = synth.producer_raw(1, M, K)
    qt, s, ro = bs.add_rms_quant_fp8_tiled(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
    c = bs.bsgemm_w4a8_mxfp4_atiled(qt, s, desc, pre, M, ws=bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, N, K))
    torch.cuda.synchronize()
    rows, cols = sample_grid(M, N, 16, 32, seed=79)
    br, bc = block_samples(M, N, 128, seed=80)
    rows, cols = np.r_[rows, br], np.r_[cols, bc]
    ur = np.unique(rows)
    qo, so, ro_ref = producer.add_rms_quant(y[ur], r[ur], w, 1e-6)
    back = layout.untile_activation(qt.cpu().numpy(), M, K)
    checks.assert_producer_close(back[ur], s.cpu().numpy()[ur], host_bits16(ro)[ur], qo, so, ro_ref,
                                 "tiled chain producer")
    # GEMM against the oracle's own producer output (rows mapped through ur)
    idx = np.searchsorted(ur, rows)
    ce, asum = oracle_at(gemm.w4a8_mxfp4_gemm_at, idx, cols, qo, so, wp, e)
    checks.assert_gemm_close(host_bits16(c)[rows, cols], ce, asum, "tiled chain GEMM")


def test_tiled_gemm_refuses_decode_sizes():
    aq, asc, wp, e = w4a8_inputs(15, 1, 64, 48, 384)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    with pytest.raises(bs.BsError, match="unsupported shape"):
        bs.bsgemm_w4a8_mxfp4_atiled(dev_u8(layout.tile_activation(aq)), dev_f32(asc), desc, pre, 64)
