"""GPU parity of the producers (add_rms_quant_fp8 and the e4m3 quantizers)
against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from block_scaled_precision_04_amd import synth
from oracle import producer, quant, checks
from tests.gpu_util import dev_bf16, host_bits16, host_u8

pytestmark = pytest.mark.gpu


def _run_producer(y, r, w, eps=1e-6, inplace=False):
    yd, rd, wd = dev_bf16(y), dev_bf16(r), dev_bf16(w)
    ro = rd if inplace else None
    q, s, ro = bs.add_rms_quant_fp8(yd, rd, wd, eps, residual_out=ro)
    torch.cuda.synchronize()
    return host_u8(q), s.cpu().numpy(), host_bits16(ro)


@pytest.mark.parametrize("case,M", [(0, 8), (1, 4096)])
def test_producer_fused_chain_sizes(case, M):
    K = 5120
    y, r, w = synth.producer_raw(case, M, K)
    qg, sg, rg = _run_producer(y, r, w)
    qo, so, ro = producer.add_rms_quant(y, r, w, 1e-6)
    rep = checks.assert_producer_close(qg, sg, rg, qo, so, ro, f"producer M={M}")
    print(rep)


@pytest.mark.parametrize("M,K", [(1, 8), (3, 2056), (5, 1000), (2, 32768), (7, 640)])
def test_producer_ragged_shapes(M, K):
    g = synth.rng(700 + K)
    y = synth.bf16_normal(g, (M, K), 1.0)
    r = synth.bf16_normal(g, (M, K), 1.0)
    w = synth.bf16_normal(g, (K,), 0.1)
    qg, sg, rg = _run_producer(y, r, w)
    qo, so, ro = producer.add_rms_quant(y, r, w, 1e-6)
    checks.assert_producer_close(qg, sg, rg, qo, so, ro, f"producer M={M} K={K}")


def test_producer_special_rows_and_inplace():
    K = 1024
    y = np.zeros((4, K), np.uint16)
    r = np.zeros((4, K), np.uint16)
    y[1] = 0x3F40                      # constant 0.75
    y[2, 17] = 0xC040                  # one-hot -3
    g = synth.rng(5)
    y[3] = synth.bf16_normal(g, (K,), 1e-4)   # ms << eps
    w = np.zeros(K, np.uint16)
    qg, sg, rg = _run_producer(y, r, w, inplace=True)
    qo, so, ro = producer.add_rms_quant(y, r, w, 1e-6)
    checks.assert_producer_close(qg, sg, rg, qo, so, ro, "special rows")
    assert np.all(qg[0] == 0) and np.float32(sg[0]) == np.float32(1.0 / (448 * 512))
    assert np.all(qg[1] == 0x7E)
    assert qg[2, 17] == 0xFE


def test_quant_per_token():
    g = synth.rng(11)
    x = synth.bf16_normal(g, (64, 5120), 1.0)
    q, s = bs.quant_fp8_per_token(dev_bf16(x))
    qo, so = quant.quant_per_token_bf16(x)
    checks.assert_codes_close(host_u8(q), s.cpu().numpy(), qo, so, "per-token")


def test_quant_group_and_block():
    g = synth.rng(12)
    x = synth.bf16_normal(g, (40, 1024), 1.0)
    q, s = bs.quant_fp8_group128(dev_bf16(x))
    qo, so = quant.quant_group128_bf16(x)
    checks.assert_codes_close(host_u8(q), s.cpu().numpy(), qo, so, "group128")
    w = synth.bf16_normal(g, (384, 640), 0.02, outlier_p=0.01)
    q, s = bs.quant_fp8_block128(dev_bf16(w))
    qo, so = quant.quant_block128_bf16(w)
    checks.assert_codes_close(host_u8(q), s.cpu().numpy(), qo, so, "block128")
