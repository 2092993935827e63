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


@pytest.mark.parametrize("M,K", [(1, 8), (3, 2056), (5, 1000), (2, 32768), (7, 640),
                                 # many rows: the 128-thread row workgroups (1..5 chunks per thread)
                                 (2048, 1032), (2050, 8), (2304, 5120)])
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


@pytest.mark.parametrize("M,K", [(64, 5120), (2048, 3080)])
def test_quant_per_token(M, K):
    g = synth.rng(11 + K)
    x = synth.bf16_normal(g, (M, K), 1.0)
    q, s = bs.quant_fp8_per_token(dev_bf16(x))
    qo, so = quant.quant_per_token_bf16(x)
    checks.assert_codes_close(host_u8(q), s.cpu().numpy(), qo, so, f"per-token M={M} K={K}")


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


# ----------------------------------------------------------------- silu_mul_quant
def _run_silu(gu):
    q, s = bs.silu_mul_quant_fp8(dev_bf16(gu))
    torch.cuda.synchronize()
    return host_u8(q), s.cpu().numpy()


@pytest.mark.parametrize("case,M", [(0, 8), (1, 4096)])
def test_silu_mul_quant_down_projection_input(case, M):
    """The down projection's input at its real width N = 17408; at M = 4096
    the oracle takes every 16th row (rows are independent)."""
    N = 17408
    gu = synth.silu_raw(case, M, N)
    qg, sg = _run_silu(gu)
    rows = np.arange(0, M, 16) if M > 64 else np.arange(M)
    qo, so = producer.silu_mul_quant(gu[rows])
    print(checks.assert_codes_close(qg[rows], sg[rows], qo, so, f"silu_mul_quant M={M}"))


@pytest.mark.parametrize("M,N", [(1, 8), (3, 136), (5, 2056), (2, 32768), (300, 1000), (257, 17400), (64, 8200)])
def test_silu_mul_quant_ragged_shapes(M, N):
    g = synth.rng(900 + N)
    gu = synth.bf16_normal(g, (M, 2 * N), 1.5)
    qg, sg = _run_silu(gu)
    qo, so = producer.silu_mul_quant(gu)
    checks.assert_codes_close(qg, sg, qo, so, f"silu_mul_quant M={M} N={N}")


@pytest.mark.parametrize("M", [4, 512])
def test_silu_mul_quant_special_rows(M):
    """Zero rows, saturated gates (+-60), a single live column and tiny rows,
    on both workgroup shapes (few rows / many rows)."""
    N = 1024
    g = synth.rng(31)
    gu = synth.bf16_normal(g, (M, 2 * N), 1.0)
    gu[0] = 0                                       # zero row: minimum scale, zero codes
    gu[1, :N] = 0x4270                              # gate 60: h = 60 * up
    gu[2, :N] = 0xC270                              # gate -60: h vanishes (min scale)
    gu[3, :N] = 0xC270
    gu[3, 17] = 0x4000                              # ... but for one column with gate 2
    gu[3, N:] = 0x3F80                              # up = 1
    qg, sg = _run_silu(gu)
    qo, so = producer.silu_mul_quant(gu)
    checks.assert_codes_close(qg, sg, qo, so, f"silu special rows M={M}")
    assert np.all((qg[0] & 0x7F) == 0) and np.float32(sg[0]) == np.float32(1.0 / (448 * 512))
    assert qg[3, 17] == 0x7E and np.all((np.delete(qg[3], 17) & 0x7F) == 0)


# ----------------------------------------------------------------- group-scale norm producer
@pytest.mark.parametrize("M,K", [(1, 128), (3, 2048), (5, 5120), (2, 32768), (300, 640), (2048, 1152)])
def test_group_producer_shapes(M, K):
    g = synth.rng(800 + K)
    y = synth.bf16_normal(g, (M, K), 1.0)
    r = synth.bf16_normal(g, (M, K), 1.0)
    w = synth.bf16_normal(g, (K,), 0.1)
    y[0, :128] = synth.bf16_normal(g, (128,), 1e-3)        # a quiet first group
    q, s, ro = bs.add_rms_quant_fp8_group128(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
    torch.cuda.synchronize()
    qo, so, roo = producer.add_rms_quant_group128(y, r, w, 1e-6)
    assert s.shape == (M, K // 128)
    checks.assert_producer_close(host_u8(q), s.cpu().numpy(), host_bits16(ro), qo, so, roo,
                                 f"group producer M={M} K={K}")
