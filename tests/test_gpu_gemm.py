"""GPU parity of the three GEMMs against the oracle (through the C ABI), at
the workloads' own sizes (full or sampled) and at ragged / edge shapes."""
import numpy as np
import pytest
import torch

import block_scaled_precision_04_amd as bs
from block_scaled_precision_04_amd import synth
from oracle import gemm, checks
from tests.gpu_util import (dev_u8, dev_bf16, dev_f32, host_bits16, fp8_block_inputs, w4a8_inputs,
                            sample_grid, block_samples, oracle_at)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ block-FP8
def _fp8_run(aq, asc, wq, wsc, col_major_scale=False):
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    a_s = dev_f32(asc)
    if col_major_scale:       # same values, stored [K/128, M] and read through strides
        a_s = dev_f32(np.ascontiguousarray(asc.T)).t()
    M, K = aq.shape
    ws = bs.alloc_workspace(bs.BS_OP_FP8_BLOCK, M, desc.N, K)
    c = bs.bsgemm_fp8_block(dev_u8(aq), a_s, desc, pre, dev_f32(wsc), ws=ws)
    c2 = bs.bsgemm_fp8_block(dev_u8(aq), a_s, desc, pre, dev_f32(wsc), ws=ws)   # workspace reused
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    return host_bits16(c)


@pytest.mark.parametrize("case", range(len(synth.WORKLOADS[2][1])))
def test_fp8_block_decode_workload(case):
    M, N, K = synth.WORKLOADS[2][1][case]
    aq, asc, wq, wsc = fp8_block_inputs(2, case, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(got, ce, asum, f"fp8 block M={M} N={N} K={K}")


def test_fp8_block_small_workload():
    M, N, K = synth.WORKLOADS[0][1][0]
    aq, asc, wq, wsc = fp8_block_inputs(0, 0, M, N, K)
    got = _fp8_run(aq, asc, wq, wsc, col_major_scale=True)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(got, ce, asum, "fp8 block small")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 256, 384), (65, 384, 640), (100, 128, 1024),
                                   (64, 1280, 2048), (3, 5120, 17408),
                                   # the 8-wave decode configurations: wide N (>= 512 tiles) and
                                   # long K (>= 96 steps) at 17..32 and 33..64 rows, ragged M
                                   (17, 8192, 384), (50, 8192, 256), (20, 256, 12288), (47, 128, 12288),
                                   # up to 16 rows past 20 K steps: 8 waves of 10 steps (ragged last
                                   # split), and wide N at 12 / 16 rows (10 waves of 4 / 8 waves of 10)
                                   (5, 640, 3200), (12, 8192, 2816), (16, 8192, 2816)])
def test_fp8_block_edges(M, N, K):
    aq, asc, wq, wsc = fp8_block_inputs(9, M + N, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(got, ce, asum, f"fp8 block edge M={M} N={N} K={K}")


# M in 65..511 runs as 64-row launches that share the workspace; the remainder
# chunk can take another configuration than the full chunks (these shapes
# once put its split-K counters inside the full chunks' partials).
@pytest.mark.parametrize("M,N,K", [(408, 8448, 1408), (469, 640, 17280), (138, 768, 16384), (269, 640, 12288),
                                   (401, 1408, 2816)])
def test_fp8_block_row_chunks_sampled(M, N, K):
    aq, asc, wq, wsc = fp8_block_inputs(10, M + K, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc)
    rows, cols = sample_grid(M, N, 24, 40, seed=M)
    _, ce, asum = gemm.fp8_block_gemm_at(aq, asc, wq, wsc, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"fp8 block row chunks M={M} N={N} K={K}")


def test_shared_workspace_across_shapes():
    """One workspace, zeroed once, serves a sequence of calls of every GEMM at
    different shapes (split and unsplit, chunked rows with differing
    configurations); each output equals the same call on a fresh workspace."""
    calls = []
    for (M, N, K) in [(100, 1280, 12288), (8, 1280, 17408), (40, 8192, 256), (21, 640, 17280)]:
        aq, asc, wq, wsc = fp8_block_inputs(13, M + N, M, N, K, outliers=True)
        pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
        args = (dev_u8(aq), dev_f32(asc), desc, pre, dev_f32(wsc))
        calls.append((bs.BS_OP_FP8_BLOCK, (M, N, K), lambda ws, a=args: bs.bsgemm_fp8_block(*a, ws=ws)))
    for (M, N, K) in [(8, 2048, 17408), (256, 1280, 5120), (40, 512, 5120)]:
        aq, asc, wp, e = w4a8_inputs(14, M + N, M, N, K)
        pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
        args = (dev_u8(aq), dev_f32(asc), desc, pre)
        calls.append((bs.BS_OP_W4A8_MXFP4, (M, N, K), lambda ws, a=args: bs.bsgemm_w4a8_mxfp4(*a, ws=ws)))
    for (M, N, K) in [(8, 256, 2048), (64, 96, 5120)]:
        xb, wb = synth.skinny_raw(M, M, N, K)
        args = (dev_bf16(xb), dev_bf16(wb))
        calls.append((bs.BS_OP_BF16_SKINNY, (M, N, K), lambda ws, a=args: bs.gemm_bf16_skinny(*a, ws=ws)))
    need = max(bs.workspace_bytes(op, *shape) for op, shape, _ in calls)
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    refs = []
    for op, shape, fn in calls:
        fresh = bs.alloc_workspace(op, *shape)
        refs.append(fn(fresh).view(torch.int16).clone())
    for rep in range(2):
        for (op, shape, fn), ref in zip(calls, refs):
            got = fn(shared if bs.workspace_bytes(op, *shape) else None)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref), f"pass {rep}: op {op} shape {shape}"


# ------------------------------------------------------------------ MXFP4 W4A8
def _w4_run(aq, asc, wp, e, out=None):
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    M, K = aq.shape
    ws = bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, desc.N, K)
    c = bs.bsgemm_w4a8_mxfp4(dev_u8(aq), dev_f32(asc), desc, pre, out=out, ws=ws)
    if ws is not None:        # split-K: a second call on the same workspace gives the same bits
        c2 = bs.bsgemm_w4a8_mxfp4(dev_u8(aq), dev_f32(asc), desc, pre, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("M,N,K", [(8, 17408, 5120), (1, 16, 128), (33, 48, 384), (64, 176, 640),
                                   (13, 2048, 17408), (65, 48, 384), (129, 176, 640), (200, 1024, 1024),
                                   (256, 1280, 5120), (300, 48, 17408), (5, 48, 12288),
                                   (16, 4096, 5120), (16, 208, 640),    # 16 rows: two tiles per wave
                                   (7, 10240, 1024), (9, 10256, 640),   # 5..15 rows, 640+ tiles: three per workgroup
                                   (1100, 4112, 256)])  # 297 small tiles (> one per CU): two waves of 64 x 128
def test_w4a8_full_oracle(M, N, K):
    aq, asc, wp, e = w4a8_inputs(8, M + N + K, M, N, K)
    got = host_bits16(_w4_run(aq, asc, wp, e))
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(got, ce, asum, f"w4a8 M={M} N={N} K={K}")


@pytest.mark.parametrize("case", range(len(synth.WORKLOADS[3][1])))
def test_w4a8_prefill_workload_sampled(case):
    """Each prefill workload shape: a grid of rows x columns (tile edges,
    first and last) plus one element in every 128x128 cell, so every output
    tile of every launch of the tile plan is checked (M=8192 N=34816: all
    4352 large tiles)."""
    M, N, K = synth.WORKLOADS[3][1][case]
    aq, asc, wp, e = w4a8_inputs(3, case, M, N, K)
    got = host_bits16(_w4_run(aq, asc, wp, e))
    rows, cols = sample_grid(M, N, 20, 40, seed=case)
    br, bc = block_samples(M, N, 128, seed=1000 + case)
    rows, cols = np.r_[rows, br], np.r_[cols, bc]
    ce, asum = oracle_at(gemm.w4a8_mxfp4_gemm_at, rows, cols, aq, asc, wp, e)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"w4a8 prefill M={M} N={N} K={K}")


def test_w4a8_large_tile_launch_full_oracle():
    """Every element of one full round of the 256x256 kernel: M = N = 4096,
    K = 5120 is 16 x 16 = 256 large tiles (one per CU), no column strip, the
    whole K pipeline (40 steps), against the full fp64 oracle."""
    M, N, K = 4096, 4096, 5120
    aq, asc, wp, e = w4a8_inputs(3, 99, M, N, K)
    assert bs.workspace_bytes(bs.BS_OP_W4A8_MXFP4, M, N, K) == 0      # one unsplit launch
    got = host_bits16(_w4_run(aq, asc, wp, e))
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(got, ce, asum, f"w4a8 large tiles full M={M} N={N} K={K}")


def test_w4a8_down_projection_sampled():
    """M=4096 N=5120 K=17408 (the SiLU chain's down projection): large tiles
    over 4096 columns plus an unsplit 256-tile column strip over K = 17408."""
    M, N, K = 4096, 5120, 17408
    aq, asc, wp, e = w4a8_inputs(5, 1, M, N, K)
    got = host_bits16(_w4_run(aq, asc, wp, e))
    rows, cols = sample_grid(M, N, 12, 40, seed=17)
    cols = np.concatenate([cols, [4095, 4096, 4097, 5119]])
    rows = np.concatenate([rows, [0, 1, M - 2, M - 1]])
    _, ce, asum = gemm.w4a8_mxfp4_gemm_at(aq, asc, wp, e, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"w4a8 down projection M={M} N={N} K={K}")


def test_w4a8_fused_chain():
    """The fused chain end to end: GPU producer -> GPU W4A8 GEMM against the
    oracle producer -> oracle GEMM on the same raw draws (the oracle never
    sees a GPU output)."""
    from oracle import producer
    K, N = 5120, 17408
    wp, e = synth.mxfp4_weight_raw(4, 0, N, K)
    pre, desc = bs.prelayout_mxfp4(dev_u8(wp), dev_u8(e))
    for case, M in ((0, 8), (1, 4096)):
        y, r, w = synth.producer_raw(case, M, K)
        q, s, ro = bs.add_rms_quant_fp8(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
        c = bs.bsgemm_w4a8_mxfp4(q, s, desc, pre, ws=bs.alloc_workspace(bs.BS_OP_W4A8_MXFP4, M, N, K))
        torch.cuda.synchronize()
        qo, so, ro_ref = producer.add_rms_quant(y, r, w, 1e-6)
        checks.assert_producer_close(q.cpu().numpy(), s.cpu().numpy(), host_bits16(ro), qo, so, ro_ref,
                                     f"chain producer M={M}")
        ch = host_bits16(c)
        if M <= 8:
            _, ce, asum = gemm.w4a8_mxfp4_gemm(qo, so, wp, e)
            checks.assert_gemm_close(ch, ce, asum, "chain decode")
        else:
            rows, cols = sample_grid(M, N, 16, 32, seed=77)
            br, bc = block_samples(M, N, 128, seed=78)
            rows, cols = np.r_[rows, br], np.r_[cols, bc]
            ce, asum = oracle_at(gemm.w4a8_mxfp4_gemm_at, rows, cols, qo, so, wp, e)
            checks.assert_gemm_close(ch[rows, cols], ce, asum, "chain prefill")


def test_w4a8_no_out_of_bounds_writes_and_ldc():
    M, N, K = 150, 176, 640
    aq, asc, wp, e = w4a8_inputs(8, 1, M, N, K)
    big = torch.full((M + 2, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[1:M + 1, 8:8 + N]
    _w4_run(aq, asc, wp, e, out=view)
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[1:M + 1, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, "w4a8 strided out")


def _guarded(M, N, pad_c=40):
    """A [M, N] view with leading dimension N + pad_c inside a frame of -7.0
    (one row above and below, 8 columns left, pad_c - 8 right)."""
    big = torch.full((M + 2, N + pad_c), -7.0, dtype=torch.bfloat16, device="cuda")
    return big, big[1:M + 1, 8:8 + N]


def _frame_untouched(big, M, N):
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[1:M + 1, 8:8 + N] = False
    return bool(np.all(host[mask] == -7.0))


# decode kernels writing into a strided view inside a guard frame: rows 1..64
# (one and several 16-row blocks, ragged), K unsplit (few steps) and split
# across workgroups (the last workgroup of a tile group writes C), and
# block-FP8 beyond 64 rows (consecutive 64-row launches)
DECODE_FRAME = [(1, 384), (5, 17408), (16, 640), (17, 5120), (33, 384), (47, 17408), (64, 5120), (100, 2048)]


@pytest.mark.parametrize("M,K", DECODE_FRAME)
def test_fp8_block_decode_strided_out(M, K):
    N = 1280
    aq, asc, wq, wsc = fp8_block_inputs(9, 31 * M + K, M, N, K, outliers=True)
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    ws = bs.alloc_workspace(bs.BS_OP_FP8_BLOCK, M, N, K)
    big, view = _guarded(M, N)
    bs.bsgemm_fp8_block(dev_u8(aq), dev_f32(asc), desc, pre, dev_f32(wsc), out=view, ws=ws)
    torch.cuda.synchronize()
    assert _frame_untouched(big, M, N)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, f"fp8 decode strided M={M} K={K}")


@pytest.mark.parametrize("M,K", [mk for mk in DECODE_FRAME if mk[0] <= 64])
def test_w4a8_decode_strided_out(M, K):
    N = 1296
    aq, asc, wp, e = w4a8_inputs(8, 37 * M + K, M, N, K)
    big, view = _guarded(M, N)
    _w4_run(aq, asc, wp, e, out=view)
    assert _frame_untouched(big, M, N)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, f"w4a8 decode strided M={M} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (8, 256, 2048), (17, 96, 5120), (64, 96, 5120), (40, 48, 384)])
def test_skinny_guarded_out(M, N, K):
    """The skinny GEMM takes a dense [M, N] output: written inside a larger
    buffer, nothing before or after it changes (split and unsplit K)."""
    g = synth.rng(7 * M + N + K)
    x = synth.bf16_normal(g, (M, K), 1.0)
    w = synth.bf16_normal(g, (N, K), 0.02)
    pad = 256
    flat = torch.full((M * N + 2 * pad,), -7.0, dtype=torch.bfloat16, device="cuda")
    out = flat[pad:pad + M * N].view(M, N)
    bs.gemm_bf16_skinny(dev_bf16(x), dev_bf16(w), out=out, ws=bs.alloc_workspace(bs.BS_OP_BF16_SKINNY, M, N, K))
    torch.cuda.synchronize()
    host = flat.float().cpu().numpy()
    assert np.all(host[:pad] == -7.0) and np.all(host[pad + M * N:] == -7.0)
    _, ce, asum = gemm.bf16_gemm(x, w)
    checks.assert_gemm_close(host_bits16(out), ce, asum, f"skinny guarded M={M} N={N} K={K}")


def test_w4a8_prefill_out_ldc_not_multiple_of_8():
    """The prefill epilogue stores 16-byte pieces when the output's leading
    dimension is a multiple of 8 elements and 8-byte pieces otherwise: here
    ldc = N + 36 (4 mod 8), first row 16-byte aligned, a guard below and
    beside the view."""
    M, N, K = 150, 176, 640
    aq, asc, wp, e = w4a8_inputs(8, 3, M, N, K)
    big = torch.full((M + 1, N + 36), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[0:M, 8:8 + N]
    assert view.stride(0) % 8 == 4
    _w4_run(aq, asc, wp, e, out=view)
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[0:M, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, "w4a8 ldc 4 mod 8")


@pytest.mark.parametrize("M,N,K", [(4000, 4240, 512),   # 16 x 16 large tiles + a 144-column strip
                                   (2000, 2544, 512)])  # 320 two-wave small tiles, ragged rows and columns
def test_w4a8_fp32_staged_epilogue_ldc_4_mod_8(M, N, K):
    """The tiles that stage fp32 accumulators in LDS (256x256, and 128x128 as
    two waves) store 8-byte pieces; here into a view whose leading dimension
    is 4 mod 8 elements, with a guard below and beside it.  Nothing outside the
    view changes and every element matches the oracle."""
    aq, asc, wp, e = w4a8_inputs(8, 17 + M, M, N, K)
    big = torch.full((M + 1, N + 44), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[0:M, 8:8 + N]    # first row 16-byte aligned, the rows after it 8 mod 16
    assert view.stride(0) % 8 == 4
    _w4_run(aq, asc, wp, e, out=view)
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[0:M, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, f"w4a8 fp32-staged ldc 4 mod 8 M={M} N={N}")


def test_w4a8_large_tiles_and_unsplit_strip_full_oracle():
    """Large tiles and an unsplit column strip of small tiles: M=2000 (last
    256-row tile 208 rows deep, last 128-row tile 80), N=8496 -> 8 x 32 large
    tiles over 8192 columns plus a 304-column strip of 16 x 3 small tiles
    (the last 48 columns wide), K=1024 (too short to split), into a view
    whose leading dimension is 4 mod 8, with a guard; every element against
    the oracle."""
    M, N, K = 2000, 8496, 1024
    aq, asc, wp, e = w4a8_inputs(8, 21, M, N, K)
    assert bs.lib().bs_workspace_bytes(bs.BS_OP_W4A8_MXFP4, M, N, K) == 0
    big = torch.full((M + 1, N + 44), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[0:M, 8:8 + N]
    assert view.stride(0) % 8 == 4
    _w4_run(aq, asc, wp, e, out=view)
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[0:M, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    _, ce, asum = gemm.w4a8_mxfp4_gemm(aq, asc, wp, e)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, "w4a8 large tiles + unsplit strip")


def test_w4a8_large_tiles_strided_out():
    """The large-tile launch and its column strip writing into a strided view:
    M=4000 (last 256-row tile 160 rows deep), N=4240 -> 16 x 16 large tiles
    over 4096 columns plus a 144-column strip of split small tiles.  Nothing
    outside the view changes; sampled values (seams included) match the
    oracle."""
    M, N, K = 4000, 4240, 2048
    aq, asc, wp, e = w4a8_inputs(8, 13, M, N, K)
    big = torch.full((M + 2, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[1:M + 1, 8:8 + N]
    _w4_run(aq, asc, wp, e, out=view)
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[1:M + 1, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    got = host_bits16(view.contiguous())
    rows, cols = sample_grid(M, N, 12, 24, seed=13)
    rr, cc = np.meshgrid(np.array([0, 255, 256, 3839, 3840, M - 1]), np.array([4095, 4096, 4223, 4224, N - 1]),
                         indexing="ij")
    rows = np.r_[rows, rr.reshape(-1)]
    cols = np.r_[cols, cc.reshape(-1)]
    _, ce, asum = gemm.w4a8_mxfp4_gemm_at(aq, asc, wp, e, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, "w4a8 large tiles strided out")


def test_w4a8_two_tile_workgroups_ragged_strided():
    """Large-tile grids of two or more rounds run two tiles per workgroup:
    M=4196 (17 row tiles, the last 100 rows deep), N=8240 (33 column tiles,
    the last 48 wide) is 561 large tiles with no column strip, so workgroups
    0..255 take tiles b and b + 305.  Written into a strided view inside a
    guard frame (whole tiles take the 16-byte store path, ragged ones the
    guarded path): nothing outside the view changes, and one element of
    every 128x128 cell plus the tile seams match the oracle."""
    M, N, K = 4196, 8240, 1024
    assert (M + 255) // 256 * ((N + 255) // 256) == 561
    assert bs.workspace_bytes(bs.BS_OP_W4A8_MXFP4, M, N, K) == 0      # one unsplit launch
    aq, asc, wp, e = w4a8_inputs(8, 29, M, N, K)
    big, view = _guarded(M, N)
    _w4_run(aq, asc, wp, e, out=view)
    assert _frame_untouched(big, M, N)
    got = host_bits16(view.contiguous())
    rows, cols = sample_grid(M, N, 12, 24, seed=29)
    br, bc = block_samples(M, N, 128, seed=30)
    rr, cc = np.meshgrid(np.array([0, 255, 256, 4095, 4096, M - 1]), np.array([0, 8191, 8192, N - 1]),
                         indexing="ij")
    rows = np.r_[rows, br, rr.reshape(-1)]
    cols = np.r_[cols, bc, cc.reshape(-1)]
    ce, asum = oracle_at(gemm.w4a8_mxfp4_gemm_at, rows, cols, aq, asc, wp, e)
    checks.assert_gemm_close(got[rows, cols], ce, asum, "w4a8 two-tile workgroups ragged strided")


def test_determinism():
    M, N, K = 256, 1280, 5120
    aq, asc, wp, e = w4a8_inputs(8, 2, M, N, K)
    a1 = host_bits16(_w4_run(aq, asc, wp, e))
    a2 = host_bits16(_w4_run(aq, asc, wp, e))
    assert np.array_equal(a1, a2)
    aq, asc, wq, wsc = fp8_block_inputs(9, 3, 8, 5120, 5120)
    assert np.array_equal(_fp8_run(aq, asc, wq, wsc), _fp8_run(aq, asc, wq, wsc))


# ------------------------------------------------------------------ skinny bf16
def _skinny_run(x, w):
    M, K = x.shape
    N = w.shape[0]
    ws = bs.alloc_workspace(bs.BS_OP_BF16_SKINNY, M, N, K)
    c = bs.gemm_bf16_skinny(dev_bf16(x), dev_bf16(w), ws=ws)
    c2 = bs.gemm_bf16_skinny(dev_bf16(x), dev_bf16(w), ws=ws)     # workspace reused: counters self-reset
    torch.cuda.synchronize()
    h1, h2 = host_bits16(c), host_bits16(c2)
    assert np.array_equal(h1, h2)
    return h1


@pytest.mark.parametrize("case", range(len(synth.WORKLOADS[1][1])))
def test_skinny_workload(case):
    M, N, K = synth.WORKLOADS[1][1][case]
    x, w = synth.skinny_raw(case, M, N, K)
    got = _skinny_run(x, w)
    _, ce, asum = gemm.bf16_gemm(x, w)
    checks.assert_gemm_close(got, ce, asum, f"skinny M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (17, 32, 384), (33, 48, 640), (64, 16, 128), (5, 1280, 5120),
                                   # K % 32 == 0 but not a multiple of 128: a partial last chunk,
                                   # alone (K = 32, 96) and after whole ones, split and unsplit
                                   (8, 16, 32), (3, 32, 96), (16, 64, 160), (33, 96, 2080), (64, 48, 5024),
                                   (8, 96, 5216),
                                   # up to 32 rows, one workgroup per column and 8 rows up to K = 2048
                                   # (all chunk slots used at 2048, idle ones below; a partial last row
                                   # group); just past either limit, the split form
                                   (8, 64, 2048), (2, 16, 1056), (6, 48, 2080), (8, 32, 8192),
                                   (27, 32, 1024), (32, 16, 2048), (33, 16, 2048), (20, 48, 96)])
def test_skinny_edges(M, N, K):
    g = synth.rng(M * 1000 + N + K)
    x = synth.bf16_normal(g, (M, K), 1.0)
    w = synth.bf16_normal(g, (N, K), 0.02)
    got = _skinny_run(x, w)
    _, ce, asum = gemm.bf16_gemm(x, w)
    checks.assert_gemm_close(got, ce, asum, f"skinny edge M={M} N={N} K={K}")


# ------------------------------------------------------------------ block-FP8, large M (tiled kernel)
FP8_PREFILL_CASES = [0, 1, 2, 4]     # M=2048 at the three (N,K) shapes, M=8192 at N=10240 K=5120


@pytest.mark.parametrize("case", FP8_PREFILL_CASES)
def test_fp8_block_prefill_workload_sampled(case):
    M, N, K = synth.WORKLOADS[6][1][case]
    assert bs.lib().bs_workspace_bytes(bs.BS_OP_FP8_BLOCK, M, N, K) == 0     # the tiled kernel needs none
    aq, asc, wq, wsc = fp8_block_inputs(6, case, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc)
    rows, cols = sample_grid(M, N, 24, 40, seed=100 + case)
    _, ce, asum = gemm.fp8_block_gemm_at(aq, asc, wq, wsc, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"fp8 block prefill M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,colmajor", [(512, 128, 128, False), (600, 384, 640, True), (1000, 1280, 1152, False),
                                            (513, 256, 384, True), (777, 640, 2048, False)])
def test_fp8_block_prefill_edges(M, N, K, colmajor):
    """Tiled kernel at ragged M (row tails inside a 256-row tile), N = 1.5 and
    2.5 tiles (a half tile of idle waves), a single K step, and activation
    scales read through column-major strides; full oracle."""
    aq, asc, wq, wsc = fp8_block_inputs(9, 7 * M + N, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc, col_major_scale=colmajor)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(got, ce, asum, f"fp8 block prefill edge M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,tiled", [(448, 5120, 5120, True), (384, 5120, 5120, True),
                                         (200, 10240, 5120, True), (320, 5120, 5120, False),
                                         (448, 5120, 17408, True), (384, 5120, 17408, False)])
def test_fp8_block_mid_m_routing(M, N, K, tiled):
    """65 <= M < 512: the tiled kernel where its one K sweep per round of
    tiles costs less than ceil(M/64) decode launches, each streaming the whole
    weight (the library's timing model), else the 64-row decode launches; the
    oracle on a grid of the edge rows and columns plus random ones (about two
    per 16-row block and two per 256-column stripe)."""
    wsb = bs.lib().bs_workspace_bytes(bs.BS_OP_FP8_BLOCK, M, N, K)
    assert (wsb == 0) == tiled
    aq, asc, wq, wsc = fp8_block_inputs(12, M + N + K, M, N, K, outliers=True)
    got = _fp8_run(aq, asc, wq, wsc)
    rows, cols = sample_grid(M, N, 2 * -(-M // 16), 2 * N // 256, seed=M + N)
    _, ce, asum = gemm.fp8_block_gemm_at(aq, asc, wq, wsc, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, f"fp8 block mid-M M={M} N={N} K={K}")


def test_fp8_block_prefill_no_out_of_bounds_writes_and_ldc():
    M, N, K = 700, 384, 512
    aq, asc, wq, wsc = fp8_block_inputs(9, 11, M, N, K)
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    big = torch.full((M + 2, N + 40), -7.0, dtype=torch.bfloat16, device="cuda")
    view = big[1:M + 1, 8:8 + N]
    bs.bsgemm_fp8_block(dev_u8(aq), dev_f32(asc), desc, pre, dev_f32(wsc), out=view)
    torch.cuda.synchronize()
    host = big.float().cpu().numpy()
    mask = np.ones(host.shape, bool)
    mask[1:M + 1, 8:8 + N] = False
    assert np.all(host[mask] == -7.0)
    _, ce, asum = gemm.fp8_block_gemm(aq, asc, wq, wsc)
    checks.assert_gemm_close(host_bits16(view.contiguous()), ce, asum, "fp8 prefill strided out")


def test_fp8_block_group_chain():
    """The group-scale chain end to end: GPU producer -> GPU block-FP8 GEMM
    against oracle producer -> oracle GEMM on the same raw draws."""
    from oracle import producer, quant
    M, N, K = synth.WORKLOADS[6][1][6]
    y, r, w = synth.group_chain_raw(M, K)
    wbits = synth.fp8_block_raw(6, 6, 1, N, K)[1]
    wq, wsc = quant.quant_block128_bf16(wbits)
    pre, desc = bs.prelayout_fp8_block(dev_u8(wq))
    q, s, ro = bs.add_rms_quant_fp8_group128(dev_bf16(y), dev_bf16(r), dev_bf16(w), 1e-6)
    c = bs.bsgemm_fp8_block(q, s, desc, pre, dev_f32(wsc))
    torch.cuda.synchronize()
    qo, so, ro_ref = producer.add_rms_quant_group128(y, r, w, 1e-6)
    checks.assert_producer_close(q.cpu().numpy(), s.cpu().numpy(), host_bits16(ro), qo, so, ro_ref, "group chain")
    rows, cols = sample_grid(M, N, 16, 32, seed=78)
    _, ce, asum = gemm.fp8_block_gemm_at(qo, so, wq, wsc, rows, cols)
    checks.assert_gemm_close(host_bits16(c)[rows, cols], ce, asum, "group chain GEMM")


def test_w4a8_prefill_column_strip():
    """A grid of 264 large tiles (8 x 33): the large-tile launch takes the
    first 8192 columns (256 tiles, one round) and a 48-column strip runs as
    split small tiles with offset weight, scale and output pointers.  The
    check covers both parts and the seam between them."""
    M, N, K = 2048, 8240, 1024
    aq, asc, wp, e = w4a8_inputs(8, 5, M, N, K)
    got = host_bits16(_w4_run(aq, asc, wp, e))
    rows, cols = sample_grid(M, N, 16, 24, seed=5)
    seam = np.array([8176, 8191, 8192, 8193, 8207, 8208, 8223, 8224, 8239])
    rr, cc = np.meshgrid(np.unique(rows), seam, indexing="ij")
    rows = np.r_[rows, rr.reshape(-1)]
    cols = np.r_[cols, cc.reshape(-1)]
    _, ce, asum = gemm.w4a8_mxfp4_gemm_at(aq, asc, wp, e, rows, cols)
    checks.assert_gemm_close(got[rows, cols], ce, asum, "w4a8 column strip")


def test_w4a8_prefill_small_tile_rounds():
    """Both levels of the tile plan.  M=2048, N=13392: 8 x 53 large tiles ->
    the large-tile launch takes 8192 columns (256 tiles, one round), the
    5200-column strip is 16 x 41 small tiles, of which 4096 columns (512
    tiles, one round of two per CU) run unsplit and the last 1104 columns
    (144 tiles) in a third launch.  M=500, N=17456, K=2048: 2 x 69 large
    tiles (too few), 4 x 137 = 548 small tiles -> 16384 columns unsplit and
    the last 1072 columns (36 tiles) split in K.  Samples cover every launch
    and the seams between them."""
    for seed, (M, N, K), seams in ((11, (500, 17456, 2048), [16383, 16384, 16399, 17455]),
                                   (12, (2048, 13392, 1024), [8191, 8192, 12287, 12288, 13391])):
        aq, asc, wp, e = w4a8_inputs(8, seed, M, N, K)
        got = host_bits16(_w4_run(aq, asc, wp, e))
        rows, cols = sample_grid(M, N, 12, 24, seed=seed)
        rr, cc = np.meshgrid(np.unique(np.r_[rows, [0, M - 1]]), np.array(seams), indexing="ij")
        rows = np.r_[rows, rr.reshape(-1)]
        cols = np.r_[cols, cc.reshape(-1)]
        _, ce, asum = gemm.w4a8_mxfp4_gemm_at(aq, asc, wp, e, rows, cols)
        checks.assert_gemm_close(got[rows, cols], ce, asum, f"w4a8 tile rounds M={M} N={N} K={K}")


def test_empty_batch_through_the_binding():
    """Zero-row inputs (torch may hand out NULL data pointers for them) give
    empty outputs and no error, for every GEMM and producer."""
    K, N = 512, 256
    wq = np.zeros((N, K), np.uint8)
    pre8, d8 = bs.prelayout_fp8_block(dev_u8(wq))
    c = bs.bsgemm_fp8_block(torch.empty((0, K), dtype=torch.uint8, device="cuda"),
                            torch.empty((0, K // 128), device="cuda"), d8, pre8,
                            torch.ones((N // 128, K // 128), device="cuda"))
    assert c.shape == (0, N)
    pre4, d4 = bs.prelayout_mxfp4(dev_u8(np.zeros((N, K // 2), np.uint8)), dev_u8(np.full((N, K // 32), 127, np.uint8)))
    c = bs.bsgemm_w4a8_mxfp4(torch.empty((0, K), dtype=torch.uint8, device="cuda"), torch.empty((0,), device="cuda"),
                             d4, pre4)
    assert c.shape == (0, N)
    x = torch.empty((0, 5120), dtype=torch.bfloat16, device="cuda")
    assert bs.gemm_bf16_skinny(x, torch.zeros((96, 5120), dtype=torch.bfloat16, device="cuda")).shape == (0, 96)
    g = torch.zeros((5120,), dtype=torch.bfloat16, device="cuda")
    q, s, r = bs.add_rms_quant_fp8(x, x, g)
    assert q.shape == (0, 5120) and s.shape == (0,) and r.shape == (0, 5120)
    q, s, r = bs.add_rms_quant_fp8_group128(x, x, g)
    assert s.shape == (0, 40)
    q, s = bs.silu_mul_quant_fp8(torch.empty((0, 2 * 17408), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 17408)
    torch.cuda.synchronize()
