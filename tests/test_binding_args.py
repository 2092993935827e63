"""Host-side argument checks of the Python binding: a tensor of the wrong
shape, dtype, row stride or device is refused before anything reaches the
library (whose C calls see raw pointers and sizes only, so a wrong output
tensor would be written as a dense [M, N] buffer).  CPU only: every call here
is refused before any device memory is touched."""
import pytest
import torch

import block_scaled_precision_04_amd as bs
from block_scaled_precision_04_amd._binding import WDesc, BS_WDESC_MAGIC, BS_LAYOUT_FP8_BLOCK, BS_LAYOUT_MXFP4

M, N, K = 8, 256, 512


def _desc(layout, total):
    return WDesc(BS_WDESC_MAGIC, layout, N, K, N * K // (1 if layout == BS_LAYOUT_FP8_BLOCK else 2), 0, 0, total)


def _fp8_args():
    return dict(a=torch.zeros((M, K), dtype=torch.uint8), a_scale=torch.ones((M, K // 128)),
                desc=_desc(BS_LAYOUT_FP8_BLOCK, N * K), w_pre=torch.zeros(N * K, dtype=torch.uint8),
                w_scale=torch.ones((N // 128, K // 128)))


def _w4_args():
    return dict(a=torch.zeros((M, K), dtype=torch.uint8), a_scale=torch.ones((M,)),
                desc=_desc(BS_LAYOUT_MXFP4, N * K), w_pre=torch.zeros(N * K, dtype=torch.uint8))


def _refused(fn, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(**kw)


@pytest.mark.parametrize("which", ["fp8", "w4a8"])
def test_gemm_output_checks(which):
    fn, args = (bs.bsgemm_fp8_block, _fp8_args()) if which == "fp8" else (bs.bsgemm_w4a8_mxfp4, _w4_args())
    _refused(fn, "out has shape", **args, out=torch.zeros((M, N - 16), dtype=torch.bfloat16))
    _refused(fn, "out has shape", **args, out=torch.zeros((M + 1, N), dtype=torch.bfloat16))
    _refused(fn, "out has dtype", **args, out=torch.zeros((M, N), dtype=torch.float32))
    _refused(fn, "unit stride", **args, out=torch.zeros((N, M), dtype=torch.bfloat16).t())
    # a padded row stride is fine for the check (the library takes ldc); the refusal is the host device
    _refused(fn, "on a GPU", **args, out=torch.zeros((M, N + 32), dtype=torch.bfloat16)[:, :N])


@pytest.mark.parametrize("which", ["fp8", "w4a8"])
def test_gemm_input_checks(which):
    fn, base = (bs.bsgemm_fp8_block, _fp8_args) if which == "fp8" else (bs.bsgemm_w4a8_mxfp4, _w4_args)
    a = base()
    a["a"] = torch.zeros((M, K), dtype=torch.float16)
    _refused(fn, "a has dtype", **a)
    a = base()
    a["a"] = torch.zeros((K, M), dtype=torch.uint8).t()
    _refused(fn, "unit stride", **a)
    a = base()
    a["a"] = torch.zeros((M, K - 128), dtype=torch.uint8)
    _refused(fn, "descriptor K", **a)
    a = base()
    a["a_scale"] = torch.ones((M + 1,) if which == "w4a8" else (M, K // 128 + 1))
    _refused(fn, "a_scale has shape", **a)
    a = base()
    a["a_scale"] = a["a_scale"].double()
    _refused(fn, "a_scale has dtype", **a)
    a = base()
    a["w_pre"] = torch.zeros(N * K - 1, dtype=torch.uint8)
    _refused(fn, "the layout needs", **a)
    if which == "fp8":
        a = base()
        a["w_scale"] = torch.ones((N // 128 + 1, K // 128))
        _refused(fn, "w_scale has shape", **a)
    _refused(fn, "on a GPU", **base())


def test_skinny_checks():
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    w = torch.zeros((96, K), dtype=torch.bfloat16)
    # the C call takes no leading dimension for c: only a dense [M, N] output is accepted
    _refused(bs.gemm_bf16_skinny, "out must be contiguous", x=x, w=w,
             out=torch.zeros((M, 128), dtype=torch.bfloat16)[:, :96])
    _refused(bs.gemm_bf16_skinny, "out has shape", x=x, w=w, out=torch.zeros((M, 80), dtype=torch.bfloat16))
    _refused(bs.gemm_bf16_skinny, "w has shape", x=x, w=torch.zeros((96, K + 128), dtype=torch.bfloat16))
    _refused(bs.gemm_bf16_skinny, "x has dtype", x=x.float(), w=w)
    _refused(bs.gemm_bf16_skinny, "on a GPU", x=x, w=w)


def test_producer_checks():
    y = torch.zeros((M, K), dtype=torch.bfloat16)
    g = torch.zeros((K,), dtype=torch.bfloat16)
    _refused(bs.add_rms_quant_fp8, "gamma has shape", y=y, residual=y, gamma=torch.zeros((K + 8,), dtype=torch.bfloat16))
    _refused(bs.add_rms_quant_fp8, "residual has shape", y=y, residual=y[:, :K - 8], gamma=g)
    _refused(bs.add_rms_quant_fp8, "q must be contiguous", y=y, residual=y, gamma=g,
             q=torch.zeros((M, 2 * K), dtype=torch.uint8)[:, :K])
    _refused(bs.add_rms_quant_fp8, "scale has shape", y=y, residual=y, gamma=g, scale=torch.zeros((M, 1)))
    _refused(bs.add_rms_quant_fp8_group128, "scale has shape", y=y, residual=y, gamma=g, scale=torch.zeros((M,)))
    _refused(bs.add_rms_quant_fp8, "residual_out has dtype", y=y, residual=y, gamma=g,
             residual_out=torch.zeros((M, K), dtype=torch.float32))
    _refused(bs.add_rms_quant_fp8, "on a GPU", y=y, residual=y, gamma=g)
    _refused(bs.silu_mul_quant_fp8, "q has shape", gu=torch.zeros((M, 2 * K), dtype=torch.bfloat16),
             q=torch.zeros((M, 2 * K), dtype=torch.uint8))
    _refused(bs.quant_fp8_per_token, "scale has dtype", x=y, scale=torch.zeros((M,), dtype=torch.float64))
    _refused(bs.quant_fp8_group128, "scale has shape", x=y, scale=torch.zeros((M,)))
    _refused(bs.quant_fp8_block128, "q has shape", w=torch.zeros((N, K), dtype=torch.bfloat16),
             q=torch.zeros((N, K - 8), dtype=torch.uint8))
