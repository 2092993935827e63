"""bsgemm for MI355X (gfx950): block-scaled low-precision linear layer + fused producer.

The compute lives in libbsgemm.so (hand-written HIP, C ABI in include/bsgemm.h);
this package is its thin Python binding.  Importing the package does not load
the library; the first call of a binding function does, and fails loudly if
the library has not been built (block_scaled_precision_04_amd.build.build()).
"""
_BINDING_NAMES = (
    "prelayout_fp8_block", "unprelayout_fp8_block", "prelayout_mxfp4", "unprelayout_mxfp4",
    "workspace_bytes", "alloc_workspace", "bsgemm_fp8_block", "bsgemm_w4a8_mxfp4", "gemm_bf16_skinny",
    "gemm_bf16_skinny_noalloc", "bsgemm_w4a8_mxfp4_atiled", "add_rms_quant_fp8_tiled", "tiled_activation_bytes",
    "add_rms_quant_fp8", "add_rms_quant_fp8_group128", "silu_mul_quant_fp8", "quant_fp8_per_token", "quant_fp8_group128", "quant_fp8_block128",
    "BsError", "WDesc", "lib", "BS_OP_FP8_BLOCK", "BS_OP_W4A8_MXFP4", "BS_OP_BF16_SKINNY",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
