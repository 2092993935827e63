"""Thin ctypes binding over libbsgemm.so (include/bsgemm.h).

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  Outputs that are not passed in are allocated with torch (device
memory plumbing).  A negative status from the library raises BsError.  If the
library is not built, importing the functions fails loudly: there is no
fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsgemm.so")

BS_OP_FP8_BLOCK = 1
BS_OP_W4A8_MXFP4 = 2
BS_OP_BF16_SKINNY = 3
BS_LAYOUT_FP8_BLOCK = 0x38423631
BS_LAYOUT_MXFP4 = 0x34584D31
BS_WDESC_MAGIC = 0x42534744


class BsError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {lib().bs_status_string(status).decode()} (status {status})")


class WDesc(ctypes.Structure):
    """Host-side weight descriptor (bs_wdesc)."""
    _fields_ = [("magic", ctypes.c_uint32), ("layout", ctypes.c_uint32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes_bytes", ctypes.c_uint64), ("scales_offset", ctypes.c_uint64),
                ("scales_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_Z = ctypes.c_size_t
_F = ctypes.c_float
_D = ctypes.POINTER(WDesc)
_FP = ctypes.POINTER(ctypes.c_float)

SIGNATURES = {
    "bs_status_string": (ctypes.c_char_p, [_I]),
    "bs_version": (_I, []),
    "bs_prelayout_fp8_block_bytes": (_Z, [_I, _I]),
    "bs_prelayout_fp8_block": (_I, [_P, _P, _Z, _I, _I, _D, _P]),
    "bs_unprelayout_fp8_block": (_I, [_D, _P, _P, _P]),
    "bs_prelayout_mxfp4_bytes": (_Z, [_I, _I]),
    "bs_prelayout_mxfp4": (_I, [_P, _P, _P, _Z, _I, _I, _D, _P]),
    "bs_unprelayout_mxfp4": (_I, [_D, _P, _P, _P, _P]),
    "bs_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "bsgemm_fp8_block": (_I, [_P, _L, _P, _L, _L, _D, _P, _P, _P, _L, _I, _I, _I, _P, _Z, _P]),
    "bsgemm_w4a8_mxfp4": (_I, [_P, _L, _P, _D, _P, _P, _L, _I, _I, _I, _P, _Z, _P]),
    "gemm_bf16_skinny": (_I, [_P, _P, _P, _I, _I, _I, _P, _Z, _P]),
    "add_rms_quant_fp8": (_I, [_P, _P, _P, _F, _P, _P, _P, _I, _I, _P]),
    "add_rms_quant_fp8_group128": (_I, [_P, _P, _P, _F, _P, _P, _P, _I, _I, _P]),
    "silu_mul_quant_fp8": (_I, [_P, _P, _P, _I, _I, _P]),
    "quant_fp8_per_token": (_I, [_P, _P, _P, _I, _I, _P]),
    "quant_fp8_group128": (_I, [_P, _P, _P, _I, _I, _P]),
    "quant_fp8_block128": (_I, [_P, _P, _P, _I, _I, _P]),
}

_LIB = None


def lib():
    """Load libbsgemm.so once and declare every C signature."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run block_scaled_precision_04_amd.build.build() "
                               "(hipcc for gfx950); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(fn, status):
    if status != 0:
        raise BsError(fn, status)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _u8(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def _bits16(t):
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bf16 data (bfloat16 or 16-bit bit patterns), got {t.dtype}")


# ------------------------------------------------------------------ layouts
def prelayout_fp8_block(w_e4m3):
    """[N, K] e4m3 codes (uint8 or float8_e4m3fn) -> (pre-laid-out uint8 buffer, WDesc)."""
    w = _u8(w_e4m3).contiguous()
    N, K = w.shape
    nbytes = lib().bs_prelayout_fp8_block_bytes(N, K)
    if nbytes == 0:
        raise BsError("bs_prelayout_fp8_block_bytes", -2)
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    desc = WDesc()
    _check("bs_prelayout_fp8_block", lib().bs_prelayout_fp8_block(_ptr(w), _ptr(out), nbytes, N, K,
                                                                   ctypes.byref(desc), _stream()))
    return out, desc


def unprelayout_fp8_block(desc, pre):
    w = torch.empty((desc.N, desc.K), dtype=torch.uint8, device=pre.device)
    _check("bs_unprelayout_fp8_block", lib().bs_unprelayout_fp8_block(ctypes.byref(desc), _ptr(pre), _ptr(w),
                                                                       _stream()))
    return w


def prelayout_mxfp4(w_packed, w_e8m0):
    """[N, K/2] packed e2m1 + [N, K/32] e8m0 -> (pre-laid-out uint8 buffer, WDesc)."""
    wp = _u8(w_packed).contiguous()
    e = _u8(w_e8m0).contiguous()
    N, Kh = wp.shape
    K = 2 * Kh
    nbytes = lib().bs_prelayout_mxfp4_bytes(N, K)
    if nbytes == 0:
        raise BsError("bs_prelayout_mxfp4_bytes", -2)
    out = torch.empty(nbytes, dtype=torch.uint8, device=wp.device)
    desc = WDesc()
    _check("bs_prelayout_mxfp4", lib().bs_prelayout_mxfp4(_ptr(wp), _ptr(e), _ptr(out), nbytes, N, K,
                                                           ctypes.byref(desc), _stream()))
    return out, desc


def unprelayout_mxfp4(desc, pre):
    wp = torch.empty((desc.N, desc.K // 2), dtype=torch.uint8, device=pre.device)
    e = torch.empty((desc.N, desc.K // 32), dtype=torch.uint8, device=pre.device)
    _check("bs_unprelayout_mxfp4", lib().bs_unprelayout_mxfp4(ctypes.byref(desc), _ptr(pre), _ptr(wp), _ptr(e),
                                                               _stream()))
    return wp, e


def workspace_bytes(op, M, N, K):
    return int(lib().bs_workspace_bytes(op, M, N, K))


def alloc_workspace(op, M, N, K, device="cuda"):
    """A zero-filled workspace for (op, M, N, K), or None when none is needed.
    Allocate once (outside graph capture) and reuse: the kernels leave it zeroed."""
    n = workspace_bytes(op, M, N, K)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


# ------------------------------------------------------------------ GEMMs
def bsgemm_fp8_block(a, a_scale, desc, w_pre, w_scale, out=None, ws=None):
    """C[M,N] bf16 = block-FP8 GEMM.  a: [M,K] e4m3 (row stride in bytes may be
    padded to a multiple of 16); a_scale: fp32 [M, K/128] with any strides;
    w_scale: fp32 [N/128, K/128] contiguous."""
    a8 = _u8(a)
    M, K = a8.shape
    N = desc.N
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a8.device)
    ws_p, ws_n = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    _check("bsgemm_fp8_block", lib().bsgemm_fp8_block(
        _ptr(a8), a8.stride(0), _ptr(a_scale), a_scale.stride(0), a_scale.stride(1), ctypes.byref(desc),
        _ptr(w_pre), _ptr(w_scale.contiguous()), _ptr(out), out.stride(0), M, N, K, ws_p, ws_n, _stream()))
    return out


def bsgemm_w4a8_mxfp4(a, a_scale, desc, w_pre, out=None, ws=None):
    """C[M,N] bf16 = MXFP4 W4A8 GEMM.  a: [M,K] e4m3; a_scale: fp32 [M]."""
    a8 = _u8(a)
    M, K = a8.shape
    N = desc.N
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a8.device)
    ws_p, ws_n = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    _check("bsgemm_w4a8_mxfp4", lib().bsgemm_w4a8_mxfp4(
        _ptr(a8), a8.stride(0), _ptr(a_scale.contiguous()), ctypes.byref(desc), _ptr(w_pre), _ptr(out),
        out.stride(0), M, N, K, ws_p, ws_n, _stream()))
    return out


def gemm_bf16_skinny(x, w, out=None, ws=None):
    """C[M,N] bf16 = x[M,K] . w[N,K]^T (M <= 64).  ws: from alloc_workspace when K is split."""
    x = _bits16(x).contiguous()
    w = _bits16(w).contiguous()
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws_p, ws_n = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    _check("gemm_bf16_skinny", lib().gemm_bf16_skinny(_ptr(x), _ptr(w), _ptr(out), M, N, K, ws_p, ws_n,
                                                       _stream()))
    return out


# ------------------------------------------------------------------ producers
def add_rms_quant_fp8(y, residual, gamma, eps=1e-6, q=None, scale=None, residual_out=None):
    """(q e4m3 [M,K] as uint8, scale fp32 [M], residual_out bf16 [M,K])."""
    y = _bits16(y).contiguous()
    residual = _bits16(residual).contiguous()
    gamma = _bits16(gamma).contiguous()
    M, K = y.shape
    dev = y.device
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=dev) if scale is None else scale
    residual_out = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if residual_out is None else residual_out
    _check("add_rms_quant_fp8", lib().add_rms_quant_fp8(
        _ptr(y), _ptr(residual), _ptr(gamma), ctypes.c_float(eps), _ptr(q), _ptr(scale), _ptr(residual_out),
        M, K, _stream()))
    return q, scale, residual_out


def add_rms_quant_fp8_group128(y, residual, gamma, eps=1e-6, q=None, scale=None, residual_out=None):
    """(q e4m3 [M,K] as uint8, scale fp32 [M, K/128], residual_out bf16 [M,K])."""
    y = _bits16(y).contiguous()
    residual = _bits16(residual).contiguous()
    gamma = _bits16(gamma).contiguous()
    M, K = y.shape
    dev = y.device
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty((M, K // 128), dtype=torch.float32, device=dev) if scale is None else scale
    residual_out = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if residual_out is None else residual_out
    _check("add_rms_quant_fp8_group128", lib().add_rms_quant_fp8_group128(
        _ptr(y), _ptr(residual), _ptr(gamma), ctypes.c_float(eps), _ptr(q), _ptr(scale), _ptr(residual_out),
        M, K, _stream()))
    return q, scale, residual_out


def silu_mul_quant_fp8(gu, q=None, scale=None):
    """gu bf16 [M, 2N] (gate half first) -> (q e4m3 [M, N] as uint8, scale fp32 [M])."""
    gu = _bits16(gu).contiguous()
    M, N2 = gu.shape
    N = N2 // 2
    q = torch.empty((M, N), dtype=torch.uint8, device=gu.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=gu.device) if scale is None else scale
    _check("silu_mul_quant_fp8", lib().silu_mul_quant_fp8(_ptr(gu), _ptr(q), _ptr(scale), M, N, _stream()))
    return q, scale


def quant_fp8_per_token(x, q=None, scale=None):
    x = _bits16(x).contiguous()
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((M,), dtype=torch.float32, device=x.device) if scale is None else scale
    _check("quant_fp8_per_token", lib().quant_fp8_per_token(_ptr(x), _ptr(q), _ptr(scale), M, K, _stream()))
    return q, scale


def quant_fp8_group128(x, q=None, scale=None):
    x = _bits16(x).contiguous()
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if scale is None else scale
    _check("quant_fp8_group128", lib().quant_fp8_group128(_ptr(x), _ptr(q), _ptr(scale), M, K, _stream()))
    return q, scale


def quant_fp8_block128(w, q=None, scale=None):
    w = _bits16(w).contiguous()
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device) if q is None else q
    scale = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device) if scale is None else scale
    _check("quant_fp8_block128", lib().quant_fp8_block128(_ptr(w), _ptr(q), _ptr(scale), N, K, _stream()))
    return q, scale
