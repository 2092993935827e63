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
    "bsgemm_w4a8_mxfp4_atiled": (_I, [_P, _P, _D, _P, _P, _L, _I, _I, _I, _P, _Z, _P]),
    "gemm_bf16_skinny": (_I, [_P, _P, _P, _I, _I, _I, _P, _Z, _P]),
    "gemm_bf16_skinny_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "add_rms_quant_fp8": (_I, [_P, _P, _P, _F, _P, _P, _P, _I, _I, _P]),
    "add_rms_quant_fp8_group128": (_I, [_P, _P, _P, _F, _P, _P, _P, _I, _I, _P]),
    "add_rms_quant_fp8_tiled": (_I, [_P, _P, _P, _F, _P, _P, _P, _I, _I, _P]),
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


# ---------------------------------------------------------------- argument checks
# The library sees raw pointers and sizes only, so every tensor's shape, dtype
# and row stride is checked here before the call: a wrong output tensor would
# otherwise be written as if it were a dense [M, N] buffer.
_FP8 = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _need(cond, fn, msg):
    if not cond:
        raise ValueError(f"{fn}: {msg}")


def _arg(fn, name, t, shape, dtypes, contiguous=False, unit_inner=True):
    """t must have `shape` and one of `dtypes`; its last dimension must be
    unit-stride (rows may be padded) or, with contiguous=True, the tensor dense."""
    _need(t is not None, fn, f"{name} is required")
    _need(isinstance(t, torch.Tensor), fn, f"{name} must be a torch.Tensor")
    _need(t.dtype in dtypes, fn, f"{name} has dtype {t.dtype}, expected one of {tuple(str(d) for d in dtypes)}")
    _need(tuple(t.shape) == tuple(shape), fn, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous:
        _need(t.is_contiguous(), fn, f"{name} must be contiguous")
    elif unit_inner and t.dim() >= 2 and t.shape[-1] > 1:
        _need(t.stride(-1) == 1, fn, f"{name} must have unit stride along its last dimension")
        _need(t.stride(0) >= t.shape[-1], fn, f"{name} rows overlap (stride {t.stride(0)} < {t.shape[-1]})")
    return t


def _on_device(fn, *ts):
    """Every tensor lives on the same GPU (a host tensor would hand the kernels a host address)."""
    devs = {t.device for t in ts if t is not None}
    _need(all(d.type == "cuda" for d in devs), fn, f"tensors must be on a GPU, got {sorted(map(str, devs))}")
    _need(len(devs) <= 1, fn, f"tensors are on different devices: {sorted(map(str, devs))}")


def _ws(fn, ws):
    """(pointer, bytes) of an optional workspace tensor (dense, any dtype)."""
    if ws is None:
        return None, 0
    _need(isinstance(ws, torch.Tensor) and ws.is_contiguous(), fn, "ws must be a contiguous tensor")
    return _ptr(ws), ws.numel() * ws.element_size()


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
    fn = "bsgemm_fp8_block"
    _need(isinstance(a, torch.Tensor) and a.dim() == 2, fn, "a must be a 2-D tensor [M, K]")
    M, K = a.shape
    N = desc.N
    _need(desc.K == K, fn, f"a has K = {K}, the weight descriptor K = {desc.K}")
    _arg(fn, "a", a, (M, K), _FP8)
    _arg(fn, "a_scale", a_scale, (M, K // 128), (torch.float32,), unit_inner=False)
    _arg(fn, "w_scale", w_scale, (N // 128, K // 128), (torch.float32,), unit_inner=False)
    _arg(fn, "w_pre", w_pre, (w_pre.numel(),), (torch.uint8,), contiguous=True)
    _need(w_pre.numel() >= desc.total_bytes, fn, f"w_pre holds {w_pre.numel()} bytes, the layout needs "
                                                 f"{desc.total_bytes}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _arg(fn, "out", out, (M, N), _BF16)
    _on_device(fn, a, a_scale, w_pre, w_scale, out, ws)
    a8 = _u8(a)
    ws_p, ws_n = _ws(fn, ws)
    _check(fn, lib().bsgemm_fp8_block(
        _ptr(a8), a8.stride(0), _ptr(a_scale), a_scale.stride(0), a_scale.stride(1), ctypes.byref(desc),
        _ptr(w_pre), _ptr(w_scale.contiguous()), _ptr(out), out.stride(0), M, N, K, ws_p, ws_n, _stream()))
    return out


def bsgemm_w4a8_mxfp4(a, a_scale, desc, w_pre, out=None, ws=None):
    """C[M,N] bf16 = MXFP4 W4A8 GEMM.  a: [M,K] e4m3; a_scale: fp32 [M]."""
    fn = "bsgemm_w4a8_mxfp4"
    _need(isinstance(a, torch.Tensor) and a.dim() == 2, fn, "a must be a 2-D tensor [M, K]")
    M, K = a.shape
    N = desc.N
    _need(desc.K == K, fn, f"a has K = {K}, the weight descriptor K = {desc.K}")
    _arg(fn, "a", a, (M, K), _FP8)
    _arg(fn, "a_scale", a_scale, (M,), (torch.float32,), unit_inner=False)
    _arg(fn, "w_pre", w_pre, (w_pre.numel(),), (torch.uint8,), contiguous=True)
    _need(w_pre.numel() >= desc.total_bytes, fn, f"w_pre holds {w_pre.numel()} bytes, the layout needs "
                                                 f"{desc.total_bytes}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _arg(fn, "out", out, (M, N), _BF16)
    _on_device(fn, a, a_scale, w_pre, out, ws)
    a8 = _u8(a)
    ws_p, ws_n = _ws(fn, ws)
    _check(fn, lib().bsgemm_w4a8_mxfp4(
        _ptr(a8), a8.stride(0), _ptr(a_scale.contiguous()), ctypes.byref(desc), _ptr(w_pre), _ptr(out),
        out.stride(0), M, N, K, ws_p, ws_n, _stream()))
    return out


def tiled_activation_bytes(M, K):
    """Bytes of an activation-tiled [M, K] e4m3 buffer (rows padded to 32)."""
    return (M + 31) // 32 * 32 * K


def bsgemm_w4a8_mxfp4_atiled(a_tiled, a_scale, desc, w_pre, M, out=None, ws=None):
    """C[M,N] bf16 = MXFP4 W4A8 GEMM on an activation in the activation-tiled
    order (uint8, tiled_activation_bytes(M, K) bytes, from
    add_rms_quant_fp8_tiled); M > 64."""
    fn = "bsgemm_w4a8_mxfp4_atiled"
    N, K = desc.N, desc.K
    _arg(fn, "a_tiled", a_tiled, (tiled_activation_bytes(M, K),), _FP8, contiguous=True)
    _arg(fn, "a_scale", a_scale, (M,), (torch.float32,), unit_inner=False)
    _arg(fn, "w_pre", w_pre, (w_pre.numel(),), (torch.uint8,), contiguous=True)
    _need(w_pre.numel() >= desc.total_bytes, fn, f"w_pre holds {w_pre.numel()} bytes, the layout needs "
                                                 f"{desc.total_bytes}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_tiled.device)
    _arg(fn, "out", out, (M, N), _BF16)
    _on_device(fn, a_tiled, a_scale, w_pre, out, ws)
    ws_p, ws_n = _ws(fn, ws)
    _check(fn, lib().bsgemm_w4a8_mxfp4_atiled(
        _ptr(a_tiled), _ptr(a_scale.contiguous()), ctypes.byref(desc), _ptr(w_pre), _ptr(out), out.stride(0),
        M, N, K, ws_p, ws_n, _stream()))
    return out


def gemm_bf16_skinny(x, w, out=None, ws=None):
    """C[M,N] bf16 = x[M,K] . w[N,K]^T (M <= 64).  ws: from alloc_workspace when K is split."""
    fn = "gemm_bf16_skinny"
    _need(isinstance(x, torch.Tensor) and x.dim() == 2 and isinstance(w, torch.Tensor) and w.dim() == 2, fn,
          "x [M, K] and w [N, K] must be 2-D tensors")
    M, K = x.shape
    N = w.shape[0]
    _arg(fn, "x", x, (M, K), _BF16, unit_inner=False)
    _arg(fn, "w", w, (N, K), _BF16, unit_inner=False)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _arg(fn, "out", out, (M, N), _BF16, contiguous=True)    # the C call takes no leading dimension for c
    _on_device(fn, x, w, out, ws)
    x = x.contiguous()
    w = w.contiguous()
    ws_p, ws_n = _ws(fn, ws)
    _check(fn, lib().gemm_bf16_skinny(_ptr(x), _ptr(w), _ptr(out), M, N, K, ws_p, ws_n, _stream()))
    return out


def gemm_bf16_skinny_noalloc(x, w, out=None):
    """gemm_bf16_skinny without a workspace: the library keeps the split-K
    scratch in a static per-GPU array (calls that overlap on one GPU race).
    The C call allocates nothing; pass `out` to allocate nothing here either."""
    fn = "gemm_bf16_skinny_noalloc"
    _need(isinstance(x, torch.Tensor) and x.dim() == 2 and isinstance(w, torch.Tensor) and w.dim() == 2, fn,
          "x [M, K] and w [N, K] must be 2-D tensors")
    M, K = x.shape
    N = w.shape[0]
    _arg(fn, "x", x, (M, K), _BF16, contiguous=True)
    _arg(fn, "w", w, (N, K), _BF16, contiguous=True)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _arg(fn, "out", out, (M, N), _BF16, contiguous=True)
    _on_device(fn, x, w, out)
    _check(fn, lib().gemm_bf16_skinny_noalloc(_ptr(x), _ptr(w), _ptr(out), M, N, K, _stream()))
    return out


# ------------------------------------------------------------------ producers
def _producer_args(fn, y, residual, gamma, q, scale, residual_out, group):
    """Checked (y, residual, gamma, q, scale, residual_out) of the norm
    producers; scale has one value per row (group = 1) or per 128 columns."""
    _need(isinstance(y, torch.Tensor) and y.dim() == 2, fn, "y must be a 2-D tensor [M, K]")
    M, K = y.shape
    dev = y.device
    _arg(fn, "y", y, (M, K), _BF16, unit_inner=False)
    _arg(fn, "residual", residual, (M, K), _BF16, unit_inner=False)
    _arg(fn, "gamma", gamma, (K,), _BF16, unit_inner=False)
    sshape = (M,) if group == 1 else (M, K // 128)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev) if q is None else q
    scale = torch.empty(sshape, dtype=torch.float32, device=dev) if scale is None else scale
    residual_out = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if residual_out is None else residual_out
    _arg(fn, "q", q, (M, K), _FP8, contiguous=True)
    _arg(fn, "scale", scale, sshape, (torch.float32,), contiguous=True)
    _arg(fn, "residual_out", residual_out, (M, K), _BF16, contiguous=True)
    _on_device(fn, y, residual, gamma, q, scale, residual_out)
    return y.contiguous(), residual.contiguous(), gamma.contiguous(), q, scale, residual_out


def _quant_args(fn, x, q, scale, qshape, sshape, in_shape=None):
    """Checked (x, q, scale) of the quantizers."""
    _arg(fn, "x", x, in_shape or qshape, _BF16, unit_inner=False)
    q = torch.empty(qshape, dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(sshape, dtype=torch.float32, device=x.device) if scale is None else scale
    _arg(fn, "q", q, qshape, _FP8, contiguous=True)
    _arg(fn, "scale", scale, sshape, (torch.float32,), contiguous=True)
    _on_device(fn, x, q, scale)
    return x.contiguous(), q, scale


def add_rms_quant_fp8(y, residual, gamma, eps=1e-6, q=None, scale=None, residual_out=None):
    """(q e4m3 [M,K] as uint8, scale fp32 [M], residual_out bf16 [M,K])."""
    fn = "add_rms_quant_fp8"
    y, residual, gamma, q, scale, residual_out = _producer_args(fn, y, residual, gamma, q, scale, residual_out, 1)
    M, K = y.shape
    _check(fn, lib().add_rms_quant_fp8(
        _ptr(y), _ptr(residual), _ptr(gamma), ctypes.c_float(eps), _ptr(q), _ptr(scale), _ptr(residual_out),
        M, K, _stream()))
    return q, scale, residual_out


def add_rms_quant_fp8_tiled(y, residual, gamma, eps=1e-6, q=None, scale=None, residual_out=None):
    """(q e4m3 in the activation-tiled order, uint8 [tiled_activation_bytes(M, K)],
    scale fp32 [M], residual_out bf16 [M,K])."""
    fn = "add_rms_quant_fp8_tiled"
    _need(isinstance(y, torch.Tensor) and y.dim() == 2, fn, "y must be a 2-D tensor [M, K]")
    M, K = y.shape
    if q is None:
        q = torch.empty((tiled_activation_bytes(M, K),), dtype=torch.uint8, device=y.device)
    _arg(fn, "q", q, (tiled_activation_bytes(M, K),), _FP8, contiguous=True)
    q2 = q.view(-1)[: M * K].view(M, K)      # shape stand-in for the shared checks only
    y, residual, gamma, _, scale, residual_out = _producer_args(fn, y, residual, gamma, q2, scale, residual_out, 1)
    _check(fn, lib().add_rms_quant_fp8_tiled(
        _ptr(y), _ptr(residual), _ptr(gamma), ctypes.c_float(eps), _ptr(q), _ptr(scale), _ptr(residual_out),
        M, K, _stream()))
    return q, scale, residual_out


def add_rms_quant_fp8_group128(y, residual, gamma, eps=1e-6, q=None, scale=None, residual_out=None):
    """(q e4m3 [M,K] as uint8, scale fp32 [M, K/128], residual_out bf16 [M,K])."""
    fn = "add_rms_quant_fp8_group128"
    y, residual, gamma, q, scale, residual_out = _producer_args(fn, y, residual, gamma, q, scale, residual_out,
                                                                128)
    M, K = y.shape
    _check(fn, lib().add_rms_quant_fp8_group128(
        _ptr(y), _ptr(residual), _ptr(gamma), ctypes.c_float(eps), _ptr(q), _ptr(scale), _ptr(residual_out),
        M, K, _stream()))
    return q, scale, residual_out


def silu_mul_quant_fp8(gu, q=None, scale=None):
    """gu bf16 [M, 2N] (gate half first) -> (q e4m3 [M, N] as uint8, scale fp32 [M])."""
    fn = "silu_mul_quant_fp8"
    _need(isinstance(gu, torch.Tensor) and gu.dim() == 2 and gu.shape[1] % 2 == 0, fn,
          "gu must be a 2-D tensor [M, 2N]")
    M, N2 = gu.shape
    N = N2 // 2
    gu, q, scale = _quant_args(fn, gu, q, scale, (M, N), (M,), in_shape=(M, N2))
    _check(fn, lib().silu_mul_quant_fp8(_ptr(gu), _ptr(q), _ptr(scale), M, N, _stream()))
    return q, scale


def quant_fp8_per_token(x, q=None, scale=None):
    fn = "quant_fp8_per_token"
    _need(isinstance(x, torch.Tensor) and x.dim() == 2, fn, "x must be a 2-D tensor [M, K]")
    M, K = x.shape
    x, q, scale = _quant_args(fn, x, q, scale, (M, K), (M,))
    _check(fn, lib().quant_fp8_per_token(_ptr(x), _ptr(q), _ptr(scale), M, K, _stream()))
    return q, scale


def quant_fp8_group128(x, q=None, scale=None):
    fn = "quant_fp8_group128"
    _need(isinstance(x, torch.Tensor) and x.dim() == 2, fn, "x must be a 2-D tensor [M, K]")
    M, K = x.shape
    x, q, scale = _quant_args(fn, x, q, scale, (M, K), (M, K // 128))
    _check(fn, lib().quant_fp8_group128(_ptr(x), _ptr(q), _ptr(scale), M, K, _stream()))
    return q, scale


def quant_fp8_block128(w, q=None, scale=None):
    fn = "quant_fp8_block128"
    _need(isinstance(w, torch.Tensor) and w.dim() == 2, fn, "w must be a 2-D tensor [N, K]")
    N, K = w.shape
    w, q, scale = _quant_args(fn, w, q, scale, (N, K), (N // 128, K // 128))
    _check(fn, lib().quant_fp8_block128(_ptr(w), _ptr(q), _ptr(scale), N, K, _stream()))
    return q, scale
