"""ctypes binding of libfa_mi355x.so.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/fa_mi355x.h.  torch supplies the
device memory and the stream; nothing here computes attention, and there is no
fallback: if the library is missing or the device is not gfx950 the call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

from .build import LIB_PATH

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM",
    4: "FA_ERR_DTYPE", 5: "FA_ERR_ALIGN", 6: "FA_ERR_SCALE", 7: "FA_ERR_ALIAS",
    8: "FA_ERR_NO_DEVICE", 9: "FA_ERR_ARCH", 10: "FA_ERR_HIP", 11: "FA_ERR_WORKSPACE",
}
STATUS_CODE = {name: code for code, name in STATUS.items()}
EXPORTS = ("flash_attn_fwd", "flash_attn_fwd_persistent", "flash_attn_bwd", "flash_attn_bwd_workspace_size", "flash_attn_fwd_fp8", "flash_attn_fwd_kvcache", "flash_attn_fwd_kvcache_noalloc",
           "flash_attn_kvcache_splits", "flash_attn_kvcache_workspace_size", "flash_attn_status_str",
           "flash_attn_last_error", "flash_attn_abi_version")
ABI_VERSION = 7

_lib = None
_lock = threading.Lock()


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.name}: {detail}" if detail else self.name)


def library_path() -> str:
    return os.environ.get("FA_MI355X_LIB", LIB_PATH)


def lib() -> ctypes.CDLL:
    """Load libfa_mi355x.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is not built; build it with "
                    "`python -m io_aware_tiled_08_amd.build` (needs hipcc)")
            L = ctypes.CDLL(path)
            L.flash_attn_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
            L.flash_attn_fwd.restype = ctypes.c_int
            L.flash_attn_fwd_persistent.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
            L.flash_attn_fwd_persistent.restype = ctypes.c_int
            L.flash_attn_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int64] * 4 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                ctypes.c_void_p]
            L.flash_attn_bwd.restype = ctypes.c_int
            L.flash_attn_bwd_workspace_size.argtypes = [ctypes.c_int64] * 3
            L.flash_attn_bwd_workspace_size.restype = ctypes.c_int64
            L.flash_attn_fwd_fp8.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                ctypes.c_void_p]
            L.flash_attn_fwd_fp8.restype = ctypes.c_int
            L.flash_attn_fwd_kvcache.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
                ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                ctypes.c_int, ctypes.c_void_p]
            L.flash_attn_fwd_kvcache.restype = ctypes.c_int
            L.flash_attn_fwd_kvcache_noalloc.argtypes = [ctypes.c_void_p] * 5 + [
                ctypes.c_int64] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
            L.flash_attn_fwd_kvcache_noalloc.restype = ctypes.c_int
            L.flash_attn_kvcache_splits.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int]
            L.flash_attn_kvcache_splits.restype = ctypes.c_int
            L.flash_attn_kvcache_workspace_size.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int]
            L.flash_attn_kvcache_workspace_size.restype = ctypes.c_int64
            L.flash_attn_status_str.argtypes = [ctypes.c_int]
            L.flash_attn_status_str.restype = ctypes.c_char_p
            L.flash_attn_last_error.argtypes = []
            L.flash_attn_last_error.restype = ctypes.c_char_p
            L.flash_attn_abi_version.argtypes = []
            L.flash_attn_abi_version.restype = ctypes.c_int
            if L.flash_attn_abi_version() != ABI_VERSION:
                raise RuntimeError(f"{path}: ABI version {L.flash_attn_abi_version()}, "
                                   f"binding expects {ABI_VERSION}")
            _lib = L
        return _lib


def last_error() -> str:
    return lib().flash_attn_last_error().decode()


def flash_attn_fwd_ptr(q: int, k: int, v: int, o: int, lse: int, B: int, H: int,
                       N: int, d: int, scale: float, causal: bool, dtype: int,
                       stream: int = 0) -> int:
    """Raw call of the C entry point on integer addresses; returns the status."""
    return lib().flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, int(bool(causal)),
                                dtype, stream)


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return codes[t.dtype]


def _forward_operands(q, k, v, o, lse, scale):
    """Check q, k, v (and o, lse when given), allocate missing outputs."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must have the same dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor like q")
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    return (B, H, N, d), code, float(scale), o, lse


def flash_attn_fwd(q, k, v, o=None, lse=None, *, scale: Optional[float] = None,
                   causal: bool = False, stream=None) -> Tuple["object", "object"]:
    """O = softmax(scale * Q K^T) V and LSE for contiguous [B, H, N, d] tensors.

    q, k, v: device tensors of one dtype (float32, float16 or bfloat16).
    o, lse: optional preallocated outputs ([B, H, N, d] of q's dtype and
    [B, H, N] float32); allocated here when omitted.
    scale: defaults to 1/sqrt(d).  causal: lower-triangular mask (j <= i).
    stream: a torch.cuda.Stream; defaults to the current stream of q's device.
    The kernel is enqueued asynchronously on that stream.
    """
    import torch
    (B, H, N, d), code, scale, o, lse = _forward_operands(q, k, v, o, lse, scale)
    L = lib()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, N, d, scale, int(bool(causal)),
                              code, s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return o, lse


def flash_attn_fwd_persistent(q, k, v, o=None, lse=None, *, scale: Optional[float] = None,
                              causal: bool = False, num_workgroups: int = 0,
                              stream=None) -> Tuple["object", "object"]:
    """flash_attn_fwd (float16 / bfloat16) on a persistent grid of
    num_workgroups resident workgroups (0: one per compute unit) that loop
    over the 256-row query blocks.  Arguments otherwise as flash_attn_fwd."""
    import torch
    (B, H, N, d), code, scale, o, lse = _forward_operands(q, k, v, o, lse, scale)
    L = lib()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_fwd_persistent(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                         lse.data_ptr(), B, H, N, d, scale, int(bool(causal)),
                                         int(num_workgroups), code, s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return o, lse


def flash_attn_fwd_persistent_ptr(q: int, k: int, v: int, o: int, lse: int, B: int, H: int,
                                  N: int, d: int, scale: float, causal: bool,
                                  num_workgroups: int, dtype: int, stream: int = 0) -> int:
    """Raw call of the C entry point on integer addresses; returns the status."""
    return lib().flash_attn_fwd_persistent(q, k, v, o, lse, B, H, N, d, scale,
                                           int(bool(causal)), num_workgroups, dtype, stream)


def kvcache_splits(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0) -> int:
    """Key ranges flash_attn_fwd_kvcache uses for these sizes (C ABI)."""
    return lib().flash_attn_kvcache_splits(B, H, Nq, Nk, d, num_splits)


def kvcache_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int,
                           num_splits: int = 0) -> int:
    """Workspace bytes flash_attn_fwd_kvcache needs for these sizes (C ABI)."""
    return lib().flash_attn_kvcache_workspace_size(B, H, Nq, Nk, d, num_splits)


def flash_attn_fwd_kvcache_ptr(q: int, k: int, v: int, o: int, lse: int, B: int, H: int,
                               Nq: int, Nk: int, d: int, scale: float, causal: bool,
                               num_splits: int, workspace: int, workspace_bytes: int,
                               dtype: int, stream: int = 0) -> int:
    """Raw call of the C entry point on integer addresses; returns the status."""
    return lib().flash_attn_fwd_kvcache(q, k, v, o, lse, B, H, Nq, Nk, d, scale,
                                        int(bool(causal)), num_splits, workspace,
                                        workspace_bytes, dtype, stream)


def _check_kvcache_tensors(q, k, v, o, lse):
    """Shapes, dtypes, devices and contiguity of a cache call's tensors;
    returns (B, H, Nq, Nk, d, dtype code)."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    Nk = k.shape[2]
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must have the same dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    code = _dtype_code(q)
    if (not isinstance(o, torch.Tensor) or o.shape != q.shape or o.dtype != q.dtype
            or o.device != q.device or not o.is_contiguous()):
        raise ValueError("o must be a contiguous tensor like q")
    if (not isinstance(lse, torch.Tensor) or lse.shape != (B, H, Nq)
            or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    return B, H, Nq, Nk, d, code


def flash_attn_fwd_kvcache_noalloc(q, k, v, o, lse, *, scale: Optional[float] = None,
                                   causal: bool = False, num_splits: int = 0, stream=None):
    """flash_attn_fwd_kvcache with the split partials in the library's own
    static device scratch (FA_MI355X_KVCACHE_SCRATCH_BYTES per GPU): neither
    the library nor this function allocates anything, so o and lse must be
    passed.  Calls that may overlap in time on one GPU race on that scratch;
    order them on one stream.  Enqueued on `stream` (default: the current
    stream of q's device) without synchronising; returns (o, lse)."""
    import torch
    B, H, Nq, Nk, d, code = _check_kvcache_tensors(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = lib()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_fwd_kvcache_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                                              float(scale), int(bool(causal)), int(num_splits),
                                              code, s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return o, lse


def flash_attn_fwd_kvcache(q, k, v, o=None, lse=None, *, scale: Optional[float] = None,
                           causal: bool = False, num_splits: int = 0, workspace=None,
                           stream=None) -> Tuple["object", "object"]:
    """Attention of q [B, H, Nq, d] against a key/value cache k, v [B, H, Nk, d].

    float16 or bfloat16 device tensors, contiguous.  causal: the queries are
    the last Nq of Nk positions, query i sees keys j <= i + Nk - Nq.
    num_splits <= 0 lets the library choose how many key ranges to compute
    separately and merge.  workspace: optional device tensor of at least
    kvcache_workspace_size(...) bytes; allocated here when needed and omitted.
    o, lse: optional preallocated outputs.  Enqueued on `stream` (default: the
    current stream of q's device) without synchronising.
    """
    import torch
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float32,
                          device=q.device)
    B, H, Nq, Nk, d, code = _check_kvcache_tensors(q, k, v, o, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = lib()
    need = L.flash_attn_kvcache_workspace_size(B, H, Nq, Nk, d, int(num_splits))
    if need < 0:
        raise ValueError("workspace size overflows")
    ws_ptr, ws_bytes = 0, 0
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr = workspace.data_ptr()
        ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_fwd_kvcache(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, Nq, Nk, d, float(scale),
                                      int(bool(causal)), int(num_splits), ws_ptr, ws_bytes,
                                      code, s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return o, lse


def flash_attn_fwd_fp8(q, k, v, o=None, lse=None, *, q_descale: float, k_descale: float,
                       v_descale: float, scale: Optional[float] = None, causal: bool = False,
                       stream=None) -> Tuple["object", "object"]:
    """8-bit forward: q, k, v contiguous [B, H, N, d] torch.float8_e4m3fn device
    tensors whose values are code * descale (one factor per tensor).  Returns
    O as bfloat16 [B, H, N, d] and LSE as float32 [B, H, N]; o and lse may be
    preallocated.  scale defaults to 1/sqrt(d).  Enqueued on `stream` (default:
    the current stream of q's device) without synchronising."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{name} must be torch.float8_e4m3fn (got {t.dtype})")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if (o.shape != q.shape or o.dtype != torch.bfloat16 or o.device != q.device
            or not o.is_contiguous()):
        raise ValueError("o must be a contiguous bfloat16 tensor of q's shape")
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    L = lib()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                                  float(q_descale), float(k_descale), float(v_descale),
                                  s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return o, lse


def flash_attn_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, *,
                   scale: Optional[float] = None, causal: bool = False, workspace=None,
                   stream=None):
    """Gradients (dq, dk, dv) of flash_attn_fwd for upstream gradient dout.

    q, k, v, o, dout: contiguous [B, H, N, d] float16 or bfloat16 device
    tensors (o and lse as flash_attn_fwd returned them for the same scale and
    causal); dq, dk, dv optional preallocated outputs; workspace optional
    device tensor of at least flash_attn_bwd_workspace_size(B, H, N) bytes
    (allocated here when omitted).  Enqueued on `stream` (default: the current
    stream of q's device) without synchronising.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    code = _dtype_code(q)
    if (lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like q")
    L = lib()
    need = L.flash_attn_bwd_workspace_size(B, H, N)
    if need < 0:
        raise ValueError("workspace size overflows")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        st = L.flash_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              code, s.cuda_stream)
    if st != 0:
        raise FlashAttnError(st, L.flash_attn_last_error().decode())
    return dq, dk, dv
