"""Python binding of the MI355X exact-attention library (include/fa.h).

Argument marshalling only: every step of the attention runs in the HIP
kernels of libfa_mi355x.so.  The names mirror the C ABI (fa_fwd, fa_fwd_query,
fa_fwd_split, fa_fwd_split_query, fa_bwd, fa_bwd_query, fa_bwd_qk, fa_bwd_qk_query, fa_status_str,
fa_fwd_fp8, fa_fwd_fp8_query, fa_abi_version); ``attention_forward``,
``attention_forward_split``, ``attention_backward`` and ``attention_forward_fp8``
are the torch-facing helpers that allocate outputs (and
workspaces) with torch and pass torch's current stream.

The library is loaded on first use; if it has not been built
(``python -m exact_attention_65_amd.build``) that use raises ImportError.
There is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

from .build import LIB_PATH

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2

FA_OK = 0
FA_ERR_NULL_POINTER = 1
FA_ERR_BAD_SHAPE = 2
FA_ERR_BAD_SCALE = 3
FA_ERR_BAD_DTYPE = 4
FA_ERR_MISALIGNED = 5
FA_ERR_ALIASING = 6
FA_ERR_UNSUPPORTED = 7
FA_ERR_HIP = 8
FA_ERR_WORKSPACE = 9

FA_SPLIT_AUTO = 0
FA_SPLIT_MAX = 256

FA_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTED = ("fa_fwd", "fa_fwd_query", "fa_fwd_split", "fa_fwd_split_query", "fa_fwd_split_static", "fa_bwd",
            "fa_bwd_query", "fa_bwd_qk", "fa_bwd_qk_query", "fa_fwd_fp8", "fa_fwd_fp8_query", "fa_status_str",
            "fa_abi_version")


class FaSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("q_bytes", "k_bytes", "v_bytes", "o_bytes", "lse_bytes", "workspace_bytes")]


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(fa_status_str(status))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m exact_attention_65_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                           ctypes.c_int, vp]
    lib.fa_fwd_query.restype = ctypes.c_int
    lib.fa_fwd_query.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(FaSizes)]
    lib.fa_fwd_split.restype = ctypes.c_int
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64,
                                 ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_fwd_split_query.restype = ctypes.c_int
    lib.fa_fwd_split_query.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(FaSizes), ctypes.POINTER(ctypes.c_int)]
    lib.fa_fwd_split_static.restype = ctypes.c_int
    lib.fa_fwd_split_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                        ctypes.c_int, ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64,
                           ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_bwd_query.restype = ctypes.c_int
    lib.fa_bwd_query.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(FaSizes)]
    lib.fa_bwd_qk.restype = ctypes.c_int
    lib.fa_bwd_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64,
                              ctypes.c_int, ctypes.c_float, ctypes.c_int, vp]
    lib.fa_bwd_qk_query.restype = ctypes.c_int
    lib.fa_bwd_qk_query.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(FaSizes)]
    lib.fa_fwd_fp8.restype = ctypes.c_int
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_float, vp]
    lib.fa_fwd_fp8_query.restype = ctypes.c_int
    lib.fa_fwd_fp8_query.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.POINTER(FaSizes)]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_abi_version.restype = ctypes.c_int
    lib.fa_abi_version.argtypes = []
    return lib


_LIB = None
library_path = LIB_PATH


def lib():
    """The loaded ctypes library (loads it on first call)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def fa_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, stream) -> int:
    """Raw C call: pointers as integers (device addresses), returns the fa_status."""
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, D, int(causal), float(scale), int(dtype), stream)


def fa_fwd_query(B, H, N, D, causal, dtype):
    """Returns (status, FaSizes)."""
    sz = FaSizes()
    st = lib().fa_fwd_query(B, H, N, D, int(causal), int(dtype), ctypes.byref(sz))
    return st, sz


def fa_fwd_split(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, D, causal, scale, n_splits,
                 dtype, stream) -> int:
    """Raw C call: pointers as integers (device addresses), returns the fa_status."""
    return lib().fa_fwd_split(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, D, int(causal),
                              float(scale), int(n_splits), int(dtype), stream)


def fa_fwd_split_static(q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale, n_splits, dtype, stream) -> int:
    """Raw C call: fa_fwd_split with the library's own scratch (no workspace argument)."""
    return lib().fa_fwd_split_static(q, k, v, o, lse, B, H, Nq, Nk, D, int(causal), float(scale), int(n_splits),
                                     int(dtype), stream)


def fa_fwd_split_query(B, H, Nq, Nk, D, causal, n_splits, dtype):
    """Returns (status, FaSizes, number of key ranges)."""
    sz = FaSizes()
    splits = ctypes.c_int(0)
    st = lib().fa_fwd_split_query(B, H, Nq, Nk, D, int(causal), int(n_splits), int(dtype), ctypes.byref(sz),
                                  ctypes.byref(splits))
    return st, sz, splits.value


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, D, causal, scale, dtype,
           stream) -> int:
    """Raw C call: pointers as integers (device addresses), returns the fa_status."""
    return lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, D, int(causal),
                        float(scale), int(dtype), stream)


def fa_bwd_query(B, H, N, D, causal, dtype):
    """Returns (status, FaSizes)."""
    sz = FaSizes()
    st = lib().fa_bwd_query(B, H, N, D, int(causal), int(dtype), ctypes.byref(sz))
    return st, sz


def fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, D, causal, scale, dtype,
              stream) -> int:
    """Raw C call: pointers as integers (device addresses), returns the fa_status."""
    return lib().fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, D,
                           int(causal), float(scale), int(dtype), stream)


def fa_bwd_qk_query(B, H, Nq, Nk, D, causal, dtype):
    """Returns (status, FaSizes)."""
    sz = FaSizes()
    st = lib().fa_bwd_qk_query(B, H, Nq, Nk, D, int(causal), int(dtype), ctypes.byref(sz))
    return st, sz


def fa_fwd_fp8(q, q_scale, k, k_scale, v, v_scale, o, lse, B, H, N, D, causal, scale, stream) -> int:
    """Raw C call: pointers as integers (device addresses), returns the fa_status."""
    return lib().fa_fwd_fp8(q, q_scale, k, k_scale, v, v_scale, o, lse, B, H, N, D, int(causal), float(scale),
                            stream)


def fa_fwd_fp8_query(B, H, N, D, causal):
    """Returns (status, FaSizes)."""
    sz = FaSizes()
    st = lib().fa_fwd_fp8_query(B, H, N, D, int(causal), ctypes.byref(sz))
    return st, sz


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def fa_abi_version() -> int:
    return lib().fa_abi_version()


def _dtype_code(dtype) -> int:
    import torch
    codes = {torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16, torch.float32: FA_DTYPE_F32}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[dtype]


def _check_given(t, name: str, shape, dtype, device) -> None:
    """A caller-supplied output or workspace tensor: the C ABI sees only its
    address, so its shape, dtype, device and layout are checked here (a tensor
    that is too small would be written past its end)."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.device != device:  # the inputs' device, a GPU (checked before)
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_workspace(t, need: int, device) -> None:
    import torch
    _check_given(t, "workspace", None, torch.uint8, device)
    if t.numel() < need:
        raise ValueError(f"workspace must hold at least {need} bytes, got {t.numel()}")


def attention_forward(q, k, v, causal: bool = False, scale: float | None = None,
                      out=None, lse=None, stream=None):
    """O, LSE = attention(q, k, v) for torch tensors [B, H, N, D] on a GPU.

    q, k, v: contiguous, same shape, dtype torch.bfloat16, torch.float16 or
    torch.float32.  Returns (o, lse): o like q, lse float32 [B, H, N].  Launches
    on ``stream`` (default: torch's current stream) and does not synchronise.
    """
    import torch
    dt = _dtype_code(q.dtype)
    for x in (q, k, v):
        if x.dtype != q.dtype or x.shape != q.shape or not x.is_cuda or not x.is_contiguous():
            raise ValueError("q, k, v must be contiguous GPU tensors of one shape and dtype")
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_given(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_given(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, N, D, causal, scale, dt, stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def attention_forward_split(q, k, v, causal: bool = False, scale: float | None = None,
                            n_splits: int = FA_SPLIT_AUTO, out=None, lse=None, workspace=None, stream=None):
    """O, LSE = attention(q, k, v) through fa_fwd_split, for bf16 or fp16 torch tensors.

    q: [B, H, Nq, D], k and v: [B, H, Nk, D] (contiguous, one dtype, on a GPU).
    Under the causal mask the queries are the last Nq positions (Nq <= Nk).
    Allocates the workspace with torch unless one (a uint8 GPU tensor) is given.
    Launches on ``stream`` (default: torch's current stream); no synchronisation.
    """
    import torch
    dt = _dtype_code(q.dtype)
    if dt == FA_DTYPE_F32:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for x in (q, k, v):
        if x.dtype != q.dtype or not x.is_cuda or not x.is_contiguous() or x.dim() != 4:
            raise ValueError("q, k, v must be contiguous 4-D GPU tensors of one dtype")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Nk, D] with q's B, H, D")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st, sz, splits = fa_fwd_split_query(B, H, Nq, Nk, D, causal, n_splits, dt)
    if st != FA_OK:
        raise FaError(st)
    if out is None:
        out = torch.empty_like(q)
    _check_given(out, "out", q.shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_given(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if workspace is None and sz.workspace_bytes > 0:
        workspace = torch.empty(sz.workspace_bytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, sz.workspace_bytes, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes,
                      B, H, Nq, Nk, D, causal, scale, n_splits, dt, stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                       dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dq, dk, dv of the forward's o for the upstream gradient dout.

    q, o, dout: contiguous bf16 or fp16 GPU tensors [B, H, Nq, D]; k, v:
    [B, H, Nk, D] of the same dtype (the gradients have it too).  o and lse as
    attention_forward (Nq = Nk, fa_bwd) or attention_forward_split (fa_bwd_qk)
    returned them for the same q, k, v, causal and scale.  Allocates the
    gradients (and the workspace, unless a uint8 GPU tensor is given) with
    torch.  Launches on ``stream`` (default: torch's current stream); no
    synchronisation.
    """
    import torch
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"unsupported dtype {q.dtype}")
    dt = _dtype_code(q.dtype)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v, o, dout must be 4-d [B, H, N, D] tensors")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    for x, shape in ((q, (B, H, Nq, D)), (o, (B, H, Nq, D)), (dout, (B, H, Nq, D)), (k, (B, H, Nk, D)),
                     (v, (B, H, Nk, D))):
        if x.dtype != q.dtype or tuple(x.shape) != shape or not x.is_cuda or not x.is_contiguous():
            raise ValueError("q, o, dout [B, H, Nq, D] and k, v [B, H, Nk, D] must be contiguous GPU tensors "
                             "of one dtype")
    _check_given(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    square = Nq == Nk
    st, sz = fa_bwd_query(B, H, Nq, D, causal, dt) if square else fa_bwd_qk_query(B, H, Nq, Nk, D, causal, dt)
    if st != FA_OK:
        raise FaError(st)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name, like in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _check_given(t, name, like.shape, q.dtype, q.device)
    if workspace is None:
        workspace = torch.empty(sz.workspace_bytes, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, sz.workspace_bytes, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size())
    if square:
        st = fa_bwd(*ptrs, B, H, Nq, D, causal, scale, dt, stream.cuda_stream)
    else:
        st = fa_bwd_qk(*ptrs, B, H, Nq, Nk, D, causal, scale, dt, stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def attention_forward_fp8(q, q_scale, k, k_scale, v, v_scale, causal: bool = False, scale: float | None = None,
                          out=None, lse=None, stream=None):
    """O (bf16), LSE of FP8 inputs with MX block scales, for torch tensors on a GPU.

    q, k, v: contiguous uint8 [B, H, N, D] E4M3 codes; q_scale, k_scale, v_scale:
    contiguous uint8 [B, H, N, D/32] E8M0 codes.  Launches on ``stream``
    (default: torch's current stream) and does not synchronise.
    """
    import torch
    B, H, N, D = q.shape
    for x in (q, k, v):
        if x.dtype != torch.uint8 or x.shape != q.shape or not x.is_cuda or not x.is_contiguous():
            raise ValueError("q, k, v must be contiguous uint8 GPU tensors of one shape")
    for x in (q_scale, k_scale, v_scale):
        if x.dtype != torch.uint8 or x.shape != (B, H, N, D // 32) or not x.is_cuda or not x.is_contiguous():
            raise ValueError("scales must be contiguous uint8 GPU tensors [B, H, N, D/32]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q.device)
    _check_given(out, "out", (B, H, N, D), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_given(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd_fp8(q.data_ptr(), q_scale.data_ptr(), k.data_ptr(), k_scale.data_ptr(), v.data_ptr(),
                    v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, D, causal, scale,
                    stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
