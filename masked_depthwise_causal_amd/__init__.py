"""Masked causal depthwise conv1d backward on MI355X (gfx950).

Python binding over the C-ABI of ``libmccb.so`` (``include/mccb.h``). This layer only marshals
arguments: every step of the computation runs in the library's HIP kernels. PyTorch is used for
device memory and streams.

The operation is the one on the page "aclnnMaskedCausalConv1dBackward", section 功能说明
(function description): gradX and gradWeight of a depthwise causal conv1d over [S,B,H] tensors with a
[3,H] weight and an optional [B,S] bool mask. ``forward`` runs that conv itself (the
MaskedCausalConv1d operator the page names beside the backward).
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import MccbError, Plan, Strides, lib, status_string  # noqa: F401

MCCB_BF16, MCCB_FP16 = 0, 1
MCCB_OK = 0
MCCB_ERR_PARAM_NULLPTR = 161001
MCCB_ERR_PARAM_INVALID = 161002
MCCB_ERR_SHAPE = 561002
MCCB_ERR_RUNTIME = -1
MCCB_ERR_SCRATCH_LIMIT = -2
MCCB_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed scratch of mccb_backward_noalloc (mccb.h)

DTYPE_CODE = {torch.bfloat16: MCCB_BF16, torch.float16: MCCB_FP16}


# -- same names and arguments as the C-ABI -----------------------------------------------------------
def mccb_get_workspace_size(S: int, B: int, H: int, dtype: int) -> int:
    out = ctypes.c_uint64(0)
    rc = lib().mccb_get_workspace_size(S, B, H, dtype, ctypes.byref(out))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_get_workspace_size")
    return int(out.value)


def mccb_get_plan(S: int, B: int, H: int, dtype: int) -> dict:
    p = Plan()
    rc = lib().mccb_get_plan(S, B, H, dtype, ctypes.byref(p))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_get_plan")
    return {name: int(getattr(p, name)) for name, _ in Plan._fields_}


def mccb_backward(gradY: int, x: int, weight: int, mask: int | None, gradX: int, gradWeight: int,
                  S: int, B: int, H: int, dtype: int, workspace: int | None, workspace_size: int,
                  stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_backward(gradY, x, weight, mask, gradX, gradWeight, S, B, H, dtype,
                                   workspace, workspace_size, stream))


def mccb_backward_noalloc(gradY: int, x: int, weight: int, mask: int | None, gradX: int,
                          gradWeight: int, S: int, B: int, H: int, dtype: int,
                          stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_backward_noalloc(gradY, x, weight, mask, gradX, gradWeight, S, B, H,
                                           dtype, stream))


def mccb_forward(x: int, weight: int, mask: int | None, y: int, S: int, B: int, H: int, dtype: int,
                 stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_forward(x, weight, mask, y, S, B, H, dtype, stream))


def mccb_get_workspace_size_ex(gradY: int, x: int, weight: int, S: int, B: int, H: int, W: int,
                               dtype: int, strides: Strides | None) -> int:
    out = ctypes.c_uint64(0)
    rc = lib().mccb_get_workspace_size_ex(gradY, x, weight, S, B, H, W, dtype,
                                          None if strides is None else ctypes.byref(strides),
                                          ctypes.byref(out))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_get_workspace_size_ex")
    return int(out.value)


def mccb_backward_ex(gradY: int, x: int, weight: int, mask: int | None, gradX: int,
                     gradWeight: int, S: int, B: int, H: int, W: int, dtype: int,
                     strides: Strides | None, workspace: int | None, workspace_size: int,
                     stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_backward_ex(gradY, x, weight, mask, gradX, gradWeight, S, B, H, W, dtype,
                                      None if strides is None else ctypes.byref(strides),
                                      workspace, workspace_size, stream))


def mccb_forward_get_workspace_size_ex(x: int, weight: int, S: int, B: int, H: int, W: int,
                                       dtype: int, strides: Strides | None) -> int:
    out = ctypes.c_uint64(0)
    rc = lib().mccb_forward_get_workspace_size_ex(
        x, weight, S, B, H, W, dtype, None if strides is None else ctypes.byref(strides),
        ctypes.byref(out))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_forward_get_workspace_size_ex")
    return int(out.value)


def mccb_forward_ex(x: int, weight: int, mask: int | None, y: int, S: int, B: int, H: int, W: int,
                    dtype: int, strides: Strides | None, workspace: int | None,
                    workspace_size: int, stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_forward_ex(x, weight, mask, y, S, B, H, W, dtype,
                                     None if strides is None else ctypes.byref(strides),
                                     workspace, workspace_size, stream))


def mccb_varlen_get_workspace_size(T: int, nseq: int, H: int, W: int, dtype: int) -> int:
    out = ctypes.c_uint64(0)
    rc = lib().mccb_varlen_get_workspace_size(T, nseq, H, W, dtype, ctypes.byref(out))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_varlen_get_workspace_size")
    return int(out.value)


def mccb_varlen_backward(gradY: int, x: int, weight: int, mask: int | None, cu_seqlens: int,
                         gradX: int, gradWeight: int, T: int, nseq: int, H: int, W: int,
                         dtype: int, workspace: int | None, workspace_size: int,
                         stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_varlen_backward(gradY, x, weight, mask, cu_seqlens, gradX, gradWeight,
                                          T, nseq, H, W, dtype, workspace, workspace_size, stream))


def mccb_varlen_forward_get_workspace_size(T: int, nseq: int, H: int, W: int, dtype: int) -> int:
    out = ctypes.c_uint64(0)
    rc = lib().mccb_varlen_forward_get_workspace_size(T, nseq, H, W, dtype, ctypes.byref(out))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_varlen_forward_get_workspace_size")
    return int(out.value)


def mccb_varlen_forward(x: int, weight: int, mask: int | None, cu_seqlens: int, y: int, T: int,
                        nseq: int, H: int, W: int, dtype: int, workspace: int | None,
                        workspace_size: int, stream: int | None) -> int:
    """Raw call with integer device addresses; returns the status code (does not raise)."""
    return int(lib().mccb_varlen_forward(x, weight, mask, cu_seqlens, y, T, nseq, H, W, dtype,
                                         workspace, workspace_size, stream))


def mccb_status_string(status: int) -> str:
    return status_string(status)


def mccb_profile_begin(max_calls: int) -> None:
    rc = lib().mccb_profile_begin(max_calls)
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_profile_begin")


def mccb_profile_end() -> tuple[float, float, int]:
    """(summed fused-kernel ms, summed reduce-kernel ms, calls recorded)."""
    f, r, n = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_int(0)
    rc = lib().mccb_profile_end(ctypes.byref(f), ctypes.byref(r), ctypes.byref(n))
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_profile_end")
    return float(f.value), float(r.value), int(n.value)


# -- tensor front end ---------------------------------------------------------------------------------
def _check_tensor(name, t, shape, dtype, device, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must live on {device} (a HIP device)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not contiguous and any(st < 0 for st in t.stride()):
        raise ValueError(f"{name} has a negative stride")


def _strides(gradY, x, weight, mask) -> Strides | None:
    """mccb_strides_t of the inputs, or None when every input is contiguous."""
    ts = [t for t in (gradY, x, weight, mask) if t is not None]
    if all(t.is_contiguous() for t in ts):
        return None
    st = Strides()
    if gradY is not None:
        st.gradY[:] = list(gradY.stride())
    else:
        st.gradY[:] = list(x.stride())
    st.x[:] = list(x.stride())
    st.weight[:] = list(weight.stride())
    S, B = int(x.shape[0]), int(x.shape[1])
    st.mask[:] = list(mask.stride()) if mask is not None else [S, 1]
    return st


def _ws_bytes(workspace: torch.Tensor, device) -> int:
    """Size in bytes of a caller's workspace tensor (any dtype), which must be contiguous device
    memory on the tensors' device."""
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace.numel() * workspace.element_size()


def workspace_for(S: int, B: int, H: int, dtype: torch.dtype, device) -> torch.Tensor:
    n = mccb_get_workspace_size(S, B, H, DTYPE_CODE[dtype])
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def backward(gradY: torch.Tensor, x: torch.Tensor, weight: torch.Tensor,
             mask: torch.Tensor | None = None, gradX: torch.Tensor | None = None,
             gradWeight: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             stream: torch.cuda.Stream | None = None):
    """gradX [S,B,H], gradWeight [W,H] on device tensors (outputs allocated if None); the window W
    is the weight's first dimension (3 on the page; 1..4 accepted).

    The inputs may be strided views (mccb_backward_ex); the outputs must be contiguous. Enqueues
    on `stream` (default: torch's current stream) and returns without synchronizing.
    """
    if gradY.dim() != 3:
        raise ValueError("gradY must be [S,B,H]")
    S, B, H = (int(s) for s in gradY.shape)
    dev = gradY.device
    dt = gradY.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"dtype {dt} not supported (bfloat16, float16)")
    _check_tensor("gradY", gradY, (S, B, H), dt, dev, contiguous=False)
    _check_tensor("x", x, (S, B, H), dt, dev, contiguous=False)
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a [W,H] tensor")
    W = int(weight.shape[0])
    _check_tensor("weight", weight, (W, H), dt, dev, contiguous=False)
    if mask is not None:
        _check_tensor("mask", mask, (B, S), None, dev, contiguous=False)
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be bool or uint8")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    # Buffers this call allocates belong to the stream the kernels run on, so that torch's caching
    # allocator does not hand them to other work before those kernels finish.
    with torch.cuda.stream(st):
        if gradX is None:
            gradX = torch.empty((S, B, H), dtype=dt, device=dev)
        if gradWeight is None:
            gradWeight = torch.empty((W, H), dtype=dt, device=dev)
    _check_tensor("gradX", gradX, (S, B, H), dt, dev)
    _check_tensor("gradWeight", gradWeight, (W, H), dt, dev)
    strides = _strides(gradY, x, weight, mask)
    mptr = None if mask is None else mask.data_ptr()
    if strides is None and W == 3:
        if workspace is None:
            with torch.cuda.stream(st):
                workspace = workspace_for(S, B, H, dt, dev)
        rc = mccb_backward(gradY.data_ptr(), x.data_ptr(), weight.data_ptr(), mptr,
                           gradX.data_ptr(), gradWeight.data_ptr(), S, B, H, DTYPE_CODE[dt],
                           workspace.data_ptr(), _ws_bytes(workspace, dev), st.cuda_stream)
        where = "mccb_backward"
    else:
        if workspace is None:
            n = mccb_get_workspace_size_ex(gradY.data_ptr(), x.data_ptr(), weight.data_ptr(), S, B,
                                           H, W, DTYPE_CODE[dt], strides)
            with torch.cuda.stream(st):
                workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        rc = mccb_backward_ex(gradY.data_ptr(), x.data_ptr(), weight.data_ptr(), mptr,
                              gradX.data_ptr(), gradWeight.data_ptr(), S, B, H, W, DTYPE_CODE[dt],
                              strides, workspace.data_ptr(), _ws_bytes(workspace, dev),
                              st.cuda_stream)
        where = "mccb_backward_ex"
    if rc != MCCB_OK:
        raise MccbError(rc, where)
    return gradX, gradWeight


def backward_noalloc(gradY: torch.Tensor, x: torch.Tensor, weight: torch.Tensor,
                     mask: torch.Tensor | None, gradX: torch.Tensor, gradWeight: torch.Tensor,
                     stream: torch.cuda.Stream | None = None):
    """mccb_backward_noalloc on contiguous device tensors: the caller passes both outputs and no
    workspace, and nothing is allocated (the library's fixed device scratch holds the gradWeight
    partials). 3-tap window only. Enqueues on `stream` (default: torch's current stream)."""
    if gradY.dim() != 3:
        raise ValueError("gradY must be [S,B,H]")
    S, B, H = (int(s) for s in gradY.shape)
    dev, dt = gradY.device, gradY.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"dtype {dt} not supported (bfloat16, float16)")
    _check_tensor("gradY", gradY, (S, B, H), dt, dev)
    _check_tensor("x", x, (S, B, H), dt, dev)
    _check_tensor("weight", weight, (3, H), dt, dev)
    if mask is not None:
        _check_tensor("mask", mask, (B, S), None, dev)
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be bool or uint8")
    _check_tensor("gradX", gradX, (S, B, H), dt, dev)
    _check_tensor("gradWeight", gradWeight, (3, H), dt, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = mccb_backward_noalloc(gradY.data_ptr(), x.data_ptr(), weight.data_ptr(),
                               None if mask is None else mask.data_ptr(), gradX.data_ptr(),
                               gradWeight.data_ptr(), S, B, H, DTYPE_CODE[dt], st.cuda_stream)
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_backward_noalloc")
    return gradX, gradWeight


def forward(x: torch.Tensor, weight: torch.Tensor, mask: torch.Tensor | None = None,
            y: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None,
            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [S,B,H] = mask * causal depthwise conv(x, weight) on device tensors (y allocated if
    None); the window W is the weight's first dimension (3 on the page; 1..4 accepted). The inputs
    may be strided views (mccb_forward_ex); y must be contiguous. Enqueues on `stream` (default:
    torch's current stream) without synchronizing."""
    if x.dim() != 3:
        raise ValueError("x must be [S,B,H]")
    S, B, H = (int(s) for s in x.shape)
    dev, dt = x.device, x.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"dtype {dt} not supported (bfloat16, float16)")
    _check_tensor("x", x, (S, B, H), dt, dev, contiguous=False)
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a [W,H] tensor")
    W = int(weight.shape[0])
    _check_tensor("weight", weight, (W, H), dt, dev, contiguous=False)
    if mask is not None:
        _check_tensor("mask", mask, (B, S), None, dev, contiguous=False)
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be bool or uint8")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    if y is None:
        with torch.cuda.stream(st):  # allocated for the stream the kernel runs on
            y = torch.empty((S, B, H), dtype=dt, device=dev)
    _check_tensor("y", y, (S, B, H), dt, dev)
    strides = _strides(None, x, weight, mask)
    mptr = None if mask is None else mask.data_ptr()
    if strides is None and W == 3:
        rc = mccb_forward(x.data_ptr(), weight.data_ptr(), mptr, y.data_ptr(), S, B, H,
                          DTYPE_CODE[dt], st.cuda_stream)
        where = "mccb_forward"
    else:
        if workspace is None:
            n = mccb_forward_get_workspace_size_ex(x.data_ptr(), weight.data_ptr(), S, B, H, W,
                                                   DTYPE_CODE[dt], strides)
            with torch.cuda.stream(st):
                workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        rc = mccb_forward_ex(x.data_ptr(), weight.data_ptr(), mptr, y.data_ptr(), S, B, H, W,
                             DTYPE_CODE[dt], strides, workspace.data_ptr(),
                             _ws_bytes(workspace, dev), st.cuda_stream)
        where = "mccb_forward_ex"
    if rc != MCCB_OK:
        raise MccbError(rc, where)
    return y


def _varlen_args(x, weight, cu_seqlens, mask):
    if x.dim() != 2:
        raise ValueError("packed tensors are [T,H]")
    T, H = (int(v) for v in x.shape)
    dev, dt = x.device, x.dtype
    if dt not in DTYPE_CODE:
        raise ValueError(f"dtype {dt} not supported (bfloat16, float16)")
    _check_tensor("x", x, (T, H), dt, dev)
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be a [W,H] tensor")
    W = int(weight.shape[0])
    _check_tensor("weight", weight, (W, H), dt, dev)
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor of cumulative sequence ends")
    _check_tensor("cu_seqlens", cu_seqlens, (int(cu_seqlens.shape[0]),), torch.int64, dev)
    if mask is not None:
        _check_tensor("mask", mask, (T,), None, dev)
        if mask.dtype not in (torch.bool, torch.uint8):
            raise ValueError("mask must be bool or uint8")
    return T, H, W, int(cu_seqlens.shape[0]), dev, dt


def varlen_backward(gradY: torch.Tensor, x: torch.Tensor, weight: torch.Tensor,
                    cu_seqlens: torch.Tensor, mask: torch.Tensor | None = None,
                    gradX: torch.Tensor | None = None, gradWeight: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None,
                    stream: torch.cuda.Stream | None = None):
    """Packed variable-length layout: gradX [T,H], gradWeight [W,H] from gradY, x [T,H], the
    weight [W,H] and the int64 cumulative sequence ends (device). Enqueues without
    synchronizing."""
    T, H, W, nseq, dev, dt = _varlen_args(x, weight, cu_seqlens, mask)
    _check_tensor("gradY", gradY, (T, H), dt, dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(st):  # what this call allocates belongs to the kernels' stream
        if gradX is None:
            gradX = torch.empty((T, H), dtype=dt, device=dev)
        if gradWeight is None:
            gradWeight = torch.empty((W, H), dtype=dt, device=dev)
        if workspace is None:
            n = mccb_varlen_get_workspace_size(T, nseq, H, W, DTYPE_CODE[dt])
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check_tensor("gradX", gradX, (T, H), dt, dev)
    _check_tensor("gradWeight", gradWeight, (W, H), dt, dev)
    rc = mccb_varlen_backward(gradY.data_ptr(), x.data_ptr(), weight.data_ptr(),
                              None if mask is None else mask.data_ptr(), cu_seqlens.data_ptr(),
                              gradX.data_ptr(), gradWeight.data_ptr(), T, nseq, H, W,
                              DTYPE_CODE[dt], workspace.data_ptr(), _ws_bytes(workspace, dev),
                              st.cuda_stream)
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_varlen_backward")
    return gradX, gradWeight


def varlen_forward(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor,
                   mask: torch.Tensor | None = None, y: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None,
                   stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Packed variable-length layout: y [T,H] = mask * causal depthwise conv(x, weight) within
    each sequence. Enqueues without synchronizing."""
    T, H, W, nseq, dev, dt = _varlen_args(x, weight, cu_seqlens, mask)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(st):  # what this call allocates belongs to the kernel's stream
        if y is None:
            y = torch.empty((T, H), dtype=dt, device=dev)
        if workspace is None:
            n = mccb_varlen_forward_get_workspace_size(T, nseq, H, W, DTYPE_CODE[dt])
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check_tensor("y", y, (T, H), dt, dev)
    rc = mccb_varlen_forward(x.data_ptr(), weight.data_ptr(),
                             None if mask is None else mask.data_ptr(), cu_seqlens.data_ptr(),
                             y.data_ptr(), T, nseq, H, W, DTYPE_CODE[dt], workspace.data_ptr(),
                             _ws_bytes(workspace, dev), st.cuda_stream)
    if rc != MCCB_OK:
        raise MccbError(rc, "mccb_varlen_forward")
    return y
