"""ctypes binding of the causal-conv1d entry points of libssd_bwd.so (include/causal_conv1d.h).

Argument marshalling only: shapes and dtypes are checked, outputs and the
workspace are allocated with torch on the inputs' device, and the C entry
point is called on the current HIP stream.  Every arithmetic step runs in the
library's kernels; the calls raise if the library is missing or returns an
error.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from state_space_model_mamba_amd import ssd

CONV1D_ACT_NONE, CONV1D_ACT_SILU = 0, 1
ACTIVATIONS = {"none": CONV1D_ACT_NONE, "silu": CONV1D_ACT_SILU}
EXPORTED = ("conv1d_fwd", "conv1d_bwd", "conv1d_bwd_workspace_size")


class Conv1dShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("width", ctypes.c_int32), ("activation", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_ready = False


def load_library():
    """The shared library with the conv entry points' argument types set (raises if it is not built)."""
    global _ready
    lib = ssd.load_library()
    if not _ready:
        vp = ctypes.c_void_p
        sp = ctypes.POINTER(Conv1dShape)
        lib.conv1d_fwd.restype = ctypes.c_int
        lib.conv1d_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        lib.conv1d_bwd_workspace_size.restype = ctypes.c_int
        lib.conv1d_bwd_workspace_size.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        lib.conv1d_bwd.restype = ctypes.c_int
        lib.conv1d_bwd.argtypes = [sp] + [vp] * 9 + [ctypes.c_size_t, vp]
        _ready = True
    return lib


def make_shape(batch, seqlen, channels, width, activation="silu", io_dtype=ssd.SSD_IO_BF16) -> Conv1dShape:
    act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    return Conv1dShape(batch, seqlen, channels, width, act, io_dtype, 0)


def workspace_size(shape: Conv1dShape) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().conv1d_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if rc:
        raise ssd.SsdError(rc, "conv1d_bwd_workspace_size")
    return n.value


def _shape(x, weight, activation):
    if x.device.type != "cuda":
        raise ValueError("causal conv1d runs on a HIP device; got tensors on " + str(x.device))
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported io dtype {x.dtype}")
    b, L, C = x.shape
    W = weight.shape[1]
    io = ssd.SSD_IO_BF16 if x.dtype == torch.bfloat16 else ssd.SSD_IO_F32
    return make_shape(b, L, C, W, activation, io)


def _check_common(x, weight, bias, seq_idx):
    b, L, C = x.shape
    dev = x.device
    ssd._check(x, "x", x.dtype, (b, L, C), dev)
    ssd._check(weight, "weight", torch.float32, (C, weight.shape[1]), dev)
    ssd._check(bias, "bias", torch.float32, (C,), dev)
    ssd._check(seq_idx, "seq_idx", torch.int32, (b, L), dev)


def conv1d_fwd(x, weight, bias=None, seq_idx=None, activation: str = "silu", out=None):
    """act(bias + causal depthwise conv of x with weight), x: (batch, seqlen, channels) channels-last."""
    lib = load_library()
    shape = _shape(x, weight, activation)
    _check_common(x, weight, bias, seq_idx)
    if out is None:
        out = torch.empty_like(x)
    ssd._check(out, "out", x.dtype, tuple(x.shape), x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = lib.conv1d_fwd(ctypes.byref(shape), ssd._ptr(x), ssd._ptr(weight), ssd._ptr(bias), ssd._ptr(seq_idx),
                        ssd._ptr(out), ctypes.c_void_p(stream))
    if rc:
        raise ssd.SsdError(rc, "conv1d_fwd")
    return out


def conv1d_bwd(x, weight, bias, seq_idx, dout, activation: str = "silu", workspace: Optional[torch.Tensor] = None,
               out: Optional[dict] = None):
    """dict of dx (like x), dweight (like weight), dbias (like bias, or None without bias)."""
    lib = load_library()
    shape = _shape(x, weight, activation)
    _check_common(x, weight, bias, seq_idx)
    ssd._check(dout, "dout", x.dtype, tuple(x.shape), x.device)
    nbytes = workspace_size(shape)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = {"dx": torch.empty_like(x), "dweight": torch.empty_like(weight),
               "dbias": torch.empty_like(bias) if bias is not None else None}
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = lib.conv1d_bwd(ctypes.byref(shape), ssd._ptr(x), ssd._ptr(weight), ssd._ptr(bias), ssd._ptr(seq_idx),
                        ssd._ptr(dout), ssd._ptr(out["dx"]), ssd._ptr(out["dweight"]), ssd._ptr(out["dbias"]),
                        ssd._ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if rc:
        raise ssd.SsdError(rc, "conv1d_bwd")
    return out


class CausalConv1d(torch.autograd.Function):
    """y = conv1d_fwd(...); backward through conv1d_bwd (deterministic)."""

    @staticmethod
    def forward(ctx, x, weight, bias, seq_idx, activation):
        ctx.save_for_backward(x, weight, bias, seq_idx)
        ctx.activation = activation
        return conv1d_fwd(x, weight, bias, seq_idx, activation)

    @staticmethod
    def backward(ctx, dy):
        x, weight, bias, seq_idx = ctx.saved_tensors
        g = conv1d_bwd(x, weight, bias, seq_idx, dy.contiguous(), ctx.activation)
        return g["dx"], g["dweight"], g["dbias"], None, None


def causal_conv1d(x, weight, bias=None, seq_idx=None, activation: str = "silu"):
    """Autograd-aware causal depthwise convolution (channels-last x)."""
    return CausalConv1d.apply(x, weight, bias, seq_idx, activation)
