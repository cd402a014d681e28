"""ctypes binding of libssd_bwd.so (see include/ssd_bwd.h).

Argument marshalling only: shapes/dtypes are checked, outputs and the
workspace are allocated with torch on the inputs' device, and the C entry
point is called on the current HIP stream.  Every arithmetic step runs in the
library's kernels.  Raises if the library is missing or returns an error.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libssd_bwd.so")

SSD_IO_BF16 = 0
SSD_IO_F32 = 1
SSD_WS_ACS, SSD_WS_HIN, SSD_WS_DSTATE = 0, 1, 2

EXPORTED = ("ssd_bwd", "ssd_bwd_workspace_size", "ssd_bwd_workspace_region", "ssd_status_string",
            "ssd_bwd_version", "ssd_bwd_profiled", "ssd_bwd_stage_count", "ssd_bwd_stage_name", "ssd_fwd",
            "ssd_fwd_ex", "ssd_bwd_ex", "ssd_set_launch_geometry", "ssd_bwd_noalloc", "ssd_set_group_path")
# bytes of the library's own device workspace used by ssd_bwd_noalloc (SSD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class SsdShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("chunk_size", ctypes.c_int64), ("nseqs", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SsdOptions(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int32),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float), ("d_per_channel", ctypes.c_int32),
                ("d_last_states", ctypes.c_void_p), ("y_pre_gate", ctypes.c_void_p)]


class SsdError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library(path: str = LIBRARY):
    """Load libssd_bwd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m state_space_model_mamba_amd.build`")
    lib = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    sp = ctypes.POINTER(SsdShape)
    lib.ssd_bwd_workspace_size.restype = ctypes.c_int
    lib.ssd_bwd_workspace_size.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_bwd_workspace_region.restype = ctypes.c_int
    lib.ssd_bwd_workspace_region.argtypes = [sp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_bwd_version.restype = ctypes.c_int
    lib.ssd_bwd_version.argtypes = []
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_bwd.argtypes = [sp] + [vp] * 17 + [ctypes.c_size_t, vp]
    lib.ssd_bwd_profiled.restype = ctypes.c_int
    lib.ssd_bwd_profiled.argtypes = [sp] + [vp] * 17 + [ctypes.c_size_t, vp, ctypes.POINTER(vp)]
    lib.ssd_fwd.restype = ctypes.c_int
    lib.ssd_fwd.argtypes = [sp] + [vp] * 10 + [vp, ctypes.c_size_t, vp]
    fp = ctypes.POINTER(SsdOptions)
    lib.ssd_fwd_ex.restype = ctypes.c_int
    lib.ssd_fwd_ex.argtypes = [sp, fp] + [vp] * 11 + [vp, ctypes.c_size_t, vp]
    lib.ssd_bwd_ex.restype = ctypes.c_int
    lib.ssd_bwd_ex.argtypes = [sp, fp] + [vp] * 20 + [ctypes.c_size_t, vp]
    lib.ssd_bwd_stage_count.restype = ctypes.c_int
    lib.ssd_bwd_stage_count.argtypes = []
    lib.ssd_bwd_stage_name.restype = ctypes.c_char_p
    lib.ssd_bwd_stage_name.argtypes = [ctypes.c_int]
    lib.ssd_bwd_noalloc.restype = ctypes.c_int
    lib.ssd_bwd_noalloc.argtypes = [sp] + [vp] * 17
    lib.ssd_set_group_path.restype = ctypes.c_int
    lib.ssd_set_group_path.argtypes = [ctypes.c_int]
    lib.ssd_set_launch_geometry.restype = ctypes.c_int
    lib.ssd_set_launch_geometry.argtypes = [ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(status).decode()


def make_shape(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size, nseqs, io_dtype) -> SsdShape:
    return SsdShape(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size, nseqs, io_dtype, 0)


def workspace_size(shape: SsdShape) -> int:
    n = ctypes.c_size_t(0)
    rc = load_library().ssd_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n))
    if rc:
        raise SsdError(rc, "ssd_bwd_workspace_size")
    return n.value


def workspace_region(shape: SsdShape, region: int) -> tuple[int, int]:
    off = ctypes.c_size_t(0)
    nb = ctypes.c_size_t(0)
    rc = load_library().ssd_bwd_workspace_region(ctypes.byref(shape), region, ctypes.byref(off),
                                                 ctypes.byref(nb))
    if rc:
        raise SsdError(rc, "ssd_bwd_workspace_region")
    return off.value, nb.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _options(dt_bias, dt_softplus, dt_limit, D, H, P, dev, d_last=None, y_pre=None):
    """The C options struct (dt front-end, per-channel D, last-state gradient, saved pre-gate
    output), or None when it would change nothing."""
    lo, hi = float(dt_limit[0]), float(dt_limit[1])
    per_channel = D is not None and D.dim() == 2
    _check(D, "D", torch.float32, (H, P) if per_channel else (H,), dev)
    if (dt_bias is None and not dt_softplus and lo == -math.inf and hi == math.inf and not per_channel
            and d_last is None and y_pre is None):
        return None
    _check(dt_bias, "dt_bias", torch.float32, (H,), dev)
    return SsdOptions(_ptr(dt_bias), 1 if dt_softplus else 0, lo, hi, 1 if per_channel else 0, _ptr(d_last),
                      _ptr(y_pre))


def shape_of(x, B, chunk_size, nseqs) -> SsdShape:
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = SSD_IO_BF16 if x.dtype == torch.bfloat16 else SSD_IO_F32
    return make_shape(b, L, H, P, G, N, chunk_size, nseqs, io)


def ssd_bwd(x, dt, A, B, C, D, dy, initial_states=None, seq_idx=None, chunk_size: int = 256,
            nseqs: Optional[int] = None, want_d_initial_states: bool = True,
            workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None, events=None,
            dt_bias=None, dt_softplus: bool = False, dt_limit=(-math.inf, math.inf), z=None,
            d_last_states=None, y_pre_gate=None):
    """Gradients of sum(dy * y) of the SSD layer, computed by libssd_bwd.

    x, dy: (b, L, H, P) and B, C: (b, L, G, N) in bf16 or fp32 (one dtype);
    dt: (b, L, H), A: (H,), D: (H,) or (H, P) (per channel), initial_states: (S, H, P, N) fp32 or None,
    seq_idx: (b, L) int32 or None.  ``nseqs`` (the number of sequence starts)
    is needed only when seq_idx is given without initial_states.
    Returns a dict with dx, ddt, dA, dB, dC, dD, d_initial_states.
    ``events``: optional list of stage_count() + 1 recorded torch.cuda.Event
    (timing enabled) handed to the profiling entry point.
    ``dt_bias`` (H,) fp32, ``dt_softplus`` and ``dt_limit`` = (min, max): the dt
    front-end of include/ssd_bwd.h (dt is then the raw input); with dt_bias the
    dict also holds ddt_bias.  ``z`` (like x): the output gate; dy is then the
    gradient of y * silu(z) and the dict also holds dz.  ``d_last_states``
    (b, H, P, N) fp32: the gradient handed in for the state after each row's
    last position (the hand-off of a sequence split across calls).
    ``y_pre_gate`` (like x, with z): y before the gate as ssd_fwd saved it; the
    gate pass then reads it instead of recomputing y (same bits).
    """
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_bwd runs on a HIP device; got tensors on " + str(dev))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = x.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported io dtype {io}")
    if initial_states is not None:
        S = initial_states.shape[0]
    elif seq_idx is None:
        S = b
    else:
        if nseqs is None and want_d_initial_states:
            raise ValueError("pass nseqs (number of sequence starts) with seq_idx")
        S = nseqs or 0
    _check(x, "x", io, (b, L, H, P), dev)
    _check(dy, "dy", io, (b, L, H, P), dev)
    _check(B, "B", io, (b, L, G, N), dev)
    _check(C, "C", io, (b, L, G, N), dev)
    _check(dt, "dt", torch.float32, (b, L, H), dev)
    _check(A, "A", torch.float32, (H,), dev)
    _check(initial_states, "initial_states", torch.float32, (S, H, P, N), dev)
    _check(seq_idx, "seq_idx", torch.int32, (b, L), dev)
    _check(d_last_states, "d_last_states", torch.float32, (b, H, P, N), dev)
    _check(z, "z", io, (b, L, H, P), dev)
    if y_pre_gate is not None:
        if z is None:
            raise ValueError("y_pre_gate goes with the gate z")
        _check(y_pre_gate, "y_pre_gate", io, (b, L, H, P), dev)
    fe = _options(dt_bias, dt_softplus, dt_limit, D, H, P, dev, d_last_states, y_pre_gate)
    if (fe is not None or z is not None) and events is not None:
        raise ValueError("stage events are not available with the dt front-end or the gate")
    shape = make_shape(b, L, H, P, G, N, chunk_size, S, SSD_IO_BF16 if io == torch.bfloat16 else SSD_IO_F32)
    nbytes = workspace_size(shape)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = {
            "dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
            "dA": torch.empty((H,), dtype=torch.float32, device=dev),
            "dB": torch.empty_like(B), "dC": torch.empty_like(C),
            "dD": torch.empty(tuple(D.shape), dtype=torch.float32, device=dev) if D is not None else None,
            "d_initial_states": (torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
                                 if want_d_initial_states and S > 0 else None),
        }
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dy),
            _ptr(initial_states), _ptr(seq_idx), _ptr(out["dx"]), _ptr(out["ddt"]),
            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
            _ptr(out["d_initial_states"]), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            ctypes.c_void_p(stream)]
    if fe is not None or z is not None:
        if dt_bias is not None and out.get("ddt_bias") is None:
            out["ddt_bias"] = torch.empty((H,), dtype=torch.float32, device=dev)
        if z is not None and out.get("dz") is None:
            out["dz"] = torch.empty_like(z)
        rc = lib.ssd_bwd_ex(args[0], ctypes.byref(fe) if fe is not None else None, *args[1:7], _ptr(z),
                            *args[7:17], _ptr(out.get("ddt_bias")), _ptr(out.get("dz")), *args[17:])
    elif events is None:
        rc = lib.ssd_bwd(*args)
    else:
        handles = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        rc = lib.ssd_bwd_profiled(*args, handles)
    if rc:
        raise SsdError(rc, "ssd_bwd")
    res = dict(out)
    res["workspace"] = workspace
    res["shape"] = shape
    return res


def ssd_bwd_noalloc(x, dt, A, B, C, D, dy, out: dict, initial_states=None, seq_idx=None,
                    chunk_size: int = 256, nseqs: Optional[int] = None):
    """ssd_bwd through the entry point that allocates nothing (its workspace is the library's
    fixed device array, see include/ssd_bwd.h): the caller passes the outputs in ``out``
    (dx, ddt, dA, dB, dC, and dD / d_initial_states or None), shaped as ssd_bwd returns them.
    Calls on one device share that array and must not overlap."""
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_bwd_noalloc runs on a HIP device; got tensors on " + str(dev))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = x.dtype
    S = initial_states.shape[0] if initial_states is not None else (b if seq_idx is None else (nseqs or 0))
    for t, name, dtype, shp in ((x, "x", io, (b, L, H, P)), (dy, "dy", io, (b, L, H, P)), (B, "B", io, (b, L, G, N)),
                                (C, "C", io, (b, L, G, N)), (dt, "dt", torch.float32, (b, L, H)),
                                (A, "A", torch.float32, (H,)), (D, "D", torch.float32, (H,)),
                                (initial_states, "initial_states", torch.float32, (S, H, P, N)),
                                (seq_idx, "seq_idx", torch.int32, (b, L)),
                                (out["dx"], "dx", io, (b, L, H, P)), (out["ddt"], "ddt", torch.float32, (b, L, H)),
                                (out["dA"], "dA", torch.float32, (H,)), (out["dB"], "dB", io, (b, L, G, N)),
                                (out["dC"], "dC", io, (b, L, G, N)), (out.get("dD"), "dD", torch.float32, (H,)),
                                (out.get("d_initial_states"), "d_initial_states", torch.float32, (S, H, P, N))):
        _check(t, name, dtype, shp, dev)
    shape = make_shape(b, L, H, P, G, N, chunk_size, S, SSD_IO_BF16 if io == torch.bfloat16 else SSD_IO_F32)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssd_bwd_noalloc(ctypes.byref(shape), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dy),
                             _ptr(initial_states), _ptr(seq_idx), _ptr(out["dx"]), _ptr(out["ddt"]),
                             _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out.get("dD")),
                             _ptr(out.get("d_initial_states")), ctypes.c_void_p(stream))
    if rc:
        raise SsdError(rc, "ssd_bwd_noalloc")
    return out


def ssd_fwd(x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, chunk_size: int = 256,
            nseqs: Optional[int] = None, want_final_states: bool = False,
            workspace: Optional[torch.Tensor] = None, dt_bias=None, dt_softplus: bool = False,
            dt_limit=(-math.inf, math.inf), z=None, want_y_pre_gate: bool = False):
    """The SSD layer's forward, computed by libssd_bwd: y, and optionally the
    state after each sequence's last position.

    Same argument conventions as ssd_bwd (including the dt front-end and the
    output gate z: y is then multiplied by silu(z)).
    Returns a dict with y (the I/O dtype, shaped like x) and final_states
    ((S, H, P, N) fp32, or None); with z and ``want_y_pre_gate`` also
    y_pre_gate, y before the gate (for ssd_bwd's ``y_pre_gate``).
    """
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd runs on a HIP device; got tensors on " + str(dev))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = x.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported io dtype {io}")
    if initial_states is not None:
        S = initial_states.shape[0]
    elif seq_idx is None:
        S = b
    else:
        if nseqs is None and want_final_states:
            raise ValueError("pass nseqs (number of sequence starts) with seq_idx")
        S = nseqs or 0
    _check(x, "x", io, (b, L, H, P), dev)
    _check(B, "B", io, (b, L, G, N), dev)
    _check(C, "C", io, (b, L, G, N), dev)
    _check(dt, "dt", torch.float32, (b, L, H), dev)
    _check(A, "A", torch.float32, (H,), dev)
    _check(initial_states, "initial_states", torch.float32, (S, H, P, N), dev)
    _check(seq_idx, "seq_idx", torch.int32, (b, L), dev)
    _check(z, "z", io, (b, L, H, P), dev)
    y_pre = torch.empty_like(x) if (z is not None and want_y_pre_gate) else None
    fe = _options(dt_bias, dt_softplus, dt_limit, D, H, P, dev, y_pre=y_pre)
    shape = make_shape(b, L, H, P, G, N, chunk_size, S, SSD_IO_BF16 if io == torch.bfloat16 else SSD_IO_F32)
    nbytes = workspace_size(shape)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    fin = (torch.empty((S, H, P, N), dtype=torch.float32, device=dev) if want_final_states and S > 0 else None)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = [_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_states), _ptr(seq_idx),
            _ptr(y), _ptr(fin), _ptr(workspace), ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream)]
    if fe is None and z is None:
        rc = lib.ssd_fwd(ctypes.byref(shape), *args)
    else:
        rc = lib.ssd_fwd_ex(ctypes.byref(shape), ctypes.byref(fe) if fe is not None else None, *args[:6], _ptr(z),
                            *args[6:])
    if rc:
        raise SsdError(rc, "ssd_fwd")
    return {"y": y, "final_states": fin, "y_pre_gate": y_pre, "workspace": workspace, "shape": shape}


class SsdChunkScan(torch.autograd.Function):
    """The SSD layer as an autograd function: ``forward`` is ssd_fwd (y only)
    and ``backward`` is ssd_bwd, which recomputes the chunk states from the
    saved inputs, so nothing but the inputs (and, with the gate z, y before
    the gate) is kept between the two."""

    @staticmethod
    def forward(ctx, x, dt, A, B, C, D, initial_states, seq_idx, dt_bias, z, chunk_size, nseqs, dt_softplus,
                dt_limit):
        fe = dict(dt_bias=dt_bias, dt_softplus=dt_softplus, dt_limit=dt_limit)
        r = ssd_fwd(x, dt, A, B, C, D, initial_states, seq_idx, chunk_size=chunk_size, nseqs=nseqs, z=z,
                    want_y_pre_gate=z is not None, **fe)
        y = r["y"]
        ctx.save_for_backward(x, dt, A, B, C, D, initial_states, seq_idx, dt_bias, z, r["y_pre_gate"])
        ctx.chunk_size, ctx.nseqs, ctx.dt_softplus, ctx.dt_limit = chunk_size, nseqs, dt_softplus, dt_limit
        return y

    @staticmethod
    def backward(ctx, dy):
        x, dt, A, B, C, D, h0, seq_idx, dt_bias, z, y_pre = ctx.saved_tensors
        want_h0 = h0 is not None and ctx.needs_input_grad[6]
        g = ssd_bwd(x, dt, A, B, C, D, dy.contiguous(), h0, seq_idx, chunk_size=ctx.chunk_size, nseqs=ctx.nseqs,
                    want_d_initial_states=want_h0, dt_bias=dt_bias, dt_softplus=ctx.dt_softplus,
                    dt_limit=ctx.dt_limit, z=z, y_pre_gate=y_pre)
        return (g["dx"], g["ddt"], g["dA"], g["dB"], g["dC"], g["dD"], g["d_initial_states"] if want_h0 else None,
                None, g.get("ddt_bias"), g.get("dz"), None, None, None, None)


def ssd_chunk_scan(x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, chunk_size: int = 256,
                   nseqs: Optional[int] = None, dt_bias=None, dt_softplus: bool = False,
                   dt_limit=(-math.inf, math.inf), z=None) -> torch.Tensor:
    """y of the SSD layer (times silu(z) when z is given) with autograd
    support (see SsdChunkScan); the gradients reach x, dt, A, B, C, D,
    initial_states, dt_bias and z."""
    return SsdChunkScan.apply(x, dt, A, B, C, D, initial_states, seq_idx, dt_bias, z, chunk_size, nseqs,
                              dt_softplus, tuple(dt_limit))


def set_launch_geometry(head_blocks: int = 0, fwd_heads_per_block: int = 0) -> None:
    """Override the launch geometry the shape does not fix (0: default); see include/ssd_bwd.h."""
    rc = load_library().ssd_set_launch_geometry(int(head_blocks), int(fwd_heads_per_block))
    if rc:
        raise SsdError(rc, "ssd_set_launch_geometry")


GROUP_PATH_BY_SHAPE, GROUP_PATH_FUSED, GROUP_PATH_SPLIT = 0, 1, 2


def set_group_path(path: int = GROUP_PATH_BY_SHAPE) -> None:
    """Force the fused or the split group kernels (or restore the choice by shape); see include/ssd_bwd.h."""
    rc = load_library().ssd_set_group_path(int(path))
    if rc:
        raise SsdError(rc, "ssd_set_group_path")


def workspace_view(result: dict, region: int) -> torch.Tensor:
    """A view of one workspace region of a finished call: Acs (float32), Hin or dS (I/O dtype)."""
    shape = result["shape"]
    off, nb = workspace_region(shape, region)
    ws = result["workspace"]
    nc = -(-shape.seqlen // shape.chunk_size)
    if region == SSD_WS_ACS:
        return ws[off:off + nb].view(torch.float32).view(shape.batch, shape.nheads, nc, shape.chunk_size)
    dt = torch.bfloat16 if shape.io_dtype == SSD_IO_BF16 else torch.float32
    return ws[off:off + nb].view(dt).view(shape.batch, shape.nheads, nc, shape.headdim, shape.dstate)


def stage_names() -> list[str]:
    lib = load_library()
    return [lib.ssd_bwd_stage_name(i).decode() for i in range(lib.ssd_bwd_stage_count())]


def make_stage_events(stream=None) -> list:
    """stage_count() + 1 timing events, each recorded once so that its HIP handle exists."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(load_library().ssd_bwd_stage_count() + 1)]
    for e in evs:
        e.record(stream)
    return evs
