"""fp64 CPU oracle for the Mamba-2 SSD layer (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``ssd_oracle.c`` (plain C, fp64, host threads)
through ctypes; see that file's header for the recurrence and the reverse
adjoint it evaluates.  The product path (the HIP library and its binding)
never imports it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssd_oracle.c")
LIBRARY = os.path.join(HERE, "libssd_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread"]


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("batch", "seqlen", "nheads", "headdim", "ngroups", "dstate", "nseqs")]


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libssd_oracle.so``."""
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
        _DEFAULT.__dict__.pop("_lib", None)
    return LIBRARY


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _dptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """The oracle bound to one compiled library (the default one, or a test variant)."""

    def __init__(self, path: str = LIBRARY):
        self.path = path

    @property
    def lib(self):
        if "_lib" not in self.__dict__:
            if self.path == LIBRARY and not os.path.exists(LIBRARY):
                build()
            lib = ctypes.CDLL(self.path)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int32)
            lib.ssdo_count_sequences.restype = ctypes.c_int64
            lib.ssdo_count_sequences.argtypes = [ctypes.POINTER(_Shape), ip]
            lib.ssdo_forward.restype = ctypes.c_int
            lib.ssdo_forward.argtypes = [ctypes.POINTER(_Shape)] + [dp] * 7 + [ip, dp, dp, ctypes.c_int]
            lib.ssdo_backward.restype = ctypes.c_int
            lib.ssdo_backward.argtypes = ([ctypes.POINTER(_Shape)] + [dp] * 7 + [ip, dp] +
                                          [ctypes.c_int64, ctypes.c_int64] + [dp] * 7 +
                                          [ctypes.c_int64, dp, dp, dp, ctypes.c_int])
            self.__dict__["_lib"] = lib
        return self.__dict__["_lib"]

    def _shape(self, x, B, h0, seq_idx):
        b, L, H, P = x.shape
        s = _Shape(b, L, H, P, B.shape[2], B.shape[3], 0)
        s.nseqs = self.lib.ssdo_count_sequences(ctypes.byref(s), _iptr(seq_idx))
        if h0 is not None and h0.shape[0] != s.nseqs:
            raise ValueError(f"initial_states has {h0.shape[0]} sequences, seq_idx gives {s.nseqs}")
        return s

    def count_sequences(self, batch: int, seqlen: int, seq_idx=None) -> int:
        s = _Shape(batch, seqlen, 1, 1, 1, 1, 0)
        return int(self.lib.ssdo_count_sequences(ctypes.byref(s), _iptr(_i32(seq_idx))))

    def forward(self, x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, nthreads=None,
                return_final_states=False):
        """y (B,L,H,P) of the SSD recurrence, in fp64 (and the final states per sequence)."""
        x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, initial_states))
        si = _i32(seq_idx)
        s = self._shape(x, B, h0, si)
        y = np.empty_like(x)
        fs = np.empty((s.nseqs, s.nheads, s.headdim, s.dstate)) if return_final_states else None
        rc = self.lib.ssdo_forward(ctypes.byref(s), _dptr(x), _dptr(dt), _dptr(A), _dptr(B),
                                   _dptr(C), _dptr(D), _dptr(h0), _iptr(si), _dptr(y), _dptr(fs),
                                   nthreads or default_threads())
        if rc:
            raise RuntimeError(f"ssdo_forward failed: {rc}")
        return (y, fs) if return_final_states else y

    def backward(self, x, dt, A, B, C, D, dy, initial_states=None, seq_idx=None, head_lo=0,
                 head_hi=None, chunk=0, nthreads=None, want_d_initial=True, partial_groups=False,
                 d_last=None):
        """All gradients of l = sum(dy * y) in fp64 (plus <d_last[b], h_{L-1}> per batch row when
        ``d_last`` (B, H, P, N) is given: the gradient handed back for the state after each row's
        last position).

        Returns a dict with dx, ddt, dA, dB, dC, dD, d_initial_states (None when
        not requested) and, when ``chunk`` > 0, ``chunk_states`` / ``chunk_dout``
        (B, nc, H, P, N).  Only heads [head_lo, head_hi) -- whole groups -- are
        evaluated; entries of other heads/groups are left as NaN.  dB/dC need
        every head of a group; with ``partial_groups`` a range may split
        groups and dB/dC of those groups stay NaN.
        """
        x, dt, A, B, C, D, dy, h0, d_last = map(_f64, (x, dt, A, B, C, D, dy, initial_states, d_last))
        si = _i32(seq_idx)
        s = self._shape(x, B, h0, si)
        if head_hi is None:
            head_hi = s.nheads
        hpg = s.nheads // s.ngroups
        if (head_lo % hpg or head_hi % hpg) and not partial_groups:
            raise ValueError("head range must cover whole groups (or pass partial_groups=True; "
                             "dB/dC are then left NaN for partly covered groups)")
        out = {
            "dx": np.full_like(x, np.nan), "ddt": np.full_like(dt, np.nan),
            "dA": np.full((s.nheads,), np.nan), "dB": np.full_like(B, np.nan),
            "dC": np.full_like(C, np.nan), "dD": np.full((s.nheads,), np.nan),
            "d_initial_states": (np.full((s.nseqs, s.nheads, s.headdim, s.dstate), np.nan)
                                 if want_d_initial else None),
        }
        cs = cd = None
        if chunk:
            nc = -(-s.seqlen // chunk)
            cs = np.full((s.batch, nc, s.nheads, s.headdim, s.dstate), np.nan)
            cd = np.full_like(cs, np.nan)
        rc = self.lib.ssdo_backward(
            ctypes.byref(s), _dptr(x), _dptr(dt), _dptr(A), _dptr(B), _dptr(C), _dptr(D),
            _dptr(h0), _iptr(si), _dptr(dy), head_lo, head_hi, _dptr(out["dx"]),
            _dptr(out["ddt"]), _dptr(out["dA"]), _dptr(out["dB"]), _dptr(out["dC"]),
            _dptr(out["dD"]), _dptr(out["d_initial_states"]), chunk, _dptr(cs), _dptr(cd),
            _dptr(d_last), nthreads or default_threads())
        if rc:
            raise RuntimeError(f"ssdo_backward failed: {rc}")
        if chunk:
            out["chunk_states"] = cs
            out["chunk_dout"] = cd
        return out


_DEFAULT = Oracle()


# --------------------------------------------------------------------------
# dt front-end (an elementwise map in front of the recurrence; numpy fp64)
# --------------------------------------------------------------------------
def dt_frontend(dt, dt_bias=None, softplus=False, dt_limit=(-math.inf, math.inf)):
    """The step the recurrence uses, from the raw dt (b, L, H), and its
    derivative with respect to the raw dt, both in fp64:

        u = dt + dt_bias[h];  v = ln(1 + e^u) (u itself above 20) if softplus else u;
        dt_eff = clamp(v, dt_min, dt_max);  d dt_eff / du = [dt_min <= v <= dt_max] * (sigmoid(u) or 1)
    """
    u = _f64(dt)
    if dt_bias is not None:
        u = u + _f64(dt_bias)[None, None, :]
    if softplus:
        low = u <= 20.0
        us = np.where(low, u, 0.0)
        v = np.where(low, np.log1p(np.exp(us)), u)
        d = np.where(low, 1.0 / (1.0 + np.exp(-us)), 1.0)
    else:
        v, d = u, np.ones_like(u)
    lo, hi = float(dt_limit[0]), float(dt_limit[1])
    inside = (v >= lo) & (v <= hi)
    return np.clip(v, lo, hi), np.where(inside, d, 0.0)


def forward_fe(x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, dt_bias=None, dt_softplus=False,
               dt_limit=(-math.inf, math.inf), **kw):
    """forward() with the dt front-end applied to the raw dt."""
    dt_eff, _ = dt_frontend(dt, dt_bias, dt_softplus, dt_limit)
    return forward(x, dt_eff, A, B, C, D, initial_states, seq_idx, **kw)


def backward_fe(x, dt, A, B, C, D, dy, initial_states=None, seq_idx=None, dt_bias=None, dt_softplus=False,
                dt_limit=(-math.inf, math.inf), **kw):
    """backward() with the dt front-end: ddt is taken with respect to the raw
    dt (chain rule through the elementwise map), and ddt_bias[h] is its sum
    over batch and positions."""
    dt_eff, d = dt_frontend(dt, dt_bias, dt_softplus, dt_limit)
    g = backward(x, dt_eff, A, B, C, D, dy, initial_states, seq_idx, **kw)
    g["ddt"] = g["ddt"] * d
    g["ddt_bias"] = g["ddt"].sum(axis=(0, 1)) if dt_bias is not None else None
    return g


def forward(*args, **kw):
    return _DEFAULT.forward(*args, **kw)


def backward(*args, **kw):
    return _DEFAULT.backward(*args, **kw)


def count_sequences(*args, **kw):
    return _DEFAULT.count_sequences(*args, **kw)


# --------------------------------------------------------------------------
# output gate (an elementwise map after the layer; numpy fp64)
# --------------------------------------------------------------------------
def silu(z):
    """silu(z) = z sigmoid(z) and its derivative sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = _f64(z)
    s = 1.0 / (1.0 + np.exp(-z))
    return z * s, s * (1.0 + z * (1.0 - s))


def _per_channel(D):
    return D is not None and np.ndim(D) == 2


def forward_ex(x, dt, A, B, C, D=None, initial_states=None, seq_idx=None, z=None, return_final_states=False,
               **kw):
    """forward_fe() (dt front-end keywords included), with D either (H,) or
    per channel (H, P): y += D[h, p] x[..., h, p]; times silu(z) when z is given."""
    if _per_channel(D):
        res = forward_fe(x, dt, A, B, C, None, initial_states, seq_idx, return_final_states=return_final_states,
                         **kw)
        dterm = _f64(x) * _f64(D)[None, None, :, :]
        res = (res[0] + dterm, res[1]) if return_final_states else res + dterm
    else:
        res = forward_fe(x, dt, A, B, C, D, initial_states, seq_idx, return_final_states=return_final_states, **kw)
    if z is None:
        return res
    y, fs = res if return_final_states else (res, None)
    g, _ = silu(z)
    return (y * g, fs) if return_final_states else y * g


def backward_ex(x, dt, A, B, C, D, dout, initial_states=None, seq_idx=None, z=None, **kw):
    """backward_fe() with a per-channel D allowed (dx += D dy, dD[h, p] the sum
    of dy x over batch and positions) and, with z, for the output
    out = y silu(z): dout is the gradient of out, so the layer sees
    dy = dout silu(z), and dz = dout y silu'(z) with y the ungated output."""
    fe = {k: kw[k] for k in ("dt_bias", "dt_softplus", "dt_limit") if k in kw}
    dy = _f64(dout)
    res_dz = None
    if z is not None:
        y = forward_ex(x, dt, A, B, C, D, initial_states, seq_idx, **fe)
        g, dg = silu(z)
        res_dz = dy * y * dg
        dy = dy * g
    if _per_channel(D):
        res = backward_fe(x, dt, A, B, C, None, dy, initial_states, seq_idx, **kw)
        res["dx"] = res["dx"] + _f64(D)[None, None, :, :] * dy
        res["dD"] = (dy * _f64(x)).sum(axis=(0, 1))
    else:
        res = backward_fe(x, dt, A, B, C, D, dy, initial_states, seq_idx, **kw)
    if z is not None:
        res["dz"] = res_dz
    return res
