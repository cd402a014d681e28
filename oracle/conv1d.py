"""fp64 CPU oracle of the depthwise causal convolution of the Mamba-2 block
(test infrastructure only: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the HIP library never does).

The page "Deterministic bwd kernel for mamba2" (state-spaces/mamba PR 827,
its section on atomic-add non-determinism) names causal-conv1d's backward as
the other place, besides the SSD kernels, where atomics make training runs
non-deterministic.  It does not write the operation out; the reading taken
here is the usual one of the Mamba-2 block, per channel c of a channels-last
input x (batch, seqlen, channels) and a filter w (channels, width):

    pre[b, t, c] = bias[c] + sum_k  w[c, k] * x[b, t - (W-1) + k, c] * m(t, t - (W-1) + k)
    out[b, t, c] = act(pre[b, t, c]),   act = identity or SiLU (u * sigmoid(u))

where the mask m(t, s) is 1 when 0 <= s and rows s and t belong to the same
sequence, else 0: the filter never reaches across a sequence start or before
the first row.  A sequence starts at row r when r = 0 or seq_idx[b, r] !=
seq_idx[b, r - 1] (the SSD's own definition of a packed batch), so rows s <= t
share a sequence when no sequence starts in (s, t]; without seq_idx every row
is one sequence.

The backward follows from the chain rule applied to that definition, with
g = dout * act'(pre):

    dx[b, s, c]  = sum_k  w[c, k] * g[b, s + (W-1) - k, c] * m(s + (W-1) - k, s)
    dw[c, k]     = sum_{b,t}  g[b, t, c] * x[b, t - (W-1) + k, c] * m(t, t - (W-1) + k)
    dbias[c]     = sum_{b,t}  g[b, t, c]

Everything is numpy float64, vectorised over (batch, time, channel) with one
plain loop over the filter taps.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

ACTIVATIONS = ("none", "silu")


def _sequence_number(seq_idx: np.ndarray) -> np.ndarray:
    """Number of sequence starts at or before each row: (batch, L) int64."""
    seq_idx = np.asarray(seq_idx)
    starts = np.ones(seq_idx.shape, dtype=np.int64)
    starts[:, 1:] = seq_idx[:, 1:] != seq_idx[:, :-1]
    return np.cumsum(starts, axis=1)


def _mask(L: int, shift: int, seq_idx: Optional[np.ndarray], batch: int) -> np.ndarray:
    """m(t, t - shift) for t in [0, L): shape (batch, L, 1), 0/1 float64."""
    t = np.arange(L)
    ok = np.broadcast_to((t - shift >= 0)[None, :], (batch, L)).astype(np.float64)
    if seq_idx is not None and shift > 0:
        num = _sequence_number(seq_idx)   # equal for two rows exactly when no start lies between them
        same = np.zeros((batch, L))
        same[:, shift:] = (num[:, shift:] == num[:, :-shift])
        ok = ok * same
    return ok[:, :, None]


def _shifted(a: np.ndarray, shift: int) -> np.ndarray:
    """a[:, t - shift] (zeros where t - shift < 0)."""
    out = np.zeros_like(a)
    if shift == 0:
        out[:] = a
    elif shift < a.shape[1]:
        out[:, shift:] = a[:, :-shift]
    return out


def _ahead(a: np.ndarray, shift: int) -> np.ndarray:
    """a[:, t + shift] (zeros where t + shift >= L)."""
    out = np.zeros_like(a)
    if shift == 0:
        out[:] = a
    elif shift < a.shape[1]:
        out[:, :-shift] = a[:, shift:]
    return out


def _sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def preactivation(x, w, bias=None, seq_idx=None):
    """pre = bias + sum_k w[:, k] * x[t - (W-1) + k] * m   (fp64, (batch, seqlen, channels))."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    batch, L, C = x.shape
    W = w.shape[1]
    pre = np.zeros_like(x)
    if bias is not None:
        pre += np.asarray(bias, np.float64)[None, None, :]
    for k in range(W):
        shift = W - 1 - k
        pre += w[None, None, :, k] * _shifted(x, shift) * _mask(L, shift, seq_idx, batch)
    return pre


def forward(x, w, bias=None, seq_idx=None, activation="none"):
    """out = act(pre)."""
    if activation not in ACTIVATIONS:
        raise ValueError(activation)
    pre = preactivation(x, w, bias, seq_idx)
    return pre * _sigmoid(pre) if activation == "silu" else pre


def backward(x, w, bias, seq_idx, dout, activation="none"):
    """Gradients of l = sum dout * out: dict with dx (fp64, like x), dw (channels, width), dbias (channels)."""
    if activation not in ACTIVATIONS:
        raise ValueError(activation)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    dout = np.asarray(dout, np.float64)
    batch, L, C = x.shape
    W = w.shape[1]
    pre = preactivation(x, w, bias, seq_idx)
    if activation == "silu":
        sg = _sigmoid(pre)
        g = dout * sg * (1.0 + pre * (1.0 - sg))
    else:
        g = dout
    dx = np.zeros_like(x)
    dw = np.zeros((C, W))
    for k in range(W):
        shift = W - 1 - k
        m = _mask(L, shift, seq_idx, batch)             # m(t, t - shift), indexed by t
        dw[:, k] = np.sum(g * _shifted(x, shift) * m, axis=(0, 1))
        # row s receives g at t = s + shift, where m(t, s) was evaluated at t
        dx += w[None, None, :, k] * _ahead(g * m, shift)
    return {"dx": dx, "dw": dw, "dbias": g.sum(axis=(0, 1))}
