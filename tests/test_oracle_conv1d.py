"""Pins of the causal-conv1d oracle (CPU only).

The forward is pinned to numpy's full convolution and to torch's grouped
conv1d (both with the causal padding cut off), the packed form to separate
per-sequence runs, and the backward to central finite differences of the
fp64 forward, to torch's autograd of the grouped conv1d and to the closed
form at a zero input.  Planted mistakes in a copy of the oracle's source must
fail these comparisons.
"""
import types

import numpy as np
import pytest
import torch

from oracle import conv1d as oc


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def seq_rows(lengths):
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)[None, :]


@pytest.mark.parametrize("W", [2, 3, 4])
def test_forward_is_numpy_convolve(W):
    x, w, bias = rand((2, 37, 5), 1), rand((5, W), 2), rand((5,), 3)
    out = oc.forward(x, w, bias)
    for b in range(2):
        for c in range(5):
            # out[t] = sum_j w[W-1-j] x[t-j]: numpy's full convolution with the reversed filter
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:37] + bias[c]
            np.testing.assert_allclose(out[b, :, c], ref, rtol=0, atol=1e-12)


def torch_conv(x, w, bias, act):
    """torch's grouped conv1d over (batch, channels, seqlen), left padding W-1, fp64."""
    C, W = w.shape
    xt = x.permute(0, 2, 1)
    y = torch.nn.functional.conv1d(xt, w[:, None, :], bias, padding=W - 1, groups=C)[..., :x.shape[1]]
    if act == "silu":
        y = torch.nn.functional.silu(y)
    return y.permute(0, 2, 1)


@pytest.mark.parametrize("act", ["none", "silu"])
def test_forward_and_backward_match_torch_grouped_conv(act):
    x, w, bias, dout = rand((2, 50, 6), 4), rand((6, 4), 5, 0.5), rand((6,), 6), rand((2, 50, 6), 7)
    xt, wt, bt = (torch.tensor(a, requires_grad=True) for a in (x, w, bias))
    y = torch_conv(xt, wt, bt, act)
    np.testing.assert_allclose(oc.forward(x, w, bias, None, act), y.detach().numpy(), rtol=0, atol=1e-12)
    (y * torch.tensor(dout)).sum().backward()
    g = oc.backward(x, w, bias, None, dout, act)
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dw"], wt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dbias"], bt.grad.numpy(), rtol=0, atol=1e-10)


def test_packed_row_is_separate_sequences():
    lengths = [5, 1, 9, 2, 7]
    L = sum(lengths)
    x, w, bias, dout = rand((1, L, 4), 8), rand((4, 4), 9), rand((4,), 10), rand((1, L, 4), 11)
    sidx = seq_rows(lengths)
    out = oc.forward(x, w, bias, sidx, "silu")
    g = oc.backward(x, w, bias, sidx, dout, "silu")
    dw, db, t0 = np.zeros_like(w), np.zeros_like(bias), 0
    for n in lengths:
        sl = slice(t0, t0 + n)
        np.testing.assert_allclose(out[:, sl], oc.forward(x[:, sl], w, bias, None, "silu"), rtol=0, atol=1e-12)
        gs = oc.backward(x[:, sl], w, bias, None, dout[:, sl], "silu")
        np.testing.assert_allclose(g["dx"][:, sl], gs["dx"], rtol=0, atol=1e-12)
        dw += gs["dw"]
        db += gs["dbias"]
        t0 += n
    np.testing.assert_allclose(g["dw"], dw, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dbias"], db, rtol=0, atol=1e-11)


def packed_equals_separate(mod, sidx, lengths, seed=30):
    """mod's forward and gradients on one packed row equal its separate runs of the given lengths."""
    L = sum(lengths)
    x, w, bias, dout = rand((1, L, 3), seed), rand((3, 4), seed + 1), rand((3,), seed + 2), rand((1, L, 3), seed + 3)
    out = mod.forward(x, w, bias, sidx, "silu")
    g = mod.backward(x, w, bias, sidx, dout, "silu")
    ok, t0, dw = True, 0, np.zeros_like(w)
    for n in lengths:
        sl = slice(t0, t0 + n)
        gs = mod.backward(x[:, sl], w, bias, None, dout[:, sl], "silu")
        ok &= np.allclose(out[:, sl], mod.forward(x[:, sl], w, bias, None, "silu"), rtol=0, atol=1e-12)
        ok &= np.allclose(g["dx"][:, sl], gs["dx"], rtol=0, atol=1e-12)
        dw += gs["dw"]
        t0 += n
    return bool(ok and np.allclose(g["dw"], dw, rtol=0, atol=1e-11))


def test_sequences_start_where_seq_idx_changes():
    """A sequence starts wherever seq_idx changes (the SSD's definition), so an id that comes back
    later opens a new sequence: ids 0, 1, 0, 2, 0 in runs of 5, 1, 6, 2, 4 are five sequences, and
    the packed row equals the five run separately.  Masking by equal ids instead would let the
    width-4 filter join the runs of id 0 across the shorter runs between them, and must fail the
    same check."""
    lengths = [5, 1, 6, 2, 4]
    sidx = np.repeat(np.array([0, 1, 0, 2, 0], dtype=np.int32), lengths)[None, :]
    assert packed_equals_separate(oc, sidx, lengths)
    src = open(oc.__file__).read()
    old = "same[:, shift:] = (num[:, shift:] == num[:, :-shift])"
    assert src.count(old) == 1
    mod = types.ModuleType("conv1d_equal_ids")
    exec(compile(src.replace(old, "same[:, shift:] = (seq_idx[:, shift:] == seq_idx[:, :-shift])"), mod.__name__,
                 "exec"), mod.__dict__)
    assert not packed_equals_separate(mod, sidx, lengths)


def fd_grads(mod, x, w, bias, sidx, dout, act, eps=1e-6):
    """Central differences of l = sum dout * forward."""
    def loss(xx, ww, bb):
        return float(np.sum(dout * mod.forward(xx, ww, bb, sidx, act)))
    res = {}
    for name, arr in (("dx", x), ("dw", w), ("dbias", bias)):
        grad = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            args = [x.copy(), w.copy(), bias.copy()]
            k = ("dx", "dw", "dbias").index(name)
            args[k][i] += eps
            lp = loss(*args)
            args[k][i] -= 2 * eps
            lm = loss(*args)
            grad[i] = (lp - lm) / (2 * eps)
        res[name] = grad
    return res


def fd_problem():
    lengths = [4, 6, 3]
    x, w, bias = rand((2, 13, 3), 12), rand((3, 4), 13, 0.6), rand((3,), 14, 0.3)
    dout = rand((2, 13, 3), 15)
    sidx = np.concatenate([seq_rows(lengths), seq_rows([13])])
    return x, w, bias, sidx, dout


def fd_agrees(mod):
    x, w, bias, sidx, dout = fd_problem()
    g = mod.backward(x, w, bias, sidx, dout, "silu")
    ref = fd_grads(oc, x, w, bias, sidx, dout, "silu")
    return all(np.allclose(g[k], ref[k], rtol=1e-6, atol=1e-7) for k in ("dx", "dw", "dbias"))


def test_backward_matches_finite_differences_packed_silu():
    x, w, bias, sidx, dout = fd_problem()
    g = oc.backward(x, w, bias, sidx, dout, "silu")
    ref = fd_grads(oc, x, w, bias, sidx, dout, "silu")
    for k in ("dx", "dw", "dbias"):
        np.testing.assert_allclose(g[k], ref[k], rtol=1e-6, atol=1e-7, err_msg=k)


def test_backward_closed_form_at_zero_input():
    """x = 0, bias = 0: pre = 0 and SiLU'(0) = 1/2, so dbias = sum(dout)/2, dw = 0 and
    dx[s] = sum_k w[k] dout[s + W-1-k] / 2."""
    L, C, W = 11, 2, 3
    w, dout = rand((C, W), 16), rand((1, L, C), 17)
    g = oc.backward(np.zeros((1, L, C)), w, np.zeros(C), None, dout, "silu")
    np.testing.assert_allclose(g["dbias"], dout.sum(axis=(0, 1)) / 2, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(g["dw"], 0.0)
    for s in range(L):
        ref = sum(w[:, k] * dout[0, s + W - 1 - k] for k in range(W) if s + W - 1 - k < L) / 2
        np.testing.assert_allclose(g["dx"][0, s], ref, rtol=0, atol=1e-12)


MUTANTS = {
    "dx_mask_taken_at_the_wrong_row": ("dx += w[None, None, :, k] * _ahead(g * m, shift)",
                                       "dx += w[None, None, :, k] * _ahead(g, shift) * m"),
    "silu_derivative_without_the_sigmoid_slope": ("g = dout * sg * (1.0 + pre * (1.0 - sg))", "g = dout * sg"),
    "dw_takes_the_unshifted_input": ("dw[:, k] = np.sum(g * _shifted(x, shift) * m, axis=(0, 1))",
                                     "dw[:, k] = np.sum(g * x * m, axis=(0, 1))"),
    "dx_filter_reversed": ("dx += w[None, None, :, k] * _ahead(g * m, shift)",
                           "dx += w[None, None, :, W - 1 - k] * _ahead(g * m, shift)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_the_pins(name):
    old, new = MUTANTS[name]
    src = open(oc.__file__).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"conv1d_{name}")
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    assert not fd_agrees(mod), f"the pins did not catch {name}"


def test_unmodified_oracle_passes_the_same_check():
    assert fd_agrees(oc)
