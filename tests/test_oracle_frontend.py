"""Pins for the oracle's dt front-end (oracle.dt_frontend / forward_fe /
backward_fe): the softplus and clamp values against their closed forms, and
the gradients with respect to the raw dt and dt_bias against central finite
differences of the composed loss sum(dy * y)."""
import math

import numpy as np

import oracle
from tests.test_oracle_pins import rand_problem


def test_softplus_closed_forms():
    dt = np.array([0.0, math.log(math.e - 1.0), 25.0, -3.0, 20.0]).reshape(1, 5, 1)
    v, d = oracle.dt_frontend(dt, softplus=True)
    v = v.ravel()
    d = d.ravel()
    assert abs(v[0] - math.log(2.0)) < 1e-15          # softplus(0) = ln 2
    assert abs(v[1] - 1.0) < 1e-15                    # softplus(ln(e - 1)) = 1
    assert v[2] == 25.0 and d[2] == 1.0               # taken as u above 20
    assert abs(v[3] - math.log1p(math.exp(-3.0))) < 1e-15
    assert abs(d[0] - 0.5) < 1e-15                    # sigmoid(0)
    assert abs(d[4] - 1.0 / (1.0 + math.exp(-20.0))) < 1e-15


def test_bias_and_clamp():
    dt = np.array([[[0.1, 2.0], [0.5, -1.0]]])        # (1, 2, 2)
    bias = np.array([0.2, 1.0])
    v, d = oracle.dt_frontend(dt, bias, softplus=False, dt_limit=(0.0, 1.0))
    np.testing.assert_allclose(v, [[[0.3, 1.0], [0.7, 0.0]]], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(d, [[[1.0, 0.0], [1.0, 1.0]]])   # v = dt_min exactly: inside (inclusive bounds)


def test_identity_options_reproduce_plain_calls():
    p = rand_problem(11, b=1, L=20, H=2, P=3, G=1, N=4)
    args = (p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"])
    np.testing.assert_array_equal(oracle.forward_fe(*args, p["initial_states"], p["seq_idx"]),
                                  oracle.forward(*args, p["initial_states"], p["seq_idx"]))
    g0 = oracle.backward(*args, p["dy"], p["initial_states"], p["seq_idx"])
    g1 = oracle.backward_fe(*args, p["dy"], p["initial_states"], p["seq_idx"])
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "d_initial_states"):
        np.testing.assert_array_equal(g0[k], g1[k])


def test_frontend_gradients_match_finite_differences():
    p = rand_problem(13, b=2, L=24, H=2, P=3, G=1, N=4, lengths=[[10, 14], [24]])
    rng = np.random.default_rng(3)
    raw = rng.standard_normal(p["dt"].shape) * 1.5 - 1.0
    bias = np.array([0.3, -0.4])
    fe = dict(dt_bias=bias, dt_softplus=True, dt_limit=(0.05, 0.9))
    v, _ = oracle.dt_frontend(raw, bias, True)
    assert ((v < 0.05) | (v > 0.9)).any() and ((v > 0.06) & (v < 0.89)).any()   # the clamp bites somewhere
    args = lambda q: (p["x"], q["dt"], p["A"], p["B"], p["C"], p["D"])
    g = oracle.backward_fe(*args({"dt": raw}), p["dy"], p["initial_states"], p["seq_idx"], **fe)

    def loss(dt_raw, b):
        y = oracle.forward_fe(*args({"dt": dt_raw}), p["initial_states"], p["seq_idx"],
                              dt_bias=b, dt_softplus=True, dt_limit=(0.05, 0.9), nthreads=1)
        return float(np.sum(y * p["dy"]))

    scale = np.max(np.abs(g["ddt"]))
    checked = 0
    for fi in rng.permutation(raw.size):
        idx = np.unravel_index(fi, raw.shape)
        if min(abs(v[idx] - 0.05), abs(v[idx] - 0.9)) < 1e-3:
            continue                                   # the clamp's kinks
        eps = 1e-6
        rp, rm = raw.copy(), raw.copy()
        rp[idx] += eps
        rm[idx] -= eps
        fd = (loss(rp, bias) - loss(rm, bias)) / (2 * eps)
        assert abs(fd - g["ddt"][idx]) <= 1e-6 * max(scale, 1e-3), (idx, fd, g["ddt"][idx])
        checked += 1
        if checked == 16:
            break
    for h in range(2):
        bp, bm = bias.copy(), bias.copy()
        bp[h] += 1e-6
        bm[h] -= 1e-6
        fd = (loss(raw, bp) - loss(raw, bm)) / 2e-6
        assert abs(fd - g["ddt_bias"][h]) <= 1e-6 * max(np.max(np.abs(g["ddt_bias"])), 1e-3), (h, fd)
