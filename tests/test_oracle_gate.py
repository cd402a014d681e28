"""Pins for the oracle's output gate (oracle.silu / forward_ex / backward_ex):
silu and its derivative at closed-form points, and the gradients of
sum(dout * y silu(z)) with respect to z, x and dt against central finite
differences."""
import math

import numpy as np

import oracle
from tests.test_oracle_pins import rand_problem


def test_silu_closed_forms():
    g, d = oracle.silu(np.array([0.0, 40.0, -40.0, 1.0]))
    assert g[0] == 0.0 and d[0] == 0.5
    assert abs(g[1] - 40.0) < 1e-12 and abs(d[1] - 1.0) < 1e-12
    assert abs(g[2]) < 1e-15 and abs(d[2]) < 1e-15
    s = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(g[3] - s) < 1e-15 and abs(d[3] - s * (2.0 - s)) < 1e-15


def test_gate_gradients_match_finite_differences():
    p = rand_problem(17, b=2, L=24, H=2, P=3, G=1, N=4, lengths=[[10, 14], [24]])
    rng = np.random.default_rng(5)
    z = rng.standard_normal(p["x"].shape)
    dout = p["dy"]
    base = (p["A"], p["B"], p["C"], p["D"])
    g = oracle.backward_ex(p["x"], p["dt"], *base, dout, p["initial_states"], p["seq_idx"], z=z)

    def loss(x, dt, zz):
        y = oracle.forward_ex(x, dt, *base, p["initial_states"], p["seq_idx"], z=zz, nthreads=1)
        return float(np.sum(y * dout))

    for name, gname in (("z", "dz"), ("x", "dx"), ("dt", "ddt")):
        arr = {"z": z, "x": p["x"], "dt": p["dt"]}[name]
        scale = np.max(np.abs(g[gname]))
        for fi in rng.choice(arr.size, size=10, replace=False):
            idx = np.unravel_index(fi, arr.shape)
            eps = 1e-6 * max(1.0, abs(arr[idx]))
            vals = {}
            for sgn in (1, -1):
                q = {"x": p["x"].copy(), "dt": p["dt"].copy(), "z": z.copy()}
                q[name][idx] += sgn * eps
                vals[sgn] = loss(q["x"], q["dt"], q["z"])
            fd = (vals[1] - vals[-1]) / (2 * eps)
            assert abs(fd - g[gname][idx]) <= 1e-6 * max(scale, 1e-3), (name, idx, fd, g[gname][idx])


def test_per_channel_D_reduces_to_scalar_D_and_matches_finite_differences():
    p = rand_problem(19, b=2, L=24, H=2, P=3, G=1, N=4, lengths=[[10, 14], [24]])
    base = (p["A"], p["B"], p["C"])
    Dhp = np.repeat(p["D"][:, None], 3, axis=1)          # the scalar D spread over the channels
    y1 = oracle.forward_ex(p["x"], p["dt"], *base, Dhp, p["initial_states"], p["seq_idx"])
    y0 = oracle.forward(p["x"], p["dt"], *base, p["D"], p["initial_states"], p["seq_idx"])
    assert np.max(np.abs(y1 - y0)) <= 1e-12 * np.max(np.abs(y0))
    g1 = oracle.backward_ex(p["x"], p["dt"], *base, Dhp, p["dy"], p["initial_states"], p["seq_idx"])
    g0 = oracle.backward(p["x"], p["dt"], *base, p["D"], p["dy"], p["initial_states"], p["seq_idx"])
    assert np.max(np.abs(g1["dx"] - g0["dx"])) <= 1e-12 * np.max(np.abs(g0["dx"]))
    assert np.max(np.abs(g1["dD"].sum(axis=1) - g0["dD"])) <= 1e-12 * np.max(np.abs(g0["dD"]))
    # a genuinely per-channel D, through the gate, against finite differences
    rng = np.random.default_rng(9)
    D = rng.standard_normal((2, 3))
    z = rng.standard_normal(p["x"].shape)
    g = oracle.backward_ex(p["x"], p["dt"], *base, D, p["dy"], p["initial_states"], p["seq_idx"], z=z)

    def loss(DD, xx):
        y = oracle.forward_ex(xx, p["dt"], *base, DD, p["initial_states"], p["seq_idx"], z=z, nthreads=1)
        return float(np.sum(y * p["dy"]))

    for idx in [(0, 0), (1, 2), (0, 1)]:
        Dp, Dm = D.copy(), D.copy()
        Dp[idx] += 1e-6
        Dm[idx] -= 1e-6
        fd = (loss(Dp, p["x"]) - loss(Dm, p["x"])) / 2e-6
        assert abs(fd - g["dD"][idx]) <= 1e-6 * max(np.max(np.abs(g["dD"])), 1e-3), (idx, fd)
    for fi in rng.choice(p["x"].size, size=6, replace=False):
        idx = np.unravel_index(fi, p["x"].shape)
        xp, xm = p["x"].copy(), p["x"].copy()
        xp[idx] += 1e-6
        xm[idx] -= 1e-6
        fd = (loss(D, xp) - loss(D, xm)) / 2e-6
        assert abs(fd - g["dx"][idx]) <= 1e-6 * max(np.max(np.abs(g["dx"])), 1e-3), (idx, fd)
