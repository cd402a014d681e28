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
