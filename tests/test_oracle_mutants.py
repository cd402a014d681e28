"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), compiles it, and checks that the pin comparisons
(hand-worked example, autograd of the quadratic form, finite differences)
reject it.  The real oracle passes the same comparisons.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import autograd_grads, rand_problem

MUTANTS = {
    "dx_drops_D_term": ("c->dx[IDX_X(s, b, t, h, p)] = dtv * acc + Dh * dyt[p];",
                        "c->dx[IDX_X(s, b, t, h, p)] = dtv * acc;"),
    "da_wrong_sign": ("const double da = decay * inner;", "const double da = -decay * inner;"),
    "dB_wrong_operand": ("for (int64_t p = 0; p < P; ++p) acc += lam[p * N + n] * xt[p];",
                         "for (int64_t p = 0; p < P; ++p) acc += lam[p * N + n] * dyt[p];"),
    "carry_not_decayed": ("for (int64_t q = 0; q < PN; ++q) lam[q] *= decay;",
                          "for (int64_t q = 0; q < PN; ++q) lam[q] *= 1.0;"),
    "d_h0_not_decayed": ("for (int64_t q = 0; q < PN; ++q) dst[q] = decay * lam[q];",
                         "for (int64_t q = 0; q < PN; ++q) dst[q] = lam[q];"),
    "ddt_drops_A_da": ("c->ddt[IDX_BLH(s, b, t, h)] = xlb + Ah * da;",
                       "c->ddt[IDX_BLH(s, b, t, h)] = xlb;"),
    "prev_state_off_by_one": ("(t > t0) ? hs + (t - t0 - 1) * PN : ckpt + k * PN;",
                              "(t > t0) ? hs + (t - t0) * PN : ckpt + k * PN;"),
    "dC_uses_previous_state": ("for (int64_t p = 0; p < P; ++p) acc += ht[p * N + n] * dyt[p];",
                               "for (int64_t p = 0; p < P; ++p) acc += hp[p * N + n] * dyt[p];"),
    "group_index_interleaved": ("const int64_t g = h / (s->nheads / s->ngroups);\n  const int64_t nblk",
                                "const int64_t g = h % s->ngroups;\n  const int64_t nblk"),
    "no_reset_at_sequence_start": ("if (!st && seq_idx) st = (seq_idx[i] != seq_idx[i - 1]);",
                                   "if (0) st = (seq_idx[i] != seq_idx[i - 1]);"),
}


def pins_pass(orc: oracle.Oracle) -> bool:
    """The pin comparisons of test_oracle_pins, run against one compiled oracle."""
    try:
        p = rand_problem(4, b=2, L=40, H=4, P=3, G=2, N=5, lengths=[[9, 8, 23], [30, 10]])
        _, ref = autograd_grads(p)
        got = orc.backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["dy"],
                           p["initial_states"], p["seq_idx"])
        for k, v in ref.items():
            if not np.max(np.abs(got[k] - v)) <= 1e-10 * max(np.max(np.abs(v)), 1e-300):
                return False
        q = rand_problem(7, b=1, L=16, H=2, P=2, G=1, N=3, lengths=[[6, 10]])
        g = orc.backward(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], q["dy"],
                         q["initial_states"], q["seq_idx"])

        def loss(qq):
            return float(np.sum(orc.forward(qq["x"], qq["dt"], qq["A"], qq["B"], qq["C"], qq["D"],
                                            qq["initial_states"], qq["seq_idx"]) * q["dy"]))
        for name, gname in (("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                            ("initial_states", "d_initial_states")):
            idx = (0,) * q[name].ndim
            eps = 1e-6
            qp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in q.items()}
            qm = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in q.items()}
            qp[name][idx] += eps
            qm[name][idx] -= eps
            fd = (loss(qp) - loss(qm)) / (2 * eps)
            if abs(fd - g[gname][idx]) > 1e-6 * max(np.max(np.abs(g[gname])), 1e-3):
                return False
        return True
    except (RuntimeError, ValueError):
        return False


def test_real_oracle_passes_the_mutation_pins():
    assert pins_pass(oracle.Oracle())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"libmutant_{name}.so")
    oracle.compile_source(str(path), so)
    assert not pins_pass(oracle.Oracle(so)), f"pins did not catch {name}"
