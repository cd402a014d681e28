"""Pins of the oracle's last-state gradient input (d_last, CPU only).

d_last[b] is the gradient that arrives for the state after the last position
of batch row b, i.e. l gains <d_last[b], h_{L-1}> for the row's last
sequence.  Pinned by finite differences of that loss, by the closed form of a
row with no input (h_{L-1} = exp(A sum dt) h0), by the hand-off identity of a
split sequence (the two halves' backwards, chained through d_last and
d_initial_states, give the whole sequence's gradients), and by a planted
mistake that the finite-difference check must reject.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import rand_problem


def last_seq_of_rows(p):
    """Index of each batch row's last sequence (sequences are numbered in row-major order of their starts)."""
    b, L = p["x"].shape[:2]
    si = p["seq_idx"]
    count = 0
    last = []
    for r in range(b):
        starts = 1 if si is None else 1 + int(np.sum(si[r, 1:] != si[r, :-1]))
        count += starts
        last.append(count - 1)
    return last


def loss_with_last(orc, p, d_last):
    y, fin = orc.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["initial_states"], p["seq_idx"],
                         return_final_states=True)
    return float(np.sum(y * p["dy"]) + np.sum(fin[last_seq_of_rows(p)] * d_last))


def fd_agrees(orc, tol=1e-6):
    p = rand_problem(11, b=2, L=14, H=2, P=3, G=1, N=2, lengths=[[5, 9], [14]])
    d_last = np.random.default_rng(12).standard_normal((2, 2, 3, 2))
    g = orc.backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["dy"], p["initial_states"], p["seq_idx"],
                     d_last=d_last)
    for name, gname in (("x", "dx"), ("dt", "ddt"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
                        ("initial_states", "d_initial_states")):
        arr = p[name]
        for idx in [(0,) * arr.ndim, tuple(s - 1 for s in arr.shape), tuple(s // 2 for s in arr.shape)]:
            eps = 1e-6
            pp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            pm = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            pp[name][idx] += eps
            pm[name][idx] -= eps
            fd = (loss_with_last(orc, pp, d_last) - loss_with_last(orc, pm, d_last)) / (2 * eps)
            if abs(fd - g[gname][idx]) > tol * max(np.max(np.abs(g[gname])), 1e-3):
                return False
    return True


def test_last_state_gradient_matches_finite_differences():
    assert fd_agrees(oracle.Oracle())


def test_closed_form_without_input():
    """x = 0, dy = 0, one sequence: h_{L-1} = exp(A sum dt) h0, so d_h0 = exp(A sum dt) d_last,
    ddt_t = A <d_last, h_{L-1}> for every t, dA = sum(dt) <d_last, h_{L-1}> and
    dx_t = dt_t exp(A sum_{u>t} dt_u) d_last B_t."""
    p = rand_problem(13, b=1, L=9, H=1, P=2, G=1, N=3)
    p["x"][:] = 0.0
    p["dy"][:] = 0.0
    d_last = np.random.default_rng(14).standard_normal((1, 1, 2, 3))
    g = oracle.backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["dy"], p["initial_states"], None,
                        d_last=d_last)
    A, S = p["A"][0], p["dt"][0, :, 0].sum()
    hl = np.exp(A * S) * p["initial_states"][0, 0]
    inner = float(np.sum(d_last[0, 0] * hl))
    np.testing.assert_allclose(g["d_initial_states"][0, 0], np.exp(A * S) * d_last[0, 0], rtol=1e-13)
    np.testing.assert_allclose(g["ddt"][0, :, 0], A * inner, rtol=1e-12)
    np.testing.assert_allclose(g["dA"][0], S * inner, rtol=1e-12)
    # lambda_t = exp(A sum_{u>t} dt_u) d_last, so dx_t = dt_t lambda_t B_t
    dt = p["dt"][0, :, 0]
    for t in range(9):
        lam = np.exp(A * dt[t + 1:].sum()) * d_last[0, 0]
        np.testing.assert_allclose(g["dx"][0, t, 0], dt[t] * lam @ p["B"][0, t, 0], rtol=1e-12)


@pytest.mark.parametrize("lengths", [None, [[7, 13, 20], [40]]])
def test_split_sequence_hand_off(lengths):
    """Rows cut at position 24: the second part starts from the first part's last states and hands
    its initial-state gradients back as the first part's d_last.  Concatenated (dA, dD summed) they
    are the gradients of the whole rows."""
    p = rand_problem(15, b=2, L=40, H=3, P=2, G=1, N=4, lengths=lengths)
    cut = 24
    full = oracle.backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["dy"], p["initial_states"],
                           p["seq_idx"])
    part = lambda lo, hi: {k: (v[:, lo:hi].copy() if k in ("x", "dt", "B", "C", "dy", "seq_idx") and v is not None
                               else v) for k, v in p.items()}
    p1, p2 = part(0, cut), part(cut, 40)
    # without seq_idx both rows cross the cut; with it, row 0's third sequence and row 1's only one do,
    # so the first part keeps every sequence's initial state and the second part has one sequence a row
    _, fin1 = oracle.forward(p1["x"], p1["dt"], p1["A"], p1["B"], p1["C"], p1["D"], p1["initial_states"],
                             p1["seq_idx"], return_final_states=True)
    p2["initial_states"] = fin1[last_seq_of_rows(p1)]
    g2 = oracle.backward(p2["x"], p2["dt"], p2["A"], p2["B"], p2["C"], p2["D"], p2["dy"], p2["initial_states"],
                         p2["seq_idx"])
    g1 = oracle.backward(p1["x"], p1["dt"], p1["A"], p1["B"], p1["C"], p1["D"], p1["dy"], p1["initial_states"],
                         p1["seq_idx"], d_last=g2["d_initial_states"])
    for k in ("dx", "ddt", "dB", "dC"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], axis=1), full[k], rtol=1e-10, atol=1e-12,
                                   err_msg=k)
    for k in ("dA", "dD"):
        np.testing.assert_allclose(g1[k] + g2[k], full[k], rtol=1e-10, err_msg=k)
    np.testing.assert_allclose(g1["d_initial_states"], full["d_initial_states"], rtol=1e-10, atol=1e-12)


def test_planted_mistake_in_the_seeding_is_caught(tmp_path):
    src = open(oracle.SOURCE).read()
    old = "memcpy(lam, c->d_last + ((b * s->nheads + h) * PN), sizeof(double) * PN);"
    assert src.count(old) == 1
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, "memcpy(lam, c->d_last + ((h * s->batch + b) * PN), sizeof(double) * PN);"))
    so = str(tmp_path / "libmutant_last.so")
    oracle.compile_source(str(path), so)
    assert not fd_agrees(oracle.Oracle(so))
