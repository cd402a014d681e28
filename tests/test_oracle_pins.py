"""Pins for the fp64 oracle, each independent of the oracle's own code.

The oracle evaluates the SSD recurrence sequentially with a hand-derived
reverse adjoint.  These tests tie it to things it cannot agree with by
accident:

* a hand-worked two-step example (tests/golden/hand_two_step.json);
* the quadratic masked ("attention-like") form of the same layer, materialised
  as an L x L matrix, and torch's CPU fp64 autograd of that form -- an
  independent gradient by a library;
* central finite differences of the oracle's forward loss;
* closed forms: full decay (exp(a) == 0 exactly), no decay (prefix sums),
  the scalar L = P = N = 1 case, dD = sum dy . x;
* packed sequences equal separate runs; chunk exports equal the state /
  state-gradient definitions.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "d_initial_states")


# --------------------------------------------------------------------------
# small random problems (fp64)
# --------------------------------------------------------------------------
def rand_problem(seed, b=2, L=40, H=4, P=3, G=2, N=5, lengths=None, h0=True, D=True,
                 a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((b, L, H)) * 0.5 - 1.0))
    A = -np.exp(rng.uniform(0, math.log(4.0), H)) * a_scale
    Bm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    Dv = rng.standard_normal(H) if D else None
    dy = rng.standard_normal((b, L, H, P))
    seq_idx = None
    if lengths is not None:
        rows = []
        for r in range(b):
            ids = np.repeat(np.arange(len(lengths[r])), lengths[r])
            assert ids.size == L
            rows.append(ids)
        seq_idx = np.stack(rows).astype(np.int32)
    S = oracle.count_sequences(b, L, seq_idx)
    h0v = rng.standard_normal((S, H, P, N)) * 0.5 if h0 else None
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=Dv, dy=dy, initial_states=h0v, seq_idx=seq_idx)


def run_oracle_bwd(p, **kw):
    return oracle.backward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["dy"],
                           p["initial_states"], p["seq_idx"], **kw)


def run_oracle_fwd(p, **kw):
    return oracle.forward(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"],
                          p["initial_states"], p["seq_idx"], **kw)


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# the quadratic masked form, written in torch so autograd can differentiate it
# --------------------------------------------------------------------------
def sequence_ids(seq_idx, b, L):
    if seq_idx is None:
        return torch.zeros((b, L), dtype=torch.int64)
    si = torch.as_tensor(seq_idx, dtype=torch.int64)
    start = torch.ones((b, L), dtype=torch.int64)
    start[:, 1:] = (si[:, 1:] != si[:, :-1]).to(torch.int64)
    return torch.cumsum(start, dim=1) - 1   # per-row sequence ordinal


def quadratic_forward(x, dt, A, B, C, D, h0, seq_idx):
    """y = (L o C B^T o dt_j) x + D x + exp(cumsum a) C h0, per (b, h), as an L x L matrix.

    L[i, j] = exp(sum_{k=j+1..i} a_k) for j <= i in the same sequence, 0 otherwise.
    """
    b, Lq, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    ords = sequence_ids(seq_idx, b, Lq)
    # global sequence number = (sequences in earlier rows) + ordinal in this row
    per_row = ords[:, -1] + 1
    base = torch.cumsum(per_row, 0) - per_row
    idx = torch.arange(Lq)
    ys = []
    for bb in range(b):
        same = (ords[bb][:, None] == ords[bb][None, :]) & (idx[None, :] <= idx[:, None])
        first = torch.zeros(Lq, dtype=torch.int64)
        for i in range(Lq):
            first[i] = i if (i == 0 or ords[bb][i] != ords[bb][i - 1]) else first[i - 1]
        yb = []
        for h in range(H):
            g = h // hpg
            a = dt[bb, :, h] * A[h]
            cs = torch.cumsum(a, 0)
            seg = cs[:, None] - cs[None, :]
            Lm = torch.exp(torch.where(same, seg, torch.full_like(seg, -math.inf)))
            CB = C[bb, :, g, :] @ B[bb, :, g, :].T
            M = Lm * CB * dt[bb, :, h][None, :]
            yh = M @ x[bb, :, h, :]
            if D is not None:
                yh = yh + D[h] * x[bb, :, h, :]
            if h0 is not None:
                decay = torch.exp(cs - cs[first] + a[first])      # sum_{k=t0..i} a_k
                s_of = base[bb] + ords[bb]
                hc = torch.einsum("ipn,in->ip", h0[s_of, h], C[bb, :, g, :])
                yh = yh + decay[:, None] * hc
            yb.append(yh)
        ys.append(torch.stack(yb, dim=1))
    return torch.stack(ys, dim=0)


def autograd_grads(p):
    t = {k: (torch.tensor(v, dtype=torch.float64, requires_grad=True)
             if v is not None and k not in ("seq_idx", "dy") else v)
         for k, v in p.items()}
    y = quadratic_forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_states"],
                          p["seq_idx"])
    loss = (y * torch.tensor(p["dy"])).sum()
    names = ["x", "dt", "A", "B", "C"] + (["D"] if p["D"] is not None else []) + \
            (["initial_states"] if p["initial_states"] is not None else [])
    grads = torch.autograd.grad(loss, [t[n] for n in names])
    key = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "initial_states": "d_initial_states"}
    return y.detach().numpy(), {key[n]: g.numpy() for n, g in zip(names, grads)}


# --------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------
def test_hand_worked_example():
    gold = json.load(open(os.path.join(GOLDEN, "hand_two_step.json")))
    ln2 = math.log(2.0)
    inp = gold["inputs"]
    x = np.array(inp["x"]).reshape(1, 2, 1, 1)
    dt = np.array(inp["dt"]).reshape(1, 2, 1)
    A = np.array([-2 * ln2])
    B = np.array(inp["B"]).reshape(1, 2, 1, 1)
    C = np.array(inp["C"]).reshape(1, 2, 1, 1)
    D = np.array([inp["D"]])
    dy = np.array(inp["dy"]).reshape(1, 2, 1, 1)
    h0 = np.array([inp["h0"]]).reshape(1, 1, 1, 1)
    ex = gold["expected"]
    y = oracle.forward(x, dt, A, B, C, D, h0, None)
    np.testing.assert_allclose(y.ravel(), ex["y"], rtol=0, atol=1e-14)
    g = oracle.backward(x, dt, A, B, C, D, dy, h0, None)
    np.testing.assert_allclose(g["dx"].ravel(), ex["dx"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["dB"].ravel(), ex["dB"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["dC"].ravel(), ex["dC"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["ddt"].ravel(), [2.75 - 1.1 * ln2, -6 - 1.05 * ln2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["dA"], [ex["dA"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["dD"], [ex["dD"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["d_initial_states"].ravel(), [ex["d_h0"]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("case", ["plain", "varlen_h0"])
def test_forward_matches_quadratic_form(case):
    if case == "plain":
        p = rand_problem(1, b=2, L=48, H=4, P=3, G=2, N=5, h0=False)
    else:
        p = rand_problem(2, b=2, L=40, H=4, P=3, G=2, N=5,
                         lengths=[[7, 17, 16], [40]], h0=True)
    y = run_oracle_fwd(p)
    t = {k: (torch.tensor(v) if v is not None and k != "seq_idx" else v) for k, v in p.items()}
    yq = quadratic_forward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_states"],
                           p["seq_idx"]).numpy()
    assert rel_err(y, yq) < 1e-12


@pytest.mark.parametrize("case", ["plain", "varlen_h0", "chunk_aligned_start", "long"])
def test_backward_matches_autograd_of_quadratic_form(case):
    if case == "plain":
        p = rand_problem(3, b=2, L=40, H=4, P=3, G=2, N=5, h0=False)
    elif case == "varlen_h0":
        p = rand_problem(4, b=2, L=40, H=4, P=3, G=2, N=5, lengths=[[9, 8, 23], [30, 10]])
    elif case == "chunk_aligned_start":
        p = rand_problem(5, b=1, L=40, H=2, P=3, G=1, N=4, lengths=[[16, 8, 16]])
    else:
        p = rand_problem(6, b=1, L=300, H=2, P=4, G=1, N=6, lengths=[[100, 137, 63]])
    _, ref = autograd_grads(p)
    got = run_oracle_bwd(p)
    for k, v in ref.items():
        assert rel_err(got[k], v) < 1e-10, k


def test_backward_matches_finite_differences():
    p = rand_problem(7, b=2, L=24, H=2, P=3, G=1, N=4, lengths=[[10, 14], [24]])
    g = run_oracle_bwd(p)
    dy = p["dy"]

    def loss(q):
        return float(np.sum(run_oracle_fwd(q, nthreads=1) * dy))

    rng = np.random.default_rng(0)
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "initial_states": "d_initial_states"}
    for name, gname in names.items():
        arr = p[name]
        flat_idx = rng.choice(arr.size, size=min(arr.size, 12), replace=False)
        scale = np.max(np.abs(g[gname]))
        for fi in flat_idx:
            idx = np.unravel_index(fi, arr.shape)
            eps = 1e-6 * max(1.0, abs(arr[idx]))
            qp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            qm = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            qp[name][idx] += eps
            qm[name][idx] -= eps
            fd = (loss(qp) - loss(qm)) / (2 * eps)
            assert abs(fd - g[gname][idx]) <= 1e-6 * max(scale, 1e-3), (name, idx, fd, g[gname][idx])


def test_closed_form_full_decay():
    """A so negative that exp(dt A) == 0 exactly: every step forgets its history."""
    p = rand_problem(8, b=2, L=20, H=4, P=3, G=2, N=5, lengths=[[8, 12], [20]])
    p["A"] = np.full(4, -1e7)
    assert np.all(np.exp(p["dt"][..., None] * p["A"]) == 0.0)
    y = run_oracle_fwd(p)
    g = run_oracle_bwd(p)
    x, dt, Bm, Cm, D, dy = p["x"], p["dt"], p["B"], p["C"], p["D"], p["dy"]
    hpg = 2
    Bh = np.repeat(Bm, hpg, axis=2)
    Ch = np.repeat(Cm, hpg, axis=2)
    cb = np.sum(Ch * Bh, -1)                       # (b, L, H)
    dyx = np.sum(dy * x, -1)
    np.testing.assert_allclose(y, (dt * cb)[..., None] * x + D[None, None, :, None] * x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g["dx"], (dt * cb + D)[..., None] * dy, rtol=1e-13, atol=1e-13)
    w = (dt * dyx).reshape(2, 20, 2, hpg).sum(-1)  # sum over the heads of a group
    np.testing.assert_allclose(g["dC"], w[..., None] * Bm, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dB"], w[..., None] * Cm, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["ddt"], cb * dyx, rtol=1e-12, atol=1e-13)
    assert np.all(g["dA"] == 0.0)
    assert np.all(g["d_initial_states"] == 0.0)
    np.testing.assert_allclose(g["dD"], dyx.sum(axis=(0, 1)), rtol=1e-13)


def test_closed_form_no_decay():
    """A = 0: the state is a running (prefix) sum, i.e. causal linear attention."""
    p = rand_problem(9, b=1, L=30, H=2, P=3, G=1, N=4, lengths=[[12, 18]])
    p["A"] = np.zeros(2)
    x, dt, Bm, Cm, D, dy, h0 = (p[k] for k in ("x", "dt", "B", "C", "D", "dy", "initial_states"))
    y = run_oracle_fwd(p)
    g = run_oracle_bwd(p)
    bounds = [(0, 12, 0), (12, 30, 1)]
    for h in range(2):
        for (t0, t1, s) in bounds:
            u = dt[0, t0:t1, h, None, None] * x[0, t0:t1, h, :, None] * Bm[0, t0:t1, 0, None, :]
            hs = np.cumsum(u, axis=0) + h0[s, h]                             # (T, P, N)
            yq = np.einsum("tpn,tn->tp", hs, Cm[0, t0:t1, 0]) + D[h] * x[0, t0:t1, h]
            np.testing.assert_allclose(y[0, t0:t1, h], yq, rtol=1e-12, atol=1e-12)
            v = dy[0, t0:t1, h, :, None] * Cm[0, t0:t1, 0, None, :]
            lam = np.cumsum(v[::-1], axis=0)[::-1]                           # reverse prefix sum
            dxq = dt[0, t0:t1, h, None] * np.einsum("tpn,tn->tp", lam, Bm[0, t0:t1, 0]) + D[h] * dy[0, t0:t1, h]
            np.testing.assert_allclose(g["dx"][0, t0:t1, h], dxq, rtol=1e-12, atol=1e-12)
            hprev = np.concatenate([h0[s, h][None], hs[:-1]], axis=0)
            ddtq = np.einsum("tp,tpn,tn->t", x[0, t0:t1, h], lam, Bm[0, t0:t1, 0])
            np.testing.assert_allclose(g["ddt"][0, t0:t1, h], ddtq, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(g["d_initial_states"][s, h], lam[0], rtol=1e-12, atol=1e-12)
        da = np.concatenate([np.einsum("tpn,tpn->t",
                                       np.cumsum((dy[0, t0:t1, h, :, None] * Cm[0, t0:t1, 0, None, :])[::-1], 0)[::-1],
                                       np.concatenate([h0[s, h][None], np.cumsum(dt[0, t0:t1, h, None, None] * x[0, t0:t1, h, :, None] * Bm[0, t0:t1, 0, None, :], 0)[:-1] + h0[s, h]], 0))
                             for (t0, t1, s) in bounds])
        np.testing.assert_allclose(g["dA"][h], np.sum(dt[0, :, h] * da), rtol=1e-12)


def test_scalar_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(20):
        x, dt, B, C, D, dy, h0 = rng.standard_normal(7)
        dt = abs(dt) + 0.1
        A = -abs(rng.standard_normal()) - 0.1
        e = math.exp(dt * A)
        args = [np.array(v).reshape(shape) for v, shape in
                ((x, (1, 1, 1, 1)), (dt, (1, 1, 1)), (A, (1,)), (B, (1, 1, 1, 1)), (C, (1, 1, 1, 1)), (D, (1,)))]
        dyv = np.array(dy).reshape(1, 1, 1, 1)
        h0v = np.array(h0).reshape(1, 1, 1, 1)
        y = oracle.forward(*args, h0v, None)
        assert abs(y.item() - (C * (e * h0 + dt * x * B) + D * x)) < 1e-13
        g = oracle.backward(*args, dyv, h0v, None)
        exp_ = {"dx": dy * (C * dt * B + D), "dB": dy * C * dt * x, "dC": dy * (e * h0 + dt * x * B),
                "ddt": dy * C * (A * e * h0 + x * B), "dA": dy * C * dt * e * h0, "dD": dy * x,
                "d_initial_states": dy * C * e}
        for k, v in exp_.items():
            assert abs(g[k].item() - v) < 1e-13 * max(1.0, abs(v)), k


def test_dD_is_sum_of_dy_dot_x():
    p = rand_problem(12, b=3, L=33, H=4, P=5, G=1, N=3, lengths=[[33], [11, 22], [1, 31, 1]])
    g = run_oracle_bwd(p)
    np.testing.assert_allclose(g["dD"], np.einsum("blhp,blhp->h", p["dy"], p["x"]), rtol=1e-13)


def test_packed_sequences_equal_separate_runs():
    lengths = [13, 1, 20, 30]
    p = rand_problem(13, b=1, L=64, H=4, P=3, G=2, N=4, lengths=[lengths])
    g = run_oracle_bwd(p)
    y = run_oracle_fwd(p)
    t0 = 0
    dA = np.zeros(4)
    dD = np.zeros(4)
    for s, n in enumerate(lengths):
        sl = slice(t0, t0 + n)
        q = {k: (v[:, sl] if k in ("x", "dt", "B", "C", "dy") else v) for k, v in p.items()}
        q["seq_idx"] = None
        q["initial_states"] = p["initial_states"][s:s + 1]
        gs = run_oracle_bwd(q)
        np.testing.assert_allclose(run_oracle_fwd(q), y[:, sl], rtol=1e-13, atol=1e-13)
        for k in ("dx", "ddt", "dB", "dC"):
            np.testing.assert_allclose(gs[k], g[k][:, sl], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gs["d_initial_states"][0], g["d_initial_states"][s], rtol=1e-12, atol=1e-13)
        dA += gs["dA"]
        dD += gs["dD"]
        t0 += n
    np.testing.assert_allclose(dA, g["dA"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dD, g["dD"], rtol=1e-12)


def test_head_range_matches_full_run():
    p = rand_problem(14, b=2, L=30, H=6, P=3, G=3, N=4, lengths=[[10, 20], [30]])
    full = run_oracle_bwd(p)
    part = run_oracle_bwd(p, head_lo=2, head_hi=4)
    for k in ("dx", "ddt"):
        np.testing.assert_array_equal(part[k][:, :, 2:4], full[k][:, :, 2:4])
        assert np.isnan(part[k][:, :, :2]).all()
    np.testing.assert_array_equal(part["dB"][:, :, 1], full["dB"][:, :, 1])
    np.testing.assert_array_equal(part["dA"][2:4], full["dA"][2:4])
    with pytest.raises(ValueError):
        run_oracle_bwd(p, head_lo=1, head_hi=4)   # not a whole group
    q = run_oracle_bwd(p, head_lo=1, head_hi=4, partial_groups=True)
    np.testing.assert_array_equal(q["dx"][:, :, 1:4], full["dx"][:, :, 1:4])
    np.testing.assert_array_equal(q["dB"][:, :, 1], full["dB"][:, :, 1])
    assert np.isnan(q["dB"][:, :, 0]).all() and np.isnan(q["dB"][:, :, 2]).all()


def test_chunk_exports_match_definitions():
    """chunk_states[c] = h at position c*Q-1; chunk_dout[c] = gradient of l w.r.t. the state at
    the end of chunk c through later positions only: sum_{i>t, same seq} exp(sum_{k=t+1..i} a_k) dy_i C_i."""
    Q = 8
    p = rand_problem(15, b=1, L=37, H=2, P=3, G=1, N=4, lengths=[[5, 11, 16, 5]])
    g = run_oracle_bwd(p, chunk=Q)
    x, dt, A, Bm, Cm, dy, h0 = (p[k] for k in ("x", "dt", "A", "B", "C", "dy", "initial_states"))
    starts = [0, 5, 16, 32]
    seq_of = np.repeat(np.arange(4), [5, 11, 16, 5])
    nc = -(-37 // Q)
    for h in range(2):
        a = dt[0, :, h] * A[h]
        for c in range(nc):
            t = c * Q - 1
            if t < 0:
                assert np.all(g["chunk_states"][0, c, h] == 0)
            else:
                s = seq_of[t]
                t0 = starts[s]
                st = np.exp(np.sum(a[t0:t + 1])) * h0[s, h]
                for j in range(t0, t + 1):
                    st = st + np.exp(np.sum(a[j + 1:t + 1])) * dt[0, j, h] * np.outer(x[0, j, h], Bm[0, j, 0])
                np.testing.assert_allclose(g["chunk_states"][0, c, h], st, rtol=1e-12, atol=1e-13)
            te = min(c * Q + Q - 1, 36)
            s = seq_of[te]
            lam = np.zeros((3, 4))
            for i in range(te + 1, 37):
                if seq_of[i] != s:
                    break
                lam += np.exp(np.sum(a[te + 1:i + 1])) * np.outer(dy[0, i, h], Cm[0, i, 0])
            np.testing.assert_allclose(g["chunk_dout"][0, c, h], lam, rtol=1e-12, atol=1e-13)


def test_linear_in_dy_and_deterministic():
    p = rand_problem(16)
    g1 = run_oracle_bwd(p, nthreads=3)
    g2 = run_oracle_bwd(p, nthreads=7)
    for k in GRADS:
        np.testing.assert_array_equal(g1[k], g2[k])
    q = dict(p)
    q["dy"] = p["dy"] * 2.0
    g3 = run_oracle_bwd(q)
    for k in ("dx", "ddt", "dB", "dC", "dA", "d_initial_states"):
        if k == "dx":   # D dy term scales too
            np.testing.assert_allclose(g3[k], 2 * g1[k], rtol=1e-13, atol=1e-14)
        else:
            np.testing.assert_allclose(g3[k], 2 * g1[k], rtol=1e-13, atol=1e-14)
