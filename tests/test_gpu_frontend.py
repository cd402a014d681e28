"""GPU parity of the dt front-end (dt_bias, softplus, clamp; ssd_fwd_ex /
ssd_bwd_ex) with the oracle's forward_fe / backward_fe: y and the final
states, every gradient with respect to the raw dt and dt_bias, and bitwise
repeats.  The raw dt and dt_bias are drawn as the workloads' dt is
(softplus of N(0, 0.5) plus a bias that puts the step in [1e-3, 1e-1])."""
import math

import numpy as np
import pytest
import torch

import oracle
from state_space_model_mamba_amd import ssd
from state_space_model_mamba_amd.workloads import Workload, make_inputs, to_f64_numpy
from tests.gpu_helpers import GRADS, TOL, bytes_equal, compare, normwise_err, to_device, to_numpy64
from tests.test_gpu_parity import packed, small

pytestmark = pytest.mark.gpu


def raw_frontend_inputs(inputs, seed):
    """Replace dt by a raw step z ~ N(0, 0.5^2) and add dt_bias = ln(e^s - 1), s ~ U[1e-3, 1e-1]."""
    g = torch.Generator().manual_seed(seed)
    b, L, H = inputs["dt"].shape
    inputs["dt"] = (torch.randn((b, L, H), generator=g) * 0.5).contiguous()
    s = torch.rand((H,), generator=g, dtype=torch.float64) * (0.1 - 1e-3) + 1e-3
    inputs["dt_bias"] = torch.log(torch.expm1(s)).float().contiguous()
    return inputs


def run_fe(inputs, chunk, fe, nseqs=None, want_final=True):
    d = to_device(inputs)
    if nseqs is None and inputs.get("initial_states") is not None:
        nseqs = inputs["initial_states"].shape[0]
    kw = dict(dt_bias=d["dt_bias"], dt_softplus=fe["softplus"], dt_limit=fe["limit"])
    f = ssd.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d.get("initial_states"), d.get("seq_idx"),
                    chunk_size=chunk, nseqs=nseqs, want_final_states=want_final, **kw)
    g = ssd.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"], d.get("initial_states"),
                    d.get("seq_idx"), chunk_size=chunk, nseqs=nseqs, **kw)
    torch.cuda.synchronize()
    return f, g


def oracle_fe(inputs, fe, want_final=True):
    f = to_f64_numpy(inputs)
    bias = inputs["dt_bias"].double().numpy()
    kw = dict(dt_bias=bias, dt_softplus=fe["softplus"], dt_limit=fe["limit"])
    y = oracle.forward_fe(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["initial_states"], f["seq_idx"],
                          return_final_states=want_final, **kw)
    g = oracle.backward_fe(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], f["initial_states"],
                           f["seq_idx"], **kw)
    return y, g


def check_fe(inputs, chunk, fe, tol, label):
    print(f"[case] front-end {label}", flush=True)
    f, g = run_fe(inputs, chunk, fe)
    (y_ref, fs_ref), g_ref = oracle_fe(inputs, fe)
    e_y = normwise_err(f["y"].double().cpu().numpy(), y_ref)
    e_f = normwise_err(f["final_states"].double().cpu().numpy(), fs_ref)
    got = to_numpy64(g)
    got["ddt_bias"] = g["ddt_bias"].double().cpu().numpy()
    errs = compare(got, g_ref, tol, keys=GRADS + ("ddt_bias",), label=f"front-end {label}")
    print(f"front-end {label}: y err {e_y:.2e}, final states err {e_f:.2e}", flush=True)
    assert e_y <= tol and e_f <= tol
    return f, g, errs


FE_SOFTPLUS = {"softplus": True, "limit": (-math.inf, math.inf)}
FE_CLAMP = {"softplus": True, "limit": (0.01, 0.08)}


def test_frontend_fp32_tiny():
    w = small("fe_f32", batch=2, seqlen=200, nheads=4, ngroups=2, headdim=16, dstate=32, chunk=64)
    inputs = raw_frontend_inputs(packed(make_inputs(w), [[64, 40, 1, 95], [200]]), 5)
    check_fe(inputs, 64, FE_SOFTPLUS, TOL["f32"], "f32 softplus packed")


def test_frontend_fp32_clamp_bites():
    w = small("fe_f32_clamp", batch=1, seqlen=300, nheads=4, ngroups=1, headdim=16, dstate=32, chunk=128)
    inputs = raw_frontend_inputs(packed(make_inputs(w), [[100, 200]]), 6)
    v, _ = oracle.dt_frontend(inputs["dt"].double().numpy(), inputs["dt_bias"].double().numpy(), True)
    assert (v < 0.01).any() and (v > 0.08).any() and ((v > 0.01) & (v < 0.08)).any()
    check_fe(inputs, 128, FE_CLAMP, TOL["f32"], "f32 softplus + clamp")


@pytest.mark.parametrize("chunk", [128, 256])
def test_frontend_bf16(chunk):
    w = Workload("fe_bf16", batch=2, seqlen=600, nheads=8, headdim=64, ngroups=2, dstate=64, chunk=chunk,
                 dtype="bf16", seed=61)
    inputs = raw_frontend_inputs(packed(make_inputs(w), [[200, 150, 250], [600]]), 7)
    check_fe(inputs, chunk, FE_CLAMP, TOL["bf16"], f"bf16 Q{chunk} softplus + clamp")


def test_frontend_bitwise_repeat_and_autograd():
    w = Workload("fe_det", batch=1, seqlen=700, nheads=8, headdim=64, ngroups=2, dstate=64, chunk=128,
                 dtype="bf16", seed=62)
    inputs = raw_frontend_inputs(packed(make_inputs(w), [[250, 450]]), 8)
    print("[case] front-end determinism and autograd", flush=True)
    f1, g1 = run_fe(inputs, 128, FE_CLAMP)
    f2, g2 = run_fe(inputs, 128, FE_CLAMP)
    assert torch.equal(f1["y"].view(torch.int16), f2["y"].view(torch.int16))
    assert not bytes_equal(g1, g2, GRADS + ("ddt_bias",))
    d = to_device(inputs)
    leaves = {k: d[k].clone().requires_grad_(True) for k in ("x", "dt", "A", "B", "C", "D", "dt_bias")}
    y = ssd.ssd_chunk_scan(leaves["x"], leaves["dt"], leaves["A"], leaves["B"], leaves["C"], leaves["D"],
                           d["initial_states"], d["seq_idx"], chunk_size=128, nseqs=2, dt_bias=leaves["dt_bias"],
                           dt_softplus=True, dt_limit=FE_CLAMP["limit"])
    y.backward(d["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y.detach().view(torch.int16), f1["y"].view(torch.int16))
    assert torch.equal(leaves["dt"].grad.view(torch.int32), g1["ddt"].view(torch.int32))
    assert torch.equal(leaves["dt_bias"].grad.view(torch.int32), g1["ddt_bias"].view(torch.int32))
    assert torch.equal(leaves["x"].grad.view(torch.int16), g1["dx"].view(torch.int16))
