"""GPU parity of the forward (y and the sequences' final states) with the fp64 oracle.

The forward shares the backward's chunk preparation and state walk; these
tests cover what it adds (the output kernel, the final states) on the same
seeded workloads and edge cases, and its determinism.
"""
import numpy as np
import pytest
import torch

import oracle
from state_space_model_mamba_amd import ssd
from state_space_model_mamba_amd.workloads import WORKLOADS, Workload, make_inputs, to_f64_numpy
from tests.gpu_helpers import TOL, normwise_err, to_device
from tests.test_gpu_parity import packed, small

pytestmark = pytest.mark.gpu


def run_fwd(inputs, chunk, want_final=False, fill=None):
    d = to_device(inputs)
    nseqs = None
    if inputs.get("initial_states") is not None:
        nseqs = inputs["initial_states"].shape[0]
    elif inputs.get("seq_idx") is not None:
        nseqs = oracle.count_sequences(inputs["x"].shape[0], inputs["x"].shape[1], inputs["seq_idx"].numpy())
    ws = None
    if fill is not None:
        x = d["x"]
        b, L, H, P = x.shape
        shape = ssd.make_shape(b, L, H, P, d["B"].shape[2], d["B"].shape[3], chunk, nseqs or b,
                               ssd.SSD_IO_BF16 if x.dtype == torch.bfloat16 else ssd.SSD_IO_F32)
        ws = torch.randint(0, 256, (ssd.workspace_size(shape),), dtype=torch.uint8, device=x.device)
    res = ssd.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"), d.get("initial_states"),
                      d.get("seq_idx"), chunk_size=chunk, nseqs=nseqs, want_final_states=want_final,
                      workspace=ws)
    torch.cuda.synchronize()
    return res


def oracle_fwd(inputs, want_final=False):
    f = to_f64_numpy(inputs)
    return oracle.forward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["initial_states"], f["seq_idx"],
                          return_final_states=want_final)


def check_fwd(inputs, chunk, tol, label, want_final=False):
    print(f"[case] forward {label}", flush=True)
    res = run_fwd(inputs, chunk, want_final)
    ref = oracle_fwd(inputs, want_final)
    y_ref, f_ref = ref if want_final else (ref, None)
    y = res["y"].double().cpu().numpy()
    assert not np.isnan(y).any()
    e_y = normwise_err(y, y_ref)
    msg = f"forward {label}: y err {e_y:.2e}"
    e_f = 0.0
    if want_final:
        fs = res["final_states"].double().cpu().numpy()
        e_f = normwise_err(fs, f_ref)
        msg += f", final states err {e_f:.2e}"
    print(msg, flush=True)
    assert e_y <= tol and e_f <= tol, msg
    return res


def test_forward_tiny_fp32():
    w = WORKLOADS["tiny_f32_L256"]
    check_fwd(make_inputs(w), w.chunk, TOL["f32"], w.name, want_final=True)


def test_forward_fp32_packed_ragged_with_initial_states():
    w = small("f32_packed_fwd", batch=2, seqlen=200, nheads=4, ngroups=2, headdim=16, dstate=32, chunk=64)
    inputs = packed(make_inputs(w), [[64, 40, 1, 95], [200]])
    check_fwd(inputs, 64, TOL["f32"], "f32 packed ragged", want_final=True)


@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_forward_bf16_chunk_sizes(chunk):
    w = Workload("bf16_fwd", batch=2, seqlen=600, nheads=8, headdim=64, ngroups=2, dstate=64, chunk=chunk,
                 dtype="bf16", seed=31)
    inputs = packed(make_inputs(w), [[200, 150, 250], [600]])
    check_fwd(inputs, chunk, TOL["bf16"], f"bf16 Q{chunk} packed", want_final=True)


def test_forward_varlen_N256_with_initial_states():
    w = Workload("bf16_varlen_fwd", batch=1, seqlen=2048, nheads=8, headdim=64, ngroups=1, dstate=256,
                 chunk=256, dtype="bf16", seed=41)
    inputs = packed(make_inputs(w), [[300, 517, 700, 531]])
    check_fwd(inputs, 256, TOL["bf16"], "bf16 varlen N256", want_final=True)


def test_forward_short_sequence_and_no_D():
    w = small("fwd_short", seqlen=37, nheads=2)
    inputs = make_inputs(w)
    inputs["D"] = None
    check_fwd(inputs, 64, TOL["f32"], "L=37, no D", want_final=True)


def test_forward_workload_L2048():
    w = WORKLOADS["bf16_L2048_H128"]
    check_fwd(make_inputs(w), w.chunk, TOL["bf16"], w.name, want_final=True)


def test_forward_bitwise_repeatable_with_garbage_workspace():
    w = Workload("bf16_fwd_det", batch=2, seqlen=1000, nheads=16, headdim=64, ngroups=4, dstate=128, chunk=256,
                 dtype="bf16", seed=21)
    inputs = packed(make_inputs(w), [[300, 300, 400], [512, 488]])
    print("[case] forward determinism", flush=True)
    a = run_fwd(inputs, 256, True, fill="garbage")
    for _ in range(5):
        b = run_fwd(inputs, 256, True, fill="garbage")
        assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))
        assert torch.equal(a["final_states"].view(torch.int32), b["final_states"].view(torch.int32))


def test_autograd_function_matches_entry_points():
    """ssd_chunk_scan: y is ssd_fwd's y, and y.backward(dy) leaves exactly
    ssd_bwd's gradients (bitwise) in every input's .grad."""
    w = Workload("bf16_autograd", batch=1, seqlen=700, nheads=8, headdim=64, ngroups=2, dstate=64, chunk=128,
                 dtype="bf16", seed=51)
    inputs = packed(make_inputs(w), [[250, 450]])
    d = to_device(inputs)
    h0 = d["initial_states"]
    print("[case] autograd function", flush=True)
    leaves = {k: d[k].clone().requires_grad_(True) for k in ("x", "dt", "A", "B", "C", "D")}
    h0_leaf = h0.clone().requires_grad_(True)
    y = ssd.ssd_chunk_scan(leaves["x"], leaves["dt"], leaves["A"], leaves["B"], leaves["C"], leaves["D"], h0_leaf,
                           d["seq_idx"], chunk_size=128, nseqs=2)
    y.backward(d["dy"])
    torch.cuda.synchronize()
    ref_y = ssd.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], h0, d["seq_idx"], chunk_size=128,
                        nseqs=2)["y"]
    ref = ssd.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"], h0, d["seq_idx"], chunk_size=128,
                      nseqs=2)
    torch.cuda.synchronize()
    assert torch.equal(y.detach().view(torch.int16), ref_y.view(torch.int16))
    for k, gk in (("x", "dx"), ("B", "dB"), ("C", "dC")):
        assert torch.equal(leaves[k].grad.view(torch.int16), ref[gk].view(torch.int16)), k
    for k, gk in (("dt", "ddt"), ("A", "dA"), ("D", "dD")):
        assert torch.equal(leaves[k].grad.view(torch.int32), ref[gk].view(torch.int32)), k
    assert torch.equal(h0_leaf.grad.view(torch.int32), ref["d_initial_states"].view(torch.int32))


def heads_slice(inputs, g, h0, h1):
    """The sub-problem of heads [h0, h1) of group g: their x, dt, A, D, dy and
    initial states, and the group's B, C."""
    sub = dict(inputs)
    for k in ("x", "dy", "dt"):
        sub[k] = inputs[k][:, :, h0:h1].contiguous()
    for k in ("A", "D"):
        sub[k] = inputs[k][h0:h1].contiguous() if inputs.get(k) is not None else None
    for k in ("B", "C"):
        sub[k] = inputs[k][:, :, g:g + 1].contiguous()
    if inputs.get("initial_states") is not None:
        sub["initial_states"] = inputs["initial_states"][:, h0:h1].contiguous()
    return sub


@pytest.mark.parametrize("name,group,nh", [("bf16_L16384_H128", 5, 16), ("bf16_varlen7_L16384_N256", 0, 8)])
def test_forward_full_size_sampled_group(name, group, nh):
    """The full-size workloads in the launch configuration bench.py times; the oracle
    evaluates the first nh heads of one group (y and final states of those heads are compared)."""
    w = WORKLOADS[name]
    inputs = make_inputs(w)
    print(f"[case] forward {name} group {group}", flush=True)
    res = run_fwd(inputs, w.chunk, want_final=True)
    h0 = group * (w.nheads // w.ngroups)
    h1 = h0 + nh
    y_ref, f_ref = oracle_fwd(heads_slice(inputs, group, h0, h1), want_final=True)
    y = res["y"][:, :, h0:h1].double().cpu().numpy()
    fs = res["final_states"][:, h0:h1].double().cpu().numpy()
    e_y, e_f = normwise_err(y, y_ref), normwise_err(fs, f_ref)
    print(f"forward {name} heads {h0}..{h1 - 1}: y err {e_y:.2e}, final states err {e_f:.2e}", flush=True)
    assert e_y <= TOL["bf16"] and e_f <= TOL["bf16"]
