"""GPU parity of the last-state gradient input and of a sequence split into two stretches.

ssd_bwd(..., d_last_states=...) against the fp64 oracle's d_last; and the
hand-off a split of the sequence axis needs: the second stretch starts from
the first stretch's last states (ssd_fwd's final states) and hands its
initial-state gradients back as the first stretch's d_last_states.  The two
stretches' gradients, concatenated (dA, dD summed), must match the oracle's
gradients of the whole sequence.  The full-size case cuts the 16384-row
headline workload into two 8192-row stretches and checks one group's heads.
"""
import numpy as np
import pytest
import torch

import oracle
from state_space_model_mamba_amd import ssd
from state_space_model_mamba_amd.workloads import WORKLOADS, Workload, make_inputs, to_f64_numpy
from tests.gpu_helpers import TOL, normwise_err, to_device
from tests.test_gpu_forward import heads_slice
from tests.test_gpu_parity import packed, small

pytestmark = pytest.mark.gpu

SEQ_KEYS = ("x", "dt", "B", "C", "dy", "seq_idx")
GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "d_initial_states")


def nseqs_of(inputs):
    if inputs.get("initial_states") is not None:
        return inputs["initial_states"].shape[0]
    if inputs.get("seq_idx") is not None:
        return oracle.count_sequences(inputs["x"].shape[0], inputs["x"].shape[1], inputs["seq_idx"].numpy())
    return inputs["x"].shape[0]


def last_seq_of_rows(inputs):
    b = inputs["x"].shape[0]
    si = inputs.get("seq_idx")
    out, count = [], 0
    for r in range(b):
        count += 1 if si is None else 1 + int((si[r, 1:] != si[r, :-1]).sum())
        out.append(count - 1)
    return out


def gpu_bwd(d, chunk, d_last=None):
    res = ssd.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"], d.get("initial_states"),
                      d.get("seq_idx"), chunk_size=chunk, nseqs=nseqs_of(d), d_last_states=d_last)
    torch.cuda.synchronize()
    return res


def compare(got, ref, tol, label, keys=GRADS):
    errs = {k: normwise_err(got[k], ref[k]) for k in keys if ref.get(k) is not None}
    msg = f"{label}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items())
    print(msg, flush=True)
    assert max(errs.values()) <= tol, msg


def host(res):
    return {k: (v.double().cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_last_state_gradient_matches_oracle(dtype):
    w = Workload(f"{dtype}_dlast", batch=2, seqlen=700, nheads=8, headdim=32 if dtype == "f32" else 64,
                 ngroups=2, dstate=32 if dtype == "f32" else 64, chunk=128, dtype=dtype, seed=61)
    inputs = packed(make_inputs(w), [[300, 1, 399], [700]])
    b, L, H, P = inputs["x"].shape
    N = inputs["B"].shape[3]
    d_last = torch.randn((b, H, P, N), generator=torch.Generator().manual_seed(62)) * 0.5
    print(f"[case] d_last {dtype}", flush=True)
    d = to_device(inputs)
    got = host(gpu_bwd(d, 128, d_last.cuda()))
    f = to_f64_numpy(inputs)
    ref = oracle.backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], f["initial_states"],
                          f["seq_idx"], d_last=d_last.double().numpy())
    compare(got, ref, TOL[dtype], f"d_last {dtype}")


def split_run(inputs, cut, chunk):
    """Forward of the first stretch, backward of the second from its last states, then the first's
    backward with the handed-back gradients; returns the concatenated gradients (host, fp64)."""
    d = to_device(inputs)
    part = lambda lo, hi: {k: (v[:, lo:hi].contiguous() if k in SEQ_KEYS and v is not None else v)
                           for k, v in d.items()}
    d1, d2 = part(0, cut), part(cut, d["x"].shape[1])
    f1 = ssd.ssd_fwd(d1["x"], d1["dt"], d1["A"], d1["B"], d1["C"], d1["D"], d1.get("initial_states"),
                     d1.get("seq_idx"), chunk_size=chunk, nseqs=nseqs_of(d1), want_final_states=True)
    rows = last_seq_of_rows(d1)
    d2["initial_states"] = f1["final_states"][rows].contiguous()
    # the second stretch's sequences: one per row here (each row's last sequence crosses the cut)
    assert nseqs_of(d2) == d["x"].shape[0]
    g2 = gpu_bwd(d2, chunk)
    g1 = gpu_bwd(d1, chunk, d_last=g2["d_initial_states"].contiguous())
    out = {}
    for k in ("dx", "ddt", "dB", "dC"):
        out[k] = torch.cat([g1[k], g2[k]], dim=1)
    for k in ("dA", "dD"):
        out[k] = g1[k] + g2[k]
    out["d_initial_states"] = g1["d_initial_states"]
    return host(out)


def test_split_hand_off_fp32_packed():
    w = small("f32_split", batch=2, seqlen=640, nheads=4, ngroups=2, headdim=16, dstate=32, chunk=64)
    inputs = packed(make_inputs(w), [[100, 1, 539], [640]])
    print("[case] split fp32 packed, cut 320", flush=True)
    got = split_run(inputs, 320, 64)
    f = to_f64_numpy(inputs)
    ref = oracle.backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], f["initial_states"],
                          f["seq_idx"])
    compare(got, ref, TOL["f32"], "split fp32 packed")


def test_split_hand_off_bf16_mid_chunk_cut():
    """A cut that is not on a chunk boundary: each stretch has a partial last chunk."""
    w = Workload("bf16_split", batch=1, seqlen=1500, nheads=8, headdim=64, ngroups=2, dstate=64, chunk=256,
                 dtype="bf16", seed=63)
    inputs = make_inputs(w)
    print("[case] split bf16, cut 700", flush=True)
    got = split_run(inputs, 700, 256)
    f = to_f64_numpy(inputs)
    ref = oracle.backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], None, None)
    compare(got, ref, TOL["bf16"], "split bf16 mid-chunk", keys=("dx", "ddt", "dA", "dB", "dC", "dD"))


def test_split_hand_off_full_size_one_group():
    """The 16384-row headline workload as two 8192-row stretches (what each of two devices would hold);
    heads 80..95 (group 5) against the oracle over the whole sequence."""
    w = WORKLOADS["bf16_L16384_H128"]
    inputs = make_inputs(w)
    print("[case] split bf16_L16384_H128 at 8192", flush=True)
    got = split_run(inputs, 8192, w.chunk)
    g, hpg = 5, w.nheads // w.ngroups
    h0, h1 = g * hpg, (g + 1) * hpg
    f = to_f64_numpy(heads_slice(inputs, g, h0, h1))
    ref = oracle.backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], None, None)
    sub = {"dx": got["dx"][:, :, h0:h1], "ddt": got["ddt"][:, :, h0:h1], "dA": got["dA"][h0:h1],
           "dD": got["dD"][h0:h1], "dB": got["dB"][:, :, g:g + 1], "dC": got["dC"][:, :, g:g + 1]}
    compare(sub, ref, TOL["bf16"], "split full size, group 5", keys=("dx", "ddt", "dA", "dB", "dC", "dD"))
