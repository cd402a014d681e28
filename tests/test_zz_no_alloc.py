"""The entry point that allocates nothing (ssd_bwd_noalloc): its workspace is a fixed
device array of the library, so its output must equal ssd_bwd's byte for byte, on
consecutive calls that leave their values in that array (the second call smaller), and a
shape whose workspace exceeds the array must be refused before anything runs."""
import pytest
import torch

from state_space_model_mamba_amd import ssd
from state_space_model_mamba_amd.workloads import WORKLOADS, Workload, make_inputs
from tests.gpu_helpers import GRADS, bytes_equal, run_library, to_device
from tests.test_gpu_parity import packed

pytestmark = pytest.mark.gpu


def nan_outputs(d, S):
    x = d["x"]
    b, L, H, P = x.shape
    N = d["B"].shape[3]
    return {"dx": torch.full_like(x, float("nan")), "ddt": torch.full_like(d["dt"], float("nan")),
            "dA": torch.full((H,), float("nan"), device=x.device),
            "dB": torch.full_like(d["B"], float("nan")), "dC": torch.full_like(d["C"], float("nan")),
            "dD": torch.full((H,), float("nan"), device=x.device),
            "d_initial_states": torch.full((S, H, P, N), float("nan"), device=x.device)}


def noalloc(inputs, chunk):
    d = to_device(inputs)
    S = d["initial_states"].shape[0] if d.get("initial_states") is not None else d["x"].shape[0]
    out = nan_outputs(d, S)
    ssd.ssd_bwd_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"], out,
                        initial_states=d.get("initial_states"), seq_idx=d.get("seq_idx"), chunk_size=chunk, nseqs=S)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_ssd_bwd_on_consecutive_calls():
    # first call: the 2048-token, 128-head workload (61 MiB of the 64 MiB array)
    w1 = WORKLOADS["bf16_L2048_H128"]
    in1 = make_inputs(w1)
    print("[case] noalloc L2048 H128", flush=True)
    got1 = noalloc(in1, w1.chunk)
    ref1 = run_library(in1, w1.chunk, fill="garbage")
    assert bytes_equal(ref1, got1, keys=GRADS) == []
    # second call, smaller, on the array the first call left its values in: packed rows with
    # initial states and a ragged tail
    w2 = Workload("bf16_noalloc_small", batch=2, seqlen=700, nheads=8, headdim=64, ngroups=2, dstate=128,
                  chunk=256, dtype="bf16", seed=71)
    in2 = packed(make_inputs(w2), [[300, 256, 144], [700]])
    print("[case] noalloc small packed", flush=True)
    got2 = noalloc(in2, 256)
    ref2 = run_library(in2, 256, fill="nan")
    assert bytes_equal(ref2, got2, keys=GRADS) == []
    # and the first workload again, after the small one
    again = noalloc(in1, w1.chunk)
    assert bytes_equal(ref1, again, keys=GRADS) == []


def test_noalloc_refuses_a_workspace_larger_than_its_array():
    w = WORKLOADS["bf16_B2_L4096_H128"].scaled(seqlen=512)   # the shape check needs sizes only
    b, H, P, G, N = 2, 128, 64, 8, 128
    shape = ssd.make_shape(b, 4096, H, P, G, N, 256, b, ssd.SSD_IO_BF16)
    assert ssd.workspace_size(shape) > ssd.NOALLOC_SCRATCH_BYTES
    inputs = make_inputs(w)
    d = to_device(inputs)
    # a (2, 4096) problem's outputs, on tensors of the right shape but never written
    big = {k: torch.empty((b, 4096) + tuple(v.shape[2:]), dtype=v.dtype, device="cuda")
           for k, v in d.items() if k in ("x", "dt", "B", "C", "dy")}
    out = nan_outputs({"x": big["x"], "dt": big["dt"], "B": big["B"], "C": big["C"]}, b)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_bwd_noalloc(big["x"], big["dt"], d["A"], big["B"], big["C"], d["D"], big["dy"], out, chunk_size=256)
    assert e.value.status == -3   # SSD_ERR_WORKSPACE_TOO_SMALL
    assert torch.isnan(out["dx"]).all()
