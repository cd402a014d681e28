"""Benchmark of the deterministic SSD backward (libssd_bwd) on one MI355X.

    python bench.py [--gpus 1] [--steps 300] [--warmup 50] [--workload bf16_L16384_H128]

One step = one full ssd_bwd call (forward-state recompute + all backward
kernels) over one synthetic batch already resident in HBM.  Prints one JSON
line: tokens/s (value), ms per step (= ms per layer), the dominant kernel's
roofline, the whole-step roofline, whether every step's outputs were bitwise
identical, and the fp64 CPU oracle timed on a bounded sample of the same
workload (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD bwd ms/layer + tokens/s at L=16K (1 GPU); bitwise repeat + % roofline"
LEG_STEPS, LEG_WARMUP, CONFIG_STEPS = 100, 20, 50   # floors for the measurements beside the headline
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["k_prep.hip", "k_state.hip", "k_group.hip", "k_dbdc.hip", "k_grp.hip", "k_head.hip", "k_fwd.hip",
                  "ssd_device.h", "ssd_tiles.h", "ssd_problem.h"]


def sizes(w, ntg):
    """Byte sizes of the tensors of one call (I/O dtype s bytes, fp32 elsewhere)."""
    s = 2 if w.dtype == "bf16" else 4
    nc = -(-w.seqlen // w.chunk)
    S = w.nseqs_packed if w.nseqs_packed else w.batch
    z = dict(
        X=w.batch * w.seqlen * w.nheads * w.headdim * s,          # x, dy or dx
        BC=w.batch * w.seqlen * w.ngroups * w.dstate * s,          # B, C, dB or dC
        DT=w.batch * w.seqlen * w.nheads * 4,                      # dt or ddt
        INIT=(S * w.nheads * w.headdim * w.dstate * 4) if w.h0_std > 0 else 0,
        DINIT=S * w.nheads * w.headdim * w.dstate * 4,
        SEQ=w.batch * w.seqlen * 4 if w.nseqs_packed else 0,
        T=w.batch * w.nheads * nc * w.headdim * w.dstate * s,      # Hin or dS (I/O dtype)
        T32=w.batch * w.nheads * nc * w.headdim * w.dstate * 4,    # Hin or dS at fp32
        CH=w.batch * w.nheads * nc * w.chunk * 4,                  # one per-chunk fp32 vector
        OFFD=w.batch * w.nheads * nc * ntg * w.chunk * 4,
        SEG=w.batch * nc * w.chunk * 4,
        CBT=w.batch * w.ngroups * nc * (w.chunk * (w.chunk + 16) // 2) * 4,   # causal C B^T tiles, fp32
        DCB=w.batch * w.ngroups * nc * w.chunk * w.chunk * s,      # dCB tile (or its transpose), split path
        CBT_FWD=w.batch * w.ngroups * nc * (w.chunk * (w.chunk + 16) // 2) * s,   # the forward's, I/O dtype
    )
    return z


def step_alg_bytes(z, state_bytes="fp32"):
    """Compulsory I/O plus one write and one read of the chunk states Hin and the state
    gradients dS -- counted at fp32 (the algorithmic model: the chunked method's published
    states) or as this library stores them (the I/O dtype)."""
    T = z["T32"] if state_bytes == "fp32" else z["T"]
    return step_compulsory_bytes(z) + 4 * T


def step_compulsory_bytes(z):
    """Read x, dy, B, C, dt (and h0, seq_idx); write dx, dB, dC, ddt (and d_init)."""
    return 3 * z["X"] + 4 * z["BC"] + 2 * z["DT"] + z["INIT"] + z["DINIT"] + z["SEQ"]


def group_fused(w):
    """The library's choice of group kernels for this workload: fused when the split kernels'
    grid has fewer than 256 blocks and a group has at most 16 heads, else split."""
    nc = -(-w.seqlen // w.chunk)
    ntg = w.dstate // next(t for t in (128, 64, 32, 16) if w.dstate % t == 0)
    return w.batch * w.ngroups * nc * ntg < 256 and w.nheads // w.ngroups <= 16


def stage_alg_bytes(z, fused=False):
    """Each operand a stage must read or write, counted once (the group stages per path)."""
    if fused:   # k_cb; k_grp
        dcb = 2 * z["BC"] + z["CBT"]
        dbdc = 2 * z["X"] + 4 * z["BC"] + 2 * z["T"] + 2 * z["CH"] + z["SEG"] + z["INIT"] + z["OFFD"]
    else:       # k_dcb; k_dc and k_db
        dcb = 2 * z["X"] + 2 * z["BC"] + 2 * z["CH"] + z["SEG"] + 2 * z["DCB"] + z["CBT"]
        dbdc = 2 * z["X"] + 4 * z["BC"] + 2 * z["T"] + 2 * z["CH"] + z["INIT"] + z["OFFD"] + 2 * z["DCB"]
    return {
        "prep": z["DT"] + z["SEQ"] + 2 * z["CH"] + z["SEG"],
        "state_fwd": z["X"] + z["BC"] + 2 * z["CH"] + z["INIT"] + z["T"],
        "state_bwd": z["X"] + z["BC"] + z["CH"] + z["T"] + z["DINIT"],
        "dcb": dcb,
        "dbdc": dbdc,
        "head_bwd": 3 * z["X"] + z["BC"] + z["T"] + z["CBT"] + 2 * z["CH"] + z["OFFD"] + z["DT"],
        "reduce": 0,
    }


def head_alg_bytes(z):
    """What the per-head kernel must touch by the method: read x, dy, B, C (for C B^T), dS (at
    fp32), dt; write dx, ddt.  Design intermediates (stored C B^T tiles, ddA partials) excluded."""
    return 3 * z["X"] + 2 * z["BC"] + z["T32"] + 2 * z["DT"]


def forward_alg_bytes(z, fin):
    """Per forward kernel (beyond the shared prep and state walk), each operand counted once;
    fin = bytes of the final states written."""
    return {
        "fwd_cbf": 2 * z["BC"] + z["CBT_FWD"],
        "fwd_y": 2 * z["X"] + z["BC"] + z["T"] + z["CBT_FWD"] + 2 * z["CH"],
        "fwd_final": fin,
    }


def step_alg_flops(w):
    """MFMA flops of the chunked method, causal Q x Q products counted at half."""
    nc = -(-w.seqlen // w.chunk)
    Q, P, N = w.chunk, w.headdim, w.dstate
    per_hc = 5 * 2 * P * N * Q + 2 * Q * Q * P
    per_gc = 3 * Q * Q * N
    return w.batch * nc * (w.nheads * per_hc + w.ngroups * per_gc)


def source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "state_space_model_mamba_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from committed rocprofv3 counter runs, or None
    when there are none for this workload or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get(stage)
    return None if ent is None else ent.get("bytes_per_launch")


# stage of each library kernel (kernel name prefix -> stage)
STAGE_OF_KERNEL = [("k_head_bwd", "head_bwd"), ("k_state_fwd", "state_fwd"), ("k_state_bwd", "state_bwd"),
                   ("k_dcb<", "dcb"), ("k_dc<", "dbdc"), ("k_db<", "dbdc"), ("k_cb<", "dcb"), ("k_grp<", "dbdc"),
                   ("k_dcb_out<", "dcb"), ("k_bd_out<", "dbdc"),
                   ("k_prep", "prep"),
                   ("k_seqbase", "prep"), ("k_reduce", "reduce"),
                   ("k_cbf<", "fwd_cbf"), ("k_y<", "fwd_y"), ("k_final<", "fwd_final"), ("k_seqstart", "fwd_final")]
CALIB_BYTES = 1 << 28   # bytes read (and written) by one calibration copy


def calibration_copy(torch, dev, reps=3):
    """A plain copy of known size (fp32 multiply by one), the reference for the HBM counters."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _counter_means(path, counter):
    import csv
    acc = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_counters(fetch_csv, write_csv, workload, out_path=TRAFFIC_FILE):
    """Per-stage HBM bytes per launch from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE,
    KiB per dispatch), each scaled by what the counter reads for the calibration copy."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    copy_f = [v for k, v in fetch.items() if "MulFunctor" in k]
    copy_w = [v for k, v in write.items() if "MulFunctor" in k]
    if not copy_f or not copy_w:
        raise SystemExit("calibration copy kernel not found in the counter files")
    f_scale = CALIB_BYTES / (copy_f[0] * 1024.0)
    w_scale = CALIB_BYTES / (copy_w[0] * 1024.0)
    stages = {}
    for name in set(fetch) | set(write):
        stage = next((s for pre, s in STAGE_OF_KERNEL if pre in name), None)
        if stage is None:
            continue
        e = stages.setdefault(stage, {"fetch_bytes": 0.0, "write_bytes": 0.0, "kernels": []})
        e["fetch_bytes"] += fetch.get(name, 0.0) * 1024.0 * f_scale
        e["write_bytes"] += write.get(name, 0.0) * 1024.0 * w_scale
        e["kernels"].append(name)
    for e in stages.values():
        e["bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
    rec = {}
    try:
        with open(out_path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        pass
    if rec.get("source_digest") != source_digest():
        rec = {"workloads": {}}
    rec["source_digest"] = source_digest()
    rec["calibration"] = {"copy_bytes": CALIB_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
                          "copy_fetch_kib": copy_f[0], "copy_write_kib": copy_w[0]}
    rec["workloads"][workload] = stages
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    return rec


# rocprofv3 --pmc passes for the per-kernel counter summaries (each within one run's limits:
# at most 8 SQ and 2 GRBM counters)
PMC_PASSES = {
    "A": ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES",
          "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAIT_INST_ANY"],
    "B": ["GRBM_GUI_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_INSTS_SALU",
          "SQ_WAVE_CYCLES", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_VMEM_RD"],
}
N_CU, N_SIMD, N_XCD = 256, 1024, 8   # MI355X


def summarize_pmc(csv_paths):
    """Per-kernel means (per dispatch) of the counters in rocprofv3 counter_collection CSVs.  The
    SQ counters are totals over the GPU; GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's
    busy cycles are GRBM_GUI_ACTIVE / 8.  Derived rates: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (cycles * SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / (cycles * CUs) (rocprofv3's VALUBusy);
    LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / (cycles * CUs); waits per wave-cycle =
    SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.  Returns markdown."""
    import csv
    vals, durs = {}, {}
    for path in csv_paths:
        with open(path) as fh:
            for row in csv.DictReader(fh):
                k = row["Kernel_Name"]
                stage = next((st for pre, st in STAGE_OF_KERNEL if pre in k), None)
                if stage is None:
                    continue
                key = (stage, k.split("(")[0].replace("void ", ""))
                vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                if row["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    durs.setdefault(key, []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    lines = ["| kernel | dispatch us | MFMA busy | VALU busy | VALU insts/wave | MFMA insts/wave | "
             "LDS insts/wave | LDS bank-conflict cycles / CU-cycles | wait-any / wave-cycles | trans f32 insts/wave |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for (stage, name), c in sorted(vals.items()):
        m = {k: sum(v) / len(v) for k, v in c.items()}
        g = m.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD
        waves = m.get("SQ_WAVES", float("nan"))
        f = lambda k, d: m[k] / d if k in m and d else float("nan")
        us = sum(durs[(stage, name)]) / len(durs[(stage, name)]) / 1e3
        lines.append(f"| {name} | {us:.1f} | {f('SQ_VALU_MFMA_BUSY_CYCLES', g * N_SIMD):.1%} | "
                     f"{f('SQ_ACTIVE_INST_VALU', g * N_CU):.1%} | {f('SQ_INSTS_VALU', waves):.0f} | "
                     f"{f('SQ_INSTS_MFMA', waves):.0f} | {f('SQ_INSTS_LDS', waves):.0f} | "
                     f"{f('SQ_LDS_BANK_CONFLICT', g * N_CU):.1%} | {f('SQ_WAIT_INST_ANY', m.get('SQ_WAVE_CYCLES')):.2f} | "
                     f"{f('SQ_INSTS_VALU_TRANS_F32', waves):.0f} |")
    return "\n".join(lines)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inputs, groups=1):
    """The fp64 oracle on the heads of `groups` groups of the workload (all tokens)."""
    import numpy as np
    import oracle
    hpg = w.nheads // w.ngroups
    h1 = groups * hpg
    g1 = groups
    f = {}
    for k in ("x", "dy"):
        f[k] = inputs[k][:, :, :h1].to(dtype=__import__("torch").float64).numpy()
    f["dt"] = inputs["dt"][:, :, :h1].double().numpy()
    f["A"] = inputs["A"][:h1].double().numpy()
    f["D"] = inputs["D"][:h1].double().numpy()
    f["B"] = inputs["B"][:, :, :g1].double().numpy()
    f["C"] = inputs["C"][:, :, :g1].double().numpy()
    h0 = inputs.get("initial_states")
    f["h0"] = None if h0 is None else h0[:, :h1].double().numpy()
    si = inputs.get("seq_idx")
    f["seq_idx"] = None if si is None else si.numpy()
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.backward(f["x"], f["dt"], f["A"], f["B"], f["C"], f["D"], f["dy"], f["h0"], f["seq_idx"],
                    nthreads=threads)
    dt = time.perf_counter() - t0
    frac = h1 / w.nheads
    return {"value": w.tokens * frac / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "seconds": round(dt, 3),
            "sample": (f"all {w.tokens} tokens, all {w.nheads} heads" if h1 == w.nheads else
                       f"all {w.tokens} tokens of heads 0..{h1 - 1} ({groups} of {w.ngroups} groups); "
                       f"tokens/s scaled by {h1}/{w.nheads} of the heads")}


def measure_forward(torch, ssd, w, d, S, ws, z, steps, warmup):
    """ssd_fwd (y and the final states) on the same workload, timed like the backward.

    Algorithmic bytes: read x, B, C, dt (and h0); write y and the final
    states; one write and one read of the chunk states."""
    def call():
        return ssd.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d.get("initial_states"),
                           d.get("seq_idx"), chunk_size=w.chunk, nseqs=S, want_final_states=True, workspace=ws)
    for _ in range(warmup):
        ref = call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        last = call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    fin = S * w.nheads * w.headdim * w.dstate * 4
    alg = 2 * z["X"] + 2 * z["BC"] + z["DT"] + z["INIT"] + 2 * z["T"] + fin + z["SEQ"]
    gbs = alg / (ms * 1e-3) / 1e9
    bitwise = (torch.equal(ref["y"].view(torch.int16) if ref["y"].dtype == torch.bfloat16 else ref["y"].view(torch.int32),
                           last["y"].view(torch.int16) if last["y"].dtype == torch.bfloat16 else last["y"].view(torch.int32))
               and torch.equal(ref["final_states"].view(torch.int32), last["final_states"].view(torch.int32)))
    return {"ms_per_call": ms, "tokens_per_s": w.tokens / (ms * 1e-3), "calls": steps, "warmup": warmup,
            "roofline": {"bound": "hbm", "alg_bytes": alg, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS},
            "bitwise_repeat": bitwise}


def measure_frontend(torch, ssd, w, d, S, ws, steps, warmup, z=None, y_pre=None):
    """ssd_bwd with the dt front-end (the raw draws, dt_bias, softplus) on the same workload:
    the same step as the headline plus the activation and the dt_bias gradient (and, with z,
    the output gate: the gated dy and dz first, from y recomputed, or with y_pre from the
    forward's saved pre-gate y, as the autograd function does)."""
    def call():
        return ssd.ssd_bwd(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d["dy"],
                           initial_states=d.get("initial_states"), seq_idx=d.get("seq_idx"), chunk_size=w.chunk,
                           nseqs=S, workspace=ws, dt_bias=d["dt_bias"], dt_softplus=True, z=z, y_pre_gate=y_pre)
    for _ in range(warmup):
        ref = call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        last = call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    same = all(torch.equal(ref[k].view(torch.int16) if ref[k].dtype == torch.bfloat16 else ref[k].view(torch.int32),
                           last[k].view(torch.int16) if last[k].dtype == torch.bfloat16 else last[k].view(torch.int32))
               for k in ref if k in ("dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dz"))
    return {"ms_per_step": ms, "tokens_per_s": w.tokens / (ms * 1e-3), "steps": steps, "warmup": warmup,
            "bitwise_repeat": same}


def conv_cpu_baseline(cw, inputs, channels=10240):
    """The fp64 conv oracle (forward and backward) on the host, over the first `channels` channels of
    the same inputs (channels are independent); tokens/s scaled by that fraction of the channels."""
    import numpy as np
    from oracle import conv1d as oc
    c1 = min(channels, cw.channels)
    x = inputs["x"][:, :, :c1].double().numpy()
    dout = inputs["dout"][:, :, :c1].double().numpy()
    w, b = inputs["weight"][:c1].double().numpy(), inputs["bias"][:c1].double().numpy()
    sidx = None if inputs["seq_idx"] is None else inputs["seq_idx"].numpy()
    t0 = time.perf_counter()
    oc.forward(x, w, b, sidx, cw.activation)
    oc.backward(x, w, b, sidx, dout, cw.activation)
    dt = time.perf_counter() - t0
    return {"value": cw.tokens * (c1 / cw.channels) / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"all {cw.tokens} tokens of channels 0..{c1 - 1} (forward and backward); tokens/s scaled "
                      f"by {c1}/{cw.channels} of the channels"}


def measure_conv1d(torch, steps, warmup, dev, cpu=False):
    """The xBC causal convolution of the headline layer (conv1d_fwd, conv1d_bwd), each timed
    over `steps` calls with HIP events on the current stream.

    Algorithmic bytes per call: forward reads x and writes out; backward reads
    x and dout and writes dx (the filter, bias and their gradients are
    channels * (width + 1) floats each way)."""
    from state_space_model_mamba_amd import conv1d
    from state_space_model_mamba_amd.workloads import CONV_HEADLINE, CONV_WORKLOADS, make_conv_inputs
    cw = CONV_WORKLOADS[CONV_HEADLINE]
    ci = make_conv_inputs(cw)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in ci.items()}
    shape = conv1d.make_shape(cw.batch, cw.seqlen, cw.channels, cw.width, cw.activation,
                              0 if cw.dtype == "bf16" else 1)
    ws = torch.empty(conv1d.workspace_size(shape), dtype=torch.uint8, device=dev)
    y = torch.empty_like(d["x"])
    g = {"dx": torch.empty_like(d["x"]), "dweight": torch.empty_like(d["weight"]),
         "dbias": torch.empty_like(d["bias"])}
    fwd = lambda: conv1d.conv1d_fwd(d["x"], d["weight"], d["bias"], d["seq_idx"], cw.activation, out=y)
    bwd = lambda: conv1d.conv1d_bwd(d["x"], d["weight"], d["bias"], d["seq_idx"], d["dout"], cw.activation,
                                    workspace=ws, out=g)

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            call()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    el = d["x"].element_size() * d["x"].numel()
    par = cw.channels * (cw.width + 1) * 4
    res = {"workload": cw.name, "batch": cw.batch, "seqlen": cw.seqlen, "channels": cw.channels,
           "width": cw.width, "activation": cw.activation, "dtype": cw.dtype}
    for name, call, alg in (("forward", fwd, 2 * el + par), ("backward", bwd, 3 * el + 2 * par)):
        ms = timed(call)
        gbs = alg / (ms * 1e-3) / 1e9
        res[name] = {"ms_per_call": ms, "tokens_per_s": cw.tokens / (ms * 1e-3), "calls": steps, "warmup": warmup,
                     "roofline": {"bound": "hbm", "alg_bytes": alg, "achieved": gbs, "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}}
    y0, g0 = y.clone(), {k: v.clone() for k, v in g.items()}
    fwd()
    bwd()
    torch.cuda.synchronize()
    if cpu:
        res["cpu_baseline"] = conv_cpu_baseline(cw, ci)
    res["bitwise_repeat"] = (torch.equal(y0.view(torch.int16), y.view(torch.int16))
                             and torch.equal(g0["dx"].view(torch.int16), g["dx"].view(torch.int16))
                             and torch.equal(g0["dweight"].view(torch.int32), g["dweight"].view(torch.int32))
                             and torch.equal(g0["dbias"].view(torch.int32), g["dbias"].view(torch.int32)))
    return res


def _bits(t):
    return t.view(torch_int_view(t))


def torch_int_view(t):
    import torch
    return {2: torch.int16, 4: torch.int32}[t.element_size()]


def measure_backward(torch, ssd, w, steps, warmup, dev, stages=True):
    """Time `steps` ssd_bwd calls on workload w (after `warmup` untimed calls) with HIP events
    on the call's stream: the whole timed region (mean) and every call (median, min).  Then,
    outside the timed region, per-stage times from the profiling entry point.  Returns the
    measurement, the inputs and the per-stage algorithmic bytes."""
    from state_space_model_mamba_amd.workloads import make_inputs
    inputs = make_inputs(w)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inputs.items()}
    S = d["initial_states"].shape[0] if d.get("initial_states") is not None else (w.nseqs_packed or w.batch)
    shape = ssd.shape_of(d["x"], d["B"], w.chunk, S)
    ws = torch.empty(ssd.workspace_size(shape), dtype=torch.uint8, device=dev)
    H, P, N = w.nheads, w.headdim, w.dstate
    out = {"dx": torch.empty_like(d["x"]), "ddt": torch.empty_like(d["dt"]),
           "dA": torch.empty(H, device=dev), "dB": torch.empty_like(d["B"]),
           "dC": torch.empty_like(d["C"]), "dD": torch.empty(H, device=dev),
           "d_initial_states": torch.empty((S, H, P, N), device=dev)}
    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        ssd.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["dy"],
                    initial_states=d.get("initial_states"), seq_idx=d.get("seq_idx"), chunk_size=w.chunk,
                    nseqs=S, workspace=ws, out=out, events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(steps):
        step()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
    mean_ms = ev[0].elapsed_time(ev[steps]) / steps
    bitwise = all(torch.equal(_bits(out[k]), _bits(ref[k])) for k in out)
    stage_ms = None
    if stages:
        # per-stage times from a second pass, with the library recording an
        # event between stages (kept out of the timed region above)
        names = ssd.stage_names()
        nprof = max(1, min(steps, 50))
        ev_steps = [ssd.make_stage_events(stream) for _ in range(nprof)]
        torch.cuda.synchronize()
        for k in range(nprof):
            step(ev_steps[k])
        torch.cuda.synchronize()
        stage_ms = {n: 0.0 for n in names}
        for evs in ev_steps:
            for i, n in enumerate(names):
                stage_ms[n] += evs[i].elapsed_time(evs[i + 1]) / nprof
    ntg = N // next(t for t in (128, 64, 32, 16) if N % t == 0)
    z = sizes(w, ntg)
    alg = step_alg_bytes(z, "fp32")
    alg_io = step_alg_bytes(z, "io")
    comp = step_compulsory_bytes(z)
    med = per_call[len(per_call) // 2]
    rec = {
        "workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": H, "headdim": P,
        "ngroups": w.ngroups, "dstate": N, "chunk": w.chunk, "nseqs": S, "initial_states": w.h0_std > 0,
        "dtype": w.dtype, "steps": steps, "warmup": warmup, "group_path": "fused" if group_fused(w) else "split",
        "ms_per_layer": {"mean": mean_ms, "median": med, "min": per_call[0], "max": per_call[-1]},
        "tokens_per_s": {"mean": w.tokens / (mean_ms * 1e-3), "median": w.tokens / (med * 1e-3),
                         "best": w.tokens / (per_call[0] * 1e-3)},
        # the algorithmic model: compulsory I/O plus one write and one read of Hin and dS at fp32
        "roofline_fp32_states": {"alg_bytes": alg, "roofline_ms": alg / (PEAK_HBM_GBS * 1e9) * 1e3,
                                 "frac_mean": alg / (PEAK_HBM_GBS * 1e9) * 1e3 / mean_ms,
                                 "frac_median": alg / (PEAK_HBM_GBS * 1e9) * 1e3 / med},
        # the same with the states as this library stores them (I/O dtype)
        "roofline_io_states": {"alg_bytes": alg_io, "frac_median": alg_io / (PEAK_HBM_GBS * 1e9) * 1e3 / med},
        # compulsory I/O only (no chunk states at all): the stricter fraction
        "roofline_compulsory": {"alg_bytes": comp, "frac_median": comp / (PEAK_HBM_GBS * 1e9) * 1e3 / med},
        "alg_mfma_tflops_median": step_alg_flops(w) / (med * 1e-3) / 1e12,
        "bitwise_repeat": bitwise,
    }
    if stage_ms is not None:
        rec["stages_ms"] = stage_ms
    return rec, inputs, d, S, ws, z


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-forward", action="store_true",
                    help="skip the forward (ssd_fwd) and the dt front-end / gate measurements")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the dt front-end / gate measurements (the backward and forward only)")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip the causal-conv1d forward / backward measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (not the other workloads of the family)")
    ap.add_argument("--group-path", choices=("auto", "fused", "split"), default="auto",
                    help="force one implementation of the group stage (default: the library's choice by shape)")
    ap.add_argument("--exact-steps", action="store_true",
                    help="time every measurement with exactly --steps / --warmup (short profiling runs); by "
                         "default the measurements beside the headline take at least %d warm-up and %d timed calls"
                         % (LEG_WARMUP, LEG_STEPS))
    ap.add_argument("--cpu-groups", type=int, default=0,
                    help="groups of heads the CPU baseline covers (0 = all)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run a plain copy of known size (reference for HBM counters)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files into the traffic record and exit")
    ap.add_argument("--pmc-pass", choices=sorted(PMC_PASSES),
                    help="print the counters of one rocprofv3 --pmc pass (space separated) and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print a per-kernel markdown table of rocprofv3 counter CSVs and exit")
    args = ap.parse_args()
    if args.pmc_pass:
        print(" ".join(PMC_PASSES[args.pmc_pass]))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.ingest_counters:
        from state_space_model_mamba_amd.workloads import HEADLINE
        rec = ingest_counters(*args.ingest_counters, workload=args.workload or HEADLINE)
        print(json.dumps(rec, indent=1, sort_keys=True))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding of this path is a design note, not a measured run)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_model_mamba_amd import ssd
    from state_space_model_mamba_amd.workloads import HEADLINE, WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    forced = {"auto": ssd.GROUP_PATH_BY_SHAPE, "fused": ssd.GROUP_PATH_FUSED, "split": ssd.GROUP_PATH_SPLIT}
    ssd.set_group_path(forced[args.group_path])
    global group_fused
    if args.group_path != "auto":
        group_fused = (lambda wl: True) if args.group_path == "fused" else (lambda wl: False)
    print(f"[bench] {w.name}: {args.warmup} warm-up and {args.steps} timed calls", file=sys.stderr, flush=True)
    rec, inputs, d, S, ws, z = measure_backward(torch, ssd, w, args.steps, args.warmup, dev)
    stage_ms = rec["stages_ms"]
    sb = stage_alg_bytes(z, group_fused(w))
    sb["head_bwd"] = head_alg_bytes(z)
    dom = max(stage_ms, key=stage_ms.get)
    achieved = sb[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = measured_traffic(w.name, dom)
    ms_per_step = rec["ms_per_layer"]["mean"]
    H = w.nheads
    res = {
        "metric": METRIC,
        "value": w.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": H, "headdim": w.headdim,
                   "ngroups": w.ngroups, "dstate": w.dstate, "chunk": w.chunk,
                   "nseqs": S, "initial_states": w.h0_std > 0, "parallelism": "single GPU"},
        "ms_per_layer": rec["ms_per_layer"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": sb[dom], "avg_ms": stage_ms[dom]},
        "step_roofline": {"bound": "hbm", "alg_bytes": rec["roofline_fp32_states"]["alg_bytes"],
                          "achieved": rec["roofline_fp32_states"]["alg_bytes"] / (ms_per_step * 1e-3) / 1e9,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": rec["roofline_fp32_states"]["frac_mean"],
                          "frac_median": rec["roofline_fp32_states"]["frac_median"],
                          "roofline_ms": rec["roofline_fp32_states"]["roofline_ms"],
                          "frac_io_states_median": rec["roofline_io_states"]["frac_median"],
                          "frac_compulsory_median": rec["roofline_compulsory"]["frac_median"],
                          "alg_mfma_tflops": step_alg_flops(w) / (ms_per_step * 1e-3) / 1e12,
                          "mfma_peak_tflops": PEAK_BF16_TFLOPS},
        "stages_ms": stage_ms,
        "bitwise_repeat": rec["bitwise_repeat"],
    }
    # the secondary measurements take at least LEG_WARMUP warm-up and LEG_STEPS timed calls, so that a
    # short run of the headline (few warm-up calls) still times them warm
    leg_steps, leg_warmup = max(args.steps, LEG_STEPS), max(args.warmup, LEG_WARMUP)
    config_steps = max(args.steps, CONFIG_STEPS)
    if args.exact_steps:
        leg_steps, leg_warmup, config_steps = args.steps, args.warmup, args.steps
    if not args.no_forward:
        res["forward"] = measure_forward(torch, ssd, w, d, S, ws, z, steps=leg_steps, warmup=leg_warmup)
    if not args.no_forward and not args.no_options:
        res["backward_with_dt_frontend"] = measure_frontend(torch, ssd, w, d, S, ws, steps=leg_steps,
                                                            warmup=leg_warmup)
        # output gate: z ~ N(0, 1) (seeded), in the I/O dtype
        gz = torch.Generator().manual_seed(w.seed + 1)
        zg = torch.randn(tuple(d["x"].shape), generator=gz).to(d["x"].dtype).to(dev)
        # the forward's pre-gate y (outside the timed region), as the autograd function keeps it
        y_pre = ssd.ssd_fwd(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"], d.get("initial_states"),
                            d.get("seq_idx"), chunk_size=w.chunk, nseqs=S, workspace=ws, dt_bias=d["dt_bias"],
                            dt_softplus=True, z=zg, want_y_pre_gate=True)["y_pre_gate"]
        res["backward_with_dt_frontend_and_gate"] = measure_frontend(
            torch, ssd, w, d, S, ws, steps=leg_steps, warmup=leg_warmup, z=zg, y_pre=y_pre)
        res["backward_with_dt_frontend_and_gate_recompute"] = measure_frontend(
            torch, ssd, w, d, S, ws, steps=leg_steps, warmup=leg_warmup, z=zg)
        del zg, y_pre
    if not args.no_conv and not args.no_options:
        res["causal_conv1d"] = measure_conv1d(torch, steps=leg_steps, warmup=leg_warmup,
                                              dev=dev, cpu=not args.no_cpu_baseline)
    del d, ws
    torch.cuda.empty_cache()
    if not args.no_configs and args.workload is None:
        # the other workloads of the family (the pages' seqlens 2048 / 4096 and the packed
        # varlen case), each timed the same way
        res["configs"] = {}
        for name in ("bf16_L2048_H128", "bf16_B2_L4096_H128", "bf16_varlen7_L16384_N256"):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            crec = measure_backward(torch, ssd, WORKLOADS[name], config_steps, leg_warmup, dev)[0]
            res["configs"][name] = crec
            torch.cuda.empty_cache()
    if args.calibration_copy:
        calibration_copy(torch, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inputs, groups=args.cpu_groups or w.ngroups)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
