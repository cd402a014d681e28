"""Seeded synthetic inputs for the SSD backward.

This module only draws random numbers with the value distributions of the
Mamba-2 layer's inputs; it contains none of the layer's arithmetic.  Both the
GPU tests/benchmark and the fp64 oracle read the tensors it returns.

Recipe (shapes and distributions of the workloads the deterministic-backward
page benchmarks at seqlens 2048 / 4096 / 16384; the model dimensions of that
page's preset are not published, so these stand in for them):

* draw order: x, B, C, dy, z_dt, u_bias, u_A, D, h0, lengths
* x, dy, B, C ~ N(0, 1); B and C scaled by 1/sqrt(N) before rounding when
  ``scale_bc`` is set; then rounded to the I/O dtype (bf16 or fp32)
* dt = softplus(z + dt_bias[h]), z ~ N(0, 0.5^2), dt_bias = log(expm1(u)),
  u ~ U[1e-3, 1e-1] per head  (dt is the already-activated step)
* A = -exp(U[0, ln 16]) per head, D ~ N(0, 1) per head
* packed variable-length batches: lengths = min_len + a seeded split of the
  remaining tokens, marked by seq_idx; initial states ~ N(0, h0_std^2)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    chunk: int
    dtype: str            # "bf16" or "f32": dtype of x, B, C, dy (and dx, dB, dC)
    seed: int
    scale_bc: bool = True
    nseqs_packed: int = 0  # >0: one packed row of this many sequences, seq_idx given
    min_len: int = 512
    h0_std: float = 0.0    # >0: per-sequence initial states are drawn
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads of the benchmark family (small parity case first).
WORKLOADS = {
    "tiny_f32_L256": Workload("tiny_f32_L256", batch=1, seqlen=256, nheads=4, headdim=16,
                              ngroups=1, dstate=16, chunk=64, dtype="f32", seed=1000,
                              scale_bc=False),
    "bf16_L2048_H128": Workload("bf16_L2048_H128", batch=1, seqlen=2048, nheads=128, headdim=64,
                                ngroups=8, dstate=128, chunk=256, dtype="bf16", seed=1001),
    "bf16_B2_L4096_H128": Workload("bf16_B2_L4096_H128", batch=2, seqlen=4096, nheads=128,
                                   headdim=64, ngroups=8, dstate=128, chunk=256, dtype="bf16",
                                   seed=1002),
    "bf16_L16384_H128": Workload("bf16_L16384_H128", batch=1, seqlen=16384, nheads=128,
                                 headdim=64, ngroups=8, dstate=128, chunk=256, dtype="bf16",
                                 seed=1003),
    "bf16_varlen7_L16384_N256": Workload("bf16_varlen7_L16384_N256", batch=1, seqlen=16384,
                                         nheads=64, headdim=64, ngroups=1, dstate=256, chunk=256,
                                         dtype="bf16", seed=1004, nseqs_packed=7, min_len=512,
                                         h0_std=0.1),
}

HEADLINE = "bf16_L16384_H128"


def _round(t: torch.Tensor, dtype) -> torch.Tensor:
    return t.to(dtype).contiguous()


def seq_lengths(total: int, nseqs: int, min_len: int, gen: torch.Generator) -> list[int]:
    """nseqs lengths >= min_len summing to total: min_len + a uniform split of the rest."""
    rest = total - nseqs * min_len
    if rest < 0:
        raise ValueError("sequence lengths do not fit")
    cuts = torch.randint(0, rest + 1, (nseqs - 1,), generator=gen).sort().values.tolist()
    edges = [0] + cuts + [rest]
    return [min_len + edges[i + 1] - edges[i] for i in range(nseqs)]


def seq_idx_from_lengths(lengths: list[int]) -> torch.Tensor:
    return torch.repeat_interleave(torch.arange(len(lengths), dtype=torch.int32),
                                   torch.tensor(lengths)).reshape(1, -1).contiguous()


def make_inputs(w: Workload, lengths: Optional[list[int]] = None) -> dict:
    """CPU tensors: x, dt, A, B, C, D, dy (+ initial_states, seq_idx when packed), and
    dt_raw, dt_bias: the draws dt is formed from (dt = softplus(dt_raw + dt_bias)).

    x/B/C/dy are in the workload's I/O dtype, dt/A/D/initial_states are fp32,
    seq_idx int32.  ``lengths`` overrides the drawn packed lengths.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    b, L, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    io = w.torch_dtype
    bc_scale = 1.0 / math.sqrt(N) if w.scale_bc else 1.0
    x = torch.randn((b, L, H, P), generator=g)
    Bm = torch.randn((b, L, G, N), generator=g) * bc_scale
    Cm = torch.randn((b, L, G, N), generator=g) * bc_scale
    dy = torch.randn((b, L, H, P), generator=g)
    z = torch.randn((b, L, H), generator=g) * 0.5
    u_bias = torch.rand((H,), generator=g, dtype=torch.float64) * (1e-1 - 1e-3) + 1e-3
    u_A = torch.rand((H,), generator=g) * math.log(16.0)
    D = torch.randn((H,), generator=g)
    dt_bias = torch.log(torch.expm1(u_bias)).to(torch.float32)
    dt = torch.nn.functional.softplus(z + dt_bias).to(torch.float32).contiguous()
    A = (-torch.exp(u_A)).to(torch.float32).contiguous()
    out = {"x": _round(x, io), "dt": dt, "A": A, "B": _round(Bm, io), "C": _round(Cm, io),
           "D": D.to(torch.float32).contiguous(), "dy": _round(dy, io),
           "initial_states": None, "seq_idx": None,
           # the same step before its front-end: dt = softplus(dt_raw + dt_bias)
           "dt_raw": z.to(torch.float32).contiguous(), "dt_bias": dt_bias.contiguous()}
    if w.nseqs_packed:
        if b != 1:
            raise ValueError("packed workloads use batch 1")
        h0 = torch.randn((w.nseqs_packed, H, P, N), generator=g) * w.h0_std
        if lengths is None:
            lengths = seq_lengths(L, w.nseqs_packed, w.min_len, g)
        out["seq_idx"] = seq_idx_from_lengths(lengths)
        out["initial_states"] = h0.to(torch.float32).contiguous() if w.h0_std > 0 else None
        out["lengths"] = lengths
    return out


def to_f64_numpy(inputs: dict) -> dict:
    """The exact values the GPU receives, upcast to fp64 numpy (seq_idx stays int32)."""
    out = {}
    for k, v in inputs.items():
        if v is None or k == "lengths":
            out[k] = v
        elif k == "seq_idx":
            out[k] = v.numpy()
        else:
            out[k] = v.to(torch.float64).numpy()
    return out


# Depthwise causal convolution over the Mamba-2 block's xBC channels
# (channels = nheads * headdim + 2 * ngroups * dstate of the SSD workload it
# feeds).  Draws: x, dout ~ N(0, 1) in the I/O dtype; the filter w and bias
# ~ U(-1/sqrt(width), 1/sqrt(width)) in fp32 (the usual fan-in bound of a
# depthwise filter of that width); packed rows reuse seq_lengths.
@dataclass(frozen=True)
class ConvWorkload:
    name: str
    batch: int
    seqlen: int
    channels: int
    width: int
    dtype: str
    seed: int
    activation: str = "silu"
    nseqs_packed: int = 0
    min_len: int = 512

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def scaled(self, **kw) -> "ConvWorkload":
        return replace(self, **kw)


CONV_WORKLOADS = {
    "conv_tiny_f32": ConvWorkload("conv_tiny_f32", batch=2, seqlen=200, channels=96, width=4, dtype="f32",
                                  seed=2000),
    # the xBC convolution of bf16_L16384_H128: 128*64 + 2*8*128 channels
    "conv_bf16_L16384_C10240": ConvWorkload("conv_bf16_L16384_C10240", batch=1, seqlen=16384, channels=10240,
                                            width=4, dtype="bf16", seed=2001),
    # the xBC convolution of bf16_varlen7_L16384_N256: 64*64 + 2*1*256 channels, 7 packed sequences
    "conv_bf16_varlen7_L16384_C4608": ConvWorkload("conv_bf16_varlen7_L16384_C4608", batch=1, seqlen=16384,
                                                   channels=4608, width=4, dtype="bf16", seed=2002,
                                                   nseqs_packed=7),
}

CONV_HEADLINE = "conv_bf16_L16384_C10240"


def make_conv_inputs(w: ConvWorkload, lengths: Optional[list[int]] = None) -> dict:
    """CPU tensors: x, dout (I/O dtype, (batch, seqlen, channels)), weight (channels, width) and
    bias (channels) in fp32, seq_idx (int32) and lengths when packed."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    b, L, C, W = w.batch, w.seqlen, w.channels, w.width
    io = w.torch_dtype
    x = torch.randn((b, L, C), generator=g)
    dout = torch.randn((b, L, C), generator=g)
    bound = 1.0 / math.sqrt(W)
    weight = (torch.rand((C, W), generator=g) * 2 - 1) * bound
    bias = (torch.rand((C,), generator=g) * 2 - 1) * bound
    out = {"x": _round(x, io), "dout": _round(dout, io), "weight": weight.contiguous(), "bias": bias.contiguous(),
           "seq_idx": None}
    if w.nseqs_packed:
        if b != 1:
            raise ValueError("packed workloads use batch 1")
        if lengths is None:
            lengths = seq_lengths(L, w.nseqs_packed, w.min_len, g)
        out["seq_idx"] = seq_idx_from_lengths(lengths)
        out["lengths"] = lengths
    return out
