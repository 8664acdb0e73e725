"""Seeded synthetic inputs for the SSD mixer core.

This module only draws random numbers with the shapes and distributions of
the workloads; it holds none of the method's arithmetic.  Both the fp64
oracle (through the tests and the benchmark) and the HIP library are fed
from it, so that the two sides see identical values.

Workloads (shapes from the Mini-K3-1H-mamba2-n64-g8 model card,
"Architecture" and "Checkpoint and training": expand 2, 32 heads x 64
channels, state 64, 8 B/C groups, conv kernel 4, 8,192-token rows, local
batch 5; the packed-document variant from the same card's document-isolation
paragraph; chunk 64 from the mojolearn.Mamba3Block description):

  tiny_fp32          B=1,   L=256,  H=4,   P=64, N=16,  G=1, fp32, no conv, no gate
  mini_k3_bf16       B=5,   L=8192, H=32,  P=64, N=64,  G=8, bf16, conv k=4, gate
  mini_k3_packed     as mini_k3_bf16 plus int32 document ids
  large_layer_bf16   B=4,   L=4096, H=128, P=64, N=128, G=8, bf16, h0 carried in
  decode_fp32        B=256, H=64,   P=64,  N=128, G=1, fp32, 4096-token prefill
                     then single-token steps
  s6_bf16            the Mamba-1 selective scan (S6) on the same token batch:
                     B=5, L=8192, D=H*P=2048 channels, state N=16 (the Mamba
                     block default of the nanochat hybrid-blocks page,
                     "Mamba-Specific Parameters"), bf16, gate

Distributions: raw x columns ~ N(0,1); raw B and C columns ~ N(0, 1/N)
(variance); dt_raw ~ N(0,1); dt_bias ~ U(-4,-1); A = -exp(U(log 1, log 16));
D ~ N(0,1); z ~ N(0,1); conv weights ~ N(0, 1/4); conv bias absent in the
workloads, N(0, 1/4) in unit tests; h0 ~ N(0, 0.1) where carried; document
lengths ~ Geometric(1/1024) on {1, 2, ...}, the last truncated at L.

Every tensor has its own torch.Generator seeded from (seed, workload,
tensor name), so a test can regenerate any one tensor alone.  Values are
drawn in fp32 and, for bf16 workloads, rounded to bf16 (round to nearest
even) by torch's dtype conversion.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int
    dtype: str            # "f32" or "bf16": the input dtype of the path
    conv: bool = True     # causal conv prologue present
    K: int = 4
    gate: bool = True     # z gate present
    docs: bool = False    # packed documents
    h0: bool = False      # initial state carried in
    steps: int = 0        # decode steps after the prefill

    @property
    def conv_dim(self) -> int:
        return self.H * self.P + 2 * self.G * self.N

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 4, 64, 16, 1, "f32", conv=False, gate=False),
    "mini_k3_bf16": Workload("mini_k3_bf16", 5, 8192, 32, 64, 64, 8, "bf16"),
    "mini_k3_packed": Workload("mini_k3_packed", 5, 8192, 32, 64, 64, 8, "bf16", docs=True),
    "large_layer_bf16": Workload("large_layer_bf16", 4, 4096, 128, 64, 128, 8, "bf16", h0=True),
    "decode_fp32": Workload("decode_fp32", 256, 4096, 64, 64, 128, 1, "f32", steps=1024),
    "s6_bf16": Workload("s6_bf16", 5, 8192, 32, 64, 16, 1, "bf16", conv=False),
}


def _gen(seed: int, wl: Workload, tensor: str, device) -> torch.Generator:
    h = hashlib.sha256(f"{seed}/{wl.name}/{tensor}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def _normal(shape, std, seed, wl, tensor, device):
    g = _gen(seed, wl, tensor, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _uniform(shape, lo, hi, seed, wl, tensor, device):
    g = _gen(seed, wl, tensor, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def params(wl: Workload, seed: int = 0, device="cpu", conv_bias: bool = False) -> dict:
    """Per-head and conv parameters, all fp32 (the card keeps the Mamba control
    parameters in FP32).  A is returned as A = -exp(A_log)."""
    H = wl.H
    A_log = _uniform((H,), 0.0, math.log(16.0), seed, wl, "A_log", device)
    out = {
        "A": -torch.exp(A_log),
        "D": _normal((H,), 1.0, seed, wl, "D", device),
        "dt_bias": _uniform((H,), -4.0, -1.0, seed, wl, "dt_bias", device),
    }
    if wl.conv:
        out["conv_w"] = _normal((wl.conv_dim, wl.K), 0.5, seed, wl, "conv_w", device)
        out["conv_b"] = _normal((wl.conv_dim,), 0.5, seed, wl, "conv_b", device) if conv_bias else None
    return out


def doc_ids(wl: Workload, seed: int = 0, L: int | None = None, mean_len: float = 1024.0) -> torch.Tensor:
    """int32 [B, L]: ids 0, 1, 2, ... per row, run lengths ~ Geometric(1/mean_len), min 1."""
    L = wl.L if L is None else L
    g = _gen(seed, wl, "doc_len", "cpu")
    p = 1.0 / mean_len
    rows = []
    for _ in range(wl.B):
        ids = torch.empty(L, dtype=torch.int32)
        t, d = 0, 0
        while t < L:
            u = torch.rand((), generator=g, dtype=torch.float64).item()
            n = max(1, int(math.ceil(math.log1p(-u) / math.log1p(-p)))) if u > 0 else 1
            ids[t:t + n] = d
            t += n
            d += 1
        rows.append(ids)
    return torch.stack(rows)


def raw_inputs(wl: Workload, seed: int = 0, device="cpu", L: int | None = None, B: int | None = None) -> dict:
    """Pre-conv inputs of the mixer core.  xbc_raw [B,L,conv_dim] (columns x | B | C),
    dt_raw [B,L,H], z [B,L,H*P] (if gated), h0 [B,H,P,N] fp32 (if carried), all in the
    workload's dtype except h0."""
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    HP, GN = wl.H * wl.P, wl.G * wl.N
    sB = 1.0 / math.sqrt(wl.N)
    dt = wl.torch_dtype
    x = _normal((B, L, HP), 1.0, seed, wl, "x_raw", device)
    bm = _normal((B, L, GN), sB, seed, wl, "B_raw", device)
    cm = _normal((B, L, GN), sB, seed, wl, "C_raw", device)
    out = {"xbc_raw": torch.cat([x, bm, cm], dim=2).to(dt)}
    del x, bm, cm
    out["dt_raw"] = _normal((B, L, wl.H), 1.0, seed, wl, "dt_raw", device).to(dt)
    out["z"] = _normal((B, L, HP), 1.0, seed, wl, "z", device).to(dt) if wl.gate else None
    out["h0"] = (_normal((B, wl.H, wl.P, wl.N), math.sqrt(0.1), seed, wl, "h0", device)
                 if wl.h0 else None)
    return out


def scan_inputs(wl: Workload, seed: int = 0, device="cpu", L: int | None = None, B: int | None = None) -> dict:
    """Direct scan inputs (no conv in front): x [B,L,H*P], Bm/Cm [B,L,G*N], dt_raw [B,L,H]
    (the scan applies softplus with dt_bias), z, h0.  Same distributions as the raw columns."""
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    HP, GN = wl.H * wl.P, wl.G * wl.N
    sB = 1.0 / math.sqrt(wl.N)
    dt = wl.torch_dtype
    return {
        "x": _normal((B, L, HP), 1.0, seed, wl, "x", device).to(dt),
        "Bm": _normal((B, L, GN), sB, seed, wl, "Bm", device).to(dt),
        "Cm": _normal((B, L, GN), sB, seed, wl, "Cm", device).to(dt),
        "dt_raw": _normal((B, L, wl.H), 1.0, seed, wl, "dt_raw", device),
        "z": _normal((B, L, HP), 1.0, seed, wl, "z", device).to(dt) if wl.gate else None,
        "h0": (_normal((B, wl.H, wl.P, wl.N), math.sqrt(0.1), seed, wl, "h0", device)
               if wl.h0 else None),
    }


def step_inputs(wl: Workload, step: int, seed: int = 0, device="cpu", B: int | None = None) -> dict:
    """Raw inputs of decode token `step`: xbc_raw [B,conv_dim], dt_raw [B,H], z [B,H*P]."""
    B = wl.B if B is None else B
    HP, GN = wl.H * wl.P, wl.G * wl.N
    sB = 1.0 / math.sqrt(wl.N)
    dt = wl.torch_dtype
    x = _normal((B, HP), 1.0, seed, wl, f"step{step}/x", device)
    bm = _normal((B, GN), sB, seed, wl, f"step{step}/B", device)
    cm = _normal((B, GN), sB, seed, wl, f"step{step}/C", device)
    return {
        "xbc_raw": torch.cat([x, bm, cm], dim=1).to(dt),
        "dt_raw": _normal((B, wl.H), 1.0, seed, wl, f"step{step}/dt", device).to(dt),
        "z": _normal((B, HP), 1.0, seed, wl, f"step{step}/z", device).to(dt) if wl.gate else None,
    }


def s6_params(wl: Workload, seed: int = 0, device="cpu") -> dict:
    """Mamba-1 (S6) parameters over D = H*P channels, fp32: A [D, N] = -exp(A_log) with
    A_log ~ U(log 1, log 16) per (d, n), D skip [D] ~ N(0,1), dt_bias [D] ~ U(-4,-1)."""
    Dn = wl.H * wl.P
    A_log = _uniform((Dn, wl.N), 0.0, math.log(16.0), seed, wl, "s6/A_log", device)
    return {
        "A": -torch.exp(A_log),
        "D_skip": _normal((Dn,), 1.0, seed, wl, "s6/D", device),
        "dt_bias": _uniform((Dn,), -4.0, -1.0, seed, wl, "s6/dt_bias", device),
    }


def s6_inputs(wl: Workload, seed: int = 0, device="cpu", L: int | None = None, B: int | None = None) -> dict:
    """Mamba-1 scan inputs in the workload's dtype: x [B,L,D] ~ N(0,1), dt_raw [B,L,D] ~ N(0,1)
    (before softplus(dt + dt_bias)), Bm/Cm [B,L,N] ~ N(0,1/N), z [B,L,D] ~ N(0,1) if gated, and
    h0 [B,D,N] ~ N(0,0.1) fp32 if carried."""
    L = wl.L if L is None else L
    B = wl.B if B is None else B
    Dn = wl.H * wl.P
    sB = 1.0 / math.sqrt(wl.N)
    dt = wl.torch_dtype
    return {
        "x": _normal((B, L, Dn), 1.0, seed, wl, "s6/x", device).to(dt),
        "dt_raw": _normal((B, L, Dn), 1.0, seed, wl, "s6/dt", device).to(dt),
        "Bm": _normal((B, L, wl.N), sB, seed, wl, "s6/B", device).to(dt),
        "Cm": _normal((B, L, wl.N), sB, seed, wl, "s6/C", device).to(dt),
        "z": _normal((B, L, Dn), 1.0, seed, wl, "s6/z", device).to(dt) if wl.gate else None,
        "h0": _normal((B, Dn, wl.N), math.sqrt(0.1), seed, wl, "s6/h0", device) if wl.h0 else None,
    }
