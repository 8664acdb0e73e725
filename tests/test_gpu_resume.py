"""GPU: chunk-resume decode (ssd_resume_fwd) continues the sequential forward bit for bit.

A prefill (ssd_conv_fwd + ssd_chunk_scan_fwd without a workspace) over a multiple of 64 tokens hands its
final state and conv state to ssd_resume_fwd, which then decodes token by token (or appends several tokens at
once).  Every decode output must equal the one-call forward over the whole sequence exactly (torch.equal:
+0 and -0 compare equal), and at every chunk end the resumed state must equal that forward's final state at
the same length.  One case is also checked against the fp64 oracle.
"""
import pytest
import torch

import oracle
import synth
from tests import helpers as hp

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def forward(lib, wl, raw, prm, L, conv_state=None, h0=None):
    """The sequential forward over the first L tokens: y, final state, conv state out."""
    HP, GN = wl.H * wl.P, wl.G * wl.N
    B = raw["xbc_raw"].shape[0]
    sl = lambda t: None if t is None else t[:, :L].contiguous()
    cs = torch.empty(B, 3, wl.conv_dim, dtype=wl.torch_dtype, device=DEV)
    xbc, dt = lib.ssd_conv_fwd(sl(raw["xbc_raw"]), prm["conv_w"], H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                               conv_b=prm.get("conv_b"), dt_raw=sl(raw["dt_raw"]), dt_bias=prm["dt_bias"],
                               conv_state_in=conv_state, conv_state_out=cs)
    fs = torch.empty(B, wl.H, wl.P, wl.N, dtype=torch.float32, device=DEV)
    y = lib.ssd_chunk_scan_fwd(xbc[..., :HP], xbc[..., HP:HP + GN], xbc[..., HP + GN:], dt, prm["A"], H=wl.H, P=wl.P,
                               N=wl.N, G=wl.G, D=prm["D"], z=sl(raw["z"]), init_state=h0, final_state=fs)
    return y, fs, cs


class Resumer:
    """The caller-owned state of chunk-resume decoding."""

    def __init__(self, lib, wl, prm, B, chunk_state, conv_state):
        self.lib, self.wl, self.prm = lib, wl, prm
        self.pos = 0
        self.state = chunk_state.clone()
        self.conv = conv_state.clone()
        self.xbc = torch.zeros(B, 64, wl.conv_dim, dtype=wl.torch_dtype, device=DEV)
        self.dt = torch.zeros(B, 64, wl.H, dtype=torch.float32, device=DEV)
        self.z = torch.zeros(B, 64, wl.H * wl.P, dtype=wl.torch_dtype, device=DEV) if wl.gate else None
        self.yw = torch.empty(B, 64, wl.H * wl.P, dtype=torch.float32, device=DEV)

    def append(self, raw, t0, n):
        wl, prm = self.wl, self.prm
        sl = lambda t: None if t is None else t[:, t0:t0 + n].contiguous()
        y = self.lib.ssd_resume_fwd(sl(raw["xbc_raw"]), sl(raw["dt_raw"]), prm["conv_w"], prm["A"], self.conv,
                                    self.xbc, self.dt, self.state, self.yw, pos=self.pos, H=wl.H, P=wl.P, N=wl.N,
                                    G=wl.G, z=sl(raw["z"]), chunk_z=self.z, conv_b=prm.get("conv_b"),
                                    dt_bias=prm["dt_bias"], D=prm["D"])
        self.pos = (self.pos + n) % 64
        return y


def setup(wl, seed, L, h0=False):
    prm = {k: (None if v is None else v.to(DEV)) for k, v in synth.params(wl, seed, conv_bias=True).items()}
    raw = synth.raw_inputs(wl.with_(L=L), seed, device=DEV)
    h = torch.randn(wl.B, wl.H, wl.P, wl.N, generator=torch.Generator().manual_seed(seed)).to(DEV) * 0.3 if h0 else None
    return prm, raw, h


CASES = [
    # dtype, H, N, G, prefill length, decode steps
    ("f32", 8, 128, 1, 256, 150),      # the decode workload's head layout, fewer heads
    ("bf16", 8, 64, 2, 128, 140),      # four heads per workgroup in the bf16 scan
    ("bf16", 4, 32, 1, 64, 70),
]


@pytest.mark.parametrize("dtype,H,N,G,L0,steps", CASES)
def test_resume_decode_bitwise(gpu_lib, dtype, H, N, G, L0, steps):
    wl = synth.Workload("resume_" + dtype, 3, L0, H, 64, N, G, dtype)
    _say(f"resume decode {dtype} H={H} N={N} G={G} prefill={L0} steps={steps}")
    prm, raw, h0 = setup(wl, 31, L0 + steps, h0=True)
    y_ref, _, _ = forward(gpu_lib, wl, raw, prm, L0 + steps, h0=h0)
    _, fs, cs = forward(gpu_lib, wl, raw, prm, L0, h0=h0)
    rs = Resumer(gpu_lib, wl, prm, wl.B, fs, cs)
    ys = []
    for s in range(steps):
        ys.append(rs.append(raw, L0 + s, 1))
        if rs.pos == 0:                                  # a chunk just completed
            _, f_at, _ = forward(gpu_lib, wl, raw, prm, L0 + s + 1, h0=h0)
            assert torch.equal(rs.state, f_at), f"state after chunk end at token {L0 + s + 1}"
    torch.cuda.synchronize()
    y = torch.cat(ys, 1)
    assert torch.equal(y, y_ref[:, L0:]), hp.report("resumed decode y vs one forward", y, y_ref[:, L0:])


def test_resume_ragged_prefill_and_multi_token(gpu_lib):
    """A prefill of 64 k + 37 tokens (the last 37 through ssd_resume_fwd), then appends of 1, 5, 20 and 1 tokens
    crossing a chunk end: every output equals the one-call forward bit for bit, and the oracle within the bf16
    bars."""
    wl = synth.Workload("resume_ragged", 2, 128, 8, 64, 64, 2, "bf16")
    L0, lead = 128, 37
    plan = [lead, 1, 5, 20, 1]                           # 37 + 1 + 5 + 20 = 63, then the chunk's last token
    plan += [1, 9]                                       # into the next chunk
    total = L0 + sum(plan)
    _say(f"resume ragged prefill, total {total}")
    prm, raw, h0 = setup(wl, 32, total)
    y_ref, f_ref, _ = forward(gpu_lib, wl, raw, prm, total)
    _, fs, cs = forward(gpu_lib, wl, raw, prm, L0)
    rs = Resumer(gpu_lib, wl, prm, wl.B, fs, cs)
    ys, t = [], L0
    for n in plan:
        ys.append(rs.append(raw, t, n))
        t += n
    torch.cuda.synchronize()
    y = torch.cat(ys, 1)
    assert torch.equal(y, y_ref[:, L0:]), hp.report("resumed y vs one forward", y, y_ref[:, L0:])
    # against the fp64 oracle, the whole sequence in one pass
    prm_c = {k: (None if v is None else v.cpu()) for k, v in prm.items()}
    for b in range(wl.B):
        sl = slice(b, b + 1)
        yr, _, _, xr, _ = oracle.forward(raw["xbc_raw"][sl].cpu(), prm_c["conv_w"], prm_c["conv_b"],
                                         raw["dt_raw"][sl].cpu(), prm_c["dt_bias"], prm_c["A"], prm_c["D"],
                                         raw["z"][sl].cpu(), H=wl.H, P=wl.P, N=wl.N, G=wl.G, round_bf16=True)
        hp.assert_pipeline(y[sl], yr[:, L0:], xr[:, L0:, :wl.H * wl.P], raw["z"][sl, L0:].cpu(), prm_c["D"], wl.H,
                           wl.P, f"resumed y row {b}")


def test_resume_decode_workload_shape(gpu_lib):
    """The decode workload's shape (H = 64, P = 64, N = 128, one group, fp32) on 4 sequences: a 4096-token
    prefill, then 64 resumed decode steps (one full chunk) equal the 4160-token forward bit for bit, and so does
    the state at the chunk end."""
    wl = synth.WORKLOADS["decode_fp32"].with_(B=4)
    steps = 64
    _say("resume decode workload shape")
    prm, raw, _ = setup(wl, 33, wl.L + steps)
    y_ref, f_ref, _ = forward(gpu_lib, wl, raw, prm, wl.L + steps)
    _, fs, cs = forward(gpu_lib, wl, raw, prm, wl.L)
    rs = Resumer(gpu_lib, wl, prm, wl.B, fs, cs)
    ys = [rs.append(raw, wl.L + s, 1) for s in range(steps)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(ys, 1), y_ref[:, wl.L:])
    assert rs.pos == 0 and torch.equal(rs.state, f_ref)


def test_resume_decode_workload_full(gpu_lib):
    """The decode workload in full: B = 256 sequences, H = 64, P = 64, N = 128, one group, fp32, a 4096-token
    prefill and then all 1024 decode steps through ssd_resume_fwd, one token per call.  Every decode output of
    every sequence equals the one-call 5120-token forward bit for bit, and so does the resumed state at the
    first, a middle and the last chunk end (the forward's final state at those lengths)."""
    wl = synth.WORKLOADS["decode_fp32"]
    steps = wl.steps
    _say(f"resume decode workload full: B={wl.B} prefill={wl.L} steps={steps}")
    prm, raw, _ = setup(wl, 35, wl.L + steps)
    y_ref, _, _ = forward(gpu_lib, wl, raw, prm, wl.L + steps)
    _, fs, cs = forward(gpu_lib, wl, raw, prm, wl.L)
    rs = Resumer(gpu_lib, wl, prm, wl.B, fs, cs)
    del fs, cs
    checked = {64, 512, steps}
    ys = []
    for s in range(steps):
        ys.append(rs.append(raw, wl.L + s, 1))
        if s + 1 in checked:
            assert rs.pos == 0
            _, f_at, _ = forward(gpu_lib, wl, raw, prm, wl.L + s + 1)
            assert torch.equal(rs.state, f_at), f"state after chunk end at token {wl.L + s + 1}"
            del f_at
            _say(f"  state equal after {s + 1} steps")
    torch.cuda.synchronize()
    y = torch.cat(ys, 1)
    assert torch.equal(y, y_ref[:, wl.L:]), hp.report("resumed decode y vs one forward", y, y_ref[:, wl.L:])
    del raw, y_ref, y, ys, rs
    torch.cuda.empty_cache()


def test_resume_refusals(gpu_lib):
    wl = synth.Workload("resume_ref", 1, 64, 4, 64, 32, 1, "bf16")
    prm, raw, _ = setup(wl, 34, 70)
    rs = Resumer(gpu_lib, wl, prm, 1, torch.zeros(1, 4, 64, 32, device=DEV),
                 torch.zeros(1, 3, wl.conv_dim, dtype=torch.bfloat16, device=DEV))
    rs.pos = 60
    with pytest.raises(gpu_lib.SSDError, match="pos \\+ n = 66"):
        rs.append(raw, 0, 6)
    rs.pos = 64
    with pytest.raises(gpu_lib.SSDError, match="pos=64"):
        rs.append(raw, 0, 1)
