"""GPU parity of ssd_step: a prefill followed by single-token steps against the
fp64 oracle's one pass over all tokens; determinism and batch invariance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import helpers as hp
from tests.test_gpu_conv_scan import gpu_forward

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def decode_run(gpu_lib, wl, prm, raw, steps, seed, gen_device):
    """GPU prefill over raw, then `steps` ssd_step calls (step inputs drawn on gen_device, the same device the
    oracle side draws them on); returns (y_prefill, [y_step], ssm, conv)."""
    y, fs, cs, _, _ = gpu_forward(gpu_lib, wl, raw, prm)
    ys = []
    g = lambda t: None if t is None else t.to(DEV)
    for s in range(steps):
        st = synth.step_inputs(wl, s, seed, device=gen_device, B=raw["xbc_raw"].shape[0])
        st = {k: g(v) for k, v in st.items()}
        ys.append(gpu_lib.ssd_step(st["xbc_raw"], st["dt_raw"], g(prm["conv_w"]), g(prm["A"]), cs, fs, H=wl.H,
                                   P=wl.P, N=wl.N, G=wl.G, z=st["z"], conv_b=g(prm["conv_b"]),
                                   dt_bias=g(prm["dt_bias"]), D=g(prm["D"])))
    torch.cuda.synchronize()
    return y, ys, fs, cs


def oracle_single_pass(wl, prm, raw, steps, seed, rows, device):
    """Oracle forward over prefill ++ step tokens for the given batch rows."""
    st = [synth.step_inputs(wl, s, seed, device=device, B=raw["xbc_raw"].shape[0]) for s in range(steps)]
    sel = lambda t: t[rows].cpu()
    xbc = torch.cat([sel(raw["xbc_raw"])] + [sel(s["xbc_raw"])[:, None] for s in st], 1)
    dtr = torch.cat([sel(raw["dt_raw"])] + [sel(s["dt_raw"])[:, None] for s in st], 1)
    z = torch.cat([sel(raw["z"])] + [sel(s["z"])[:, None] for s in st], 1)
    return oracle.forward(xbc, prm["conv_w"], prm["conv_b"], dtr, prm["dt_bias"], prm["A"], prm["D"], z, H=wl.H,
                          P=wl.P, N=wl.N, G=wl.G, round_bf16=(wl.dtype == "bf16"))


@pytest.mark.parametrize("dtype,N,G,H,L,steps", [
    ("f32", 128, 1, 8, 200, 24),
    ("f32", 16, 2, 4, 64, 10),
    ("bf16", 64, 2, 8, 130, 12),
    # H*P rows that leave the last round of the step's state sweep partly empty
    ("f32", 64, 1, 3, 100, 8),
    ("bf16", 128, 1, 1, 70, 6),
    ("f32", 16, 1, 1, 65, 5),
    # N = 32 (8 lanes per state row); one head per group (H/G = 1); three heads per group
    ("bf16", 32, 3, 3, 90, 7),
    ("f32", 32, 2, 6, 75, 6),
])
def test_prefill_then_steps_small(gpu_lib, dtype, N, G, H, L, steps):
    wl = synth.Workload("dec_" + dtype, 3, L, H, 64, N, G, dtype, steps=steps)
    _say(f"decode small {dtype} N={N} G={G} H={H} L={L} steps={steps}")
    prm = synth.params(wl, 7, conv_bias=True)
    raw = synth.raw_inputs(wl, 7)
    y, ys, fs, cs = decode_run(gpu_lib, wl, prm, raw, steps, 7, "cpu")
    rows = list(range(wl.B))
    yr, fr, cr, xr, _ = oracle_single_pass(wl, prm, raw, steps, 7, rows, "cpu")
    yall = torch.cat([y.cpu()] + [s.cpu()[:, None] for s in ys], 1)
    if dtype == "f32":
        hp.assert_fp32(yall, yr, "prefill ++ decode y")
        hp.assert_fp32(fs, fr, "ssm state")
    else:
        hp.assert_pipeline(yall, yr, xr[..., :H * 64], torch.cat([raw["z"]] + [synth.step_inputs(wl, s, 7)["z"][:, None] for s in range(steps)], 1),
                           prm["D"], H, 64, "prefill ++ decode y")
        hp.assert_bf16(fs, fr, "ssm state")
    np.testing.assert_array_equal(hp.np64(cs), cr)


def test_decode_workload_full(gpu_lib):
    """B=256, H=64, P=64, N=128, G=1, fp32: a 4096-token prefill, then 1024 steps; sampled rows against
    the oracle's single 5120-token pass."""
    wl = synth.WORKLOADS["decode_fp32"]
    _say("decode workload: prefill 256 x 4096")
    prm = synth.params(wl, 0)
    raw = synth.raw_inputs(wl, 0, device=DEV)
    y, ys, fs, cs = decode_run(gpu_lib, wl, prm, raw, wl.steps, 0, DEV)
    _say("decode workload: oracle rows")
    rows = [0, 137]
    yr, fr, cr, _, _ = oracle_single_pass(wl, prm, raw, wl.steps, 0, rows, DEV)
    yall = torch.cat([y[rows].cpu()] + [s[rows].cpu()[:, None] for s in ys], 1)
    hp.assert_fp32(yall, yr, "prefill ++ 1024 decode steps, y")
    hp.assert_fp32(fs[rows], fr, "ssm state after 5120 tokens")
    np.testing.assert_array_equal(hp.np64(cs[rows]), cr)


def test_step_deterministic_and_batch_invariant(gpu_lib):
    wl = synth.WORKLOADS["decode_fp32"]
    _say("step determinism / batch invariance")
    prm = synth.params(wl, 1)
    g = lambda t: None if t is None else t.to(DEV)
    gen = torch.Generator(device=DEV).manual_seed(3)
    ssm0 = torch.randn(wl.B, wl.H, wl.P, wl.N, generator=gen, device=DEV) * 0.3
    conv0 = torch.randn(wl.B, 3, wl.conv_dim, generator=gen, device=DEV)
    st = synth.step_inputs(wl, 0, 1, device=DEV)

    def call(rows, ssm, conv):
        return gpu_lib.ssd_step(st["xbc_raw"][rows].contiguous(), st["dt_raw"][rows].contiguous(), g(prm["conv_w"]),
                                g(prm["A"]), conv, ssm, H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                                z=st["z"][rows].contiguous(), dt_bias=g(prm["dt_bias"]), D=g(prm["D"]))

    full = slice(0, wl.B)
    s1, c1 = ssm0.clone(), conv0.clone()
    y1 = call(full, s1, c1)
    s2, c2 = ssm0.clone(), conv0.clone()
    y2 = call(full, s2, c2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2) and torch.equal(c1, c2)
    half = wl.B // 2
    lo, hi = slice(0, half), slice(half, wl.B)
    sl, cl = ssm0[lo].clone(), conv0[lo].clone()
    sh, ch = ssm0[hi].clone(), conv0[hi].clone()
    yl = call(lo, sl, cl)
    yh = call(hi, sh, ch)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([yl, yh]), y1)
    assert torch.equal(torch.cat([sl, sh]), s1)
    assert torch.equal(torch.cat([cl, ch]), c1)
