"""GPU parity: ssd_s6_scan_fwd (the Mamba-1 selective scan) against the fp64 oracle.

Bars: fp32 inputs, max |gpu - oracle| <= 1e-3 * RMS(oracle) per tensor (y and final state); bf16 inputs (the
oracle reads the same bf16 values widened to fp64), max |gpu - oracle| <= 0.03125.  Shapes span several
256-channel workgroups with a ragged last one, ragged lengths, every supported N, documents, carried states,
the D skip, the gate, both dt forms, and the sequence split (workspace) against the sequential pass.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import helpers as hp

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _oracle(inp, prm, *, softplus=True, gate=True, docs=None, h0=None, chan=None):
    """The fp64 oracle on the given channels (all if chan is None).  Returns y [B,L,Dsel], state [B,Dsel,N]."""
    sel = slice(None) if chan is None else chan
    c = lambda t: None if t is None else t.cpu()
    x = c(inp["x"])[:, :, sel]
    dt = c(inp["dt_raw"])[:, :, sel]
    z = c(inp["z"])[:, :, sel] if gate and inp["z"] is not None else None
    A = c(prm["A"])[sel]
    Dk = c(prm["D_skip"])[sel] if prm.get("D_skip") is not None else None
    db = c(prm["dt_bias"])[sel] if softplus else None
    h = None if h0 is None else c(h0)[:, sel]
    return oracle.s6(x, dt, A, c(inp["Bm"]), c(inp["Cm"]), D=Dk, z=z, doc_ids=c(docs), init_state=h,
                     dt_softplus=softplus, dt_bias=db, want_state=True)


def _run(lib, inp, prm, *, softplus=True, gate=True, docs=None, h0=None, split=False, final=True, dt=None):
    B, L, Dn = inp["x"].shape
    N = prm["A"].shape[1]
    g = lambda t: None if t is None else t.to(DEV)
    fs = torch.empty(B, Dn, N, device=DEV) if final else None
    ws = None
    if split:
        nb = lib.ssd_s6_workspace_size(B, L, Dn, N)
        ws = torch.empty(max(nb, 16) // 4 + 4, dtype=torch.float32, device=DEV) if nb else None
    y = lib.ssd_s6_scan_fwd(g(inp["x"]), g(inp["dt_raw"] if dt is None else dt), g(prm["A"]), g(inp["Bm"]),
                            g(inp["Cm"]), D_skip=g(prm.get("D_skip")), z=g(inp["z"]) if gate else None,
                            doc_ids=g(docs), init_state=g(h0), final_state=fs, dt_softplus=softplus,
                            dt_bias=g(prm["dt_bias"]) if softplus else None, workspace=ws)
    torch.cuda.synchronize()
    return y, fs


def _check(dtype, got, ref, name):
    if dtype == "f32":
        return hp.assert_fp32(got, ref, name)
    return hp.assert_bf16(got, ref, name)


def _wl(dtype, B, L, Dn, N, h0=False, gate=True):
    # D = H*P channels; H = Dn / 64 when that divides, else H = Dn with P = 1 (the generator only uses H*P)
    H, P = (Dn // 64, 64) if Dn % 64 == 0 else (Dn, 1)
    return synth.Workload(f"s6_{dtype}_{B}_{L}_{Dn}_{N}", B, L, H, P, N, 1, dtype, conv=False, gate=gate, h0=h0)


def _docs(wl, seed, L, mean_len):
    return synth.doc_ids(wl, seed, L=L, mean_len=mean_len)


CASES = [
    # dtype, B, L, D, N, docs, h0, gate, softplus
    ("f32", 2, 300, 320, 16, False, False, True, True),     # two workgroups, the second ragged (64 of 256)
    ("f32", 1, 1, 256, 16, False, True, True, True),        # a single token
    ("f32", 3, 777, 100, 8, True, True, False, True),       # fewer channels than a workgroup
    ("f32", 2, 513, 520, 32, True, False, True, False),     # N = 32, dt already activated
    ("bf16", 2, 1000, 768, 16, True, True, True, True),
    ("bf16", 1, 2049, 2048, 16, False, False, True, True),
    ("bf16", 4, 130, 264, 8, True, False, False, True),
    ("bf16", 2, 257, 512, 32, False, True, True, True),
]


@pytest.mark.parametrize("split", [False, True], ids=["single_pass", "seq_split"])
@pytest.mark.parametrize("dtype,B,L,Dn,N,docs,h0,gate,softplus", CASES)
def test_s6_vs_oracle(gpu_lib, dtype, B, L, Dn, N, docs, h0, gate, softplus, split):
    wl = _wl(dtype, B, L, Dn, N, h0=h0, gate=gate)
    _say(f"s6 {dtype} B={B} L={L} D={Dn} N={N} docs={docs} h0={h0} gate={gate} softplus={softplus} split={split}")
    prm = synth.s6_params(wl, 1)
    inp = synth.s6_inputs(wl, 1)
    if not softplus:                                   # an activated dt (>= 0) of the same spread
        inp["dt_raw"] = torch.nn.functional.softplus(inp["dt_raw"].float() - 2.5).to(inp["dt_raw"].dtype)
    ids = _docs(wl, 2, L, 150.0) if docs else None
    y, fs = _run(gpu_lib, inp, prm, softplus=softplus, gate=gate, docs=ids, h0=inp["h0"], split=split)
    yr, fr = _oracle(inp, prm, softplus=softplus, gate=gate, docs=ids, h0=inp["h0"])
    _check(dtype, y, yr, "y")
    _check(dtype, fs, fr, "final_state")


def test_s6_split_matches_sequential(gpu_lib):
    """The superchunk split agrees with the sequential pass to fp32 rounding (fp32 inputs, documents, state)."""
    wl = _wl("f32", 2, 4096, 512, 16, h0=True)
    _say("s6 split vs sequential")
    prm, inp = synth.s6_params(wl, 3), synth.s6_inputs(wl, 3)
    ids = _docs(wl, 3, wl.L, 700.0)
    assert gpu_lib.ssd_s6_workspace_size(wl.B, wl.L, 512, 16) > 0
    y1, f1 = _run(gpu_lib, inp, prm, docs=ids, h0=inp["h0"], split=False)
    y2, f2 = _run(gpu_lib, inp, prm, docs=ids, h0=inp["h0"], split=True)
    hp.assert_fp32(y2, y1, "y split vs sequential")
    hp.assert_fp32(f2, f1, "state split vs sequential")


def test_s6_in_place_state(gpu_lib):
    """final_state may be init_state itself, with and without the split."""
    wl = _wl("bf16", 2, 3000, 512, 16, h0=True)
    prm, inp = synth.s6_params(wl, 4), synth.s6_inputs(wl, 4)
    _say("s6 in-place state")
    yr, fr = _oracle(inp, prm, h0=inp["h0"])
    for split in (False, True):
        st = inp["h0"].to(DEV).clone()
        ws = None
        if split:
            ws = torch.empty(gpu_lib.ssd_s6_workspace_size(2, 3000, 512, 16) // 4 + 4, device=DEV)
        g = lambda t: t.to(DEV)
        y = gpu_lib.ssd_s6_scan_fwd(g(inp["x"]), g(inp["dt_raw"]), g(prm["A"]), g(inp["Bm"]), g(inp["Cm"]),
                                    D_skip=g(prm["D_skip"]), z=g(inp["z"]), init_state=st, final_state=st,
                                    dt_softplus=True, dt_bias=g(prm["dt_bias"]), workspace=ws)
        torch.cuda.synchronize()
        hp.assert_bf16(y, yr, f"y (split={split})")
        hp.assert_bf16(st, fr, f"in-place state (split={split})")


def test_s6_column_slices_and_chunked_calls(gpu_lib):
    """B and C as column slices of one x_proj-shaped row [dt_rank | B | C] (row stride 48 + 2N), and a sequence
    processed as two calls with the state carried equals one call (sequential pass: bit for bit)."""
    Dn, N, B, L = 384, 16, 2, 600
    wl = _wl("bf16", B, L, Dn, N)
    prm, inp = synth.s6_params(wl, 5), synth.s6_inputs(wl, 5)
    _say("s6 column slices and chunked calls")
    xproj = torch.zeros(B, L, 48 + 2 * N, dtype=torch.bfloat16)
    xproj[:, :, 48:48 + N] = inp["Bm"]
    xproj[:, :, 48 + N:] = inp["Cm"]
    xproj = xproj.to(DEV)
    g = lambda t: t.to(DEV)
    A, Dk, db = g(prm["A"]), g(prm["D_skip"]), g(prm["dt_bias"])
    x, dt, z = g(inp["x"]), g(inp["dt_raw"]), g(inp["z"])
    Bv, Cv = xproj[:, :, 48:48 + N], xproj[:, :, 48 + N:]
    fs = torch.empty(B, Dn, N, device=DEV)
    y = gpu_lib.ssd_s6_scan_fwd(x, dt, A, Bv, Cv, D_skip=Dk, z=z, final_state=fs, dt_softplus=True, dt_bias=db)
    yr, fr = _oracle(inp, prm)
    hp.assert_bf16(y, yr, "y with sliced B/C")
    hp.assert_bf16(fs, fr, "state with sliced B/C")
    # two calls: tokens [0, 250) then [250, 600) with the state carried
    cut = 250
    s1 = torch.empty(B, Dn, N, device=DEV)
    ya = gpu_lib.ssd_s6_scan_fwd(x[:, :cut].contiguous(), dt[:, :cut].contiguous(), A, inp["Bm"][:, :cut].to(DEV),
                                 inp["Cm"][:, :cut].to(DEV), D_skip=Dk, z=z[:, :cut].contiguous(), final_state=s1,
                                 dt_softplus=True, dt_bias=db)
    s2 = torch.empty(B, Dn, N, device=DEV)
    yb = gpu_lib.ssd_s6_scan_fwd(x[:, cut:].contiguous(), dt[:, cut:].contiguous(), A, inp["Bm"][:, cut:].to(DEV),
                                 inp["Cm"][:, cut:].to(DEV), D_skip=Dk, z=z[:, cut:].contiguous(), init_state=s1,
                                 final_state=s2, dt_softplus=True, dt_bias=db)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb], 1), y)
    assert torch.equal(s2, fs)


def test_s6_empty_and_state_passthrough(gpu_lib):
    """L = 0 copies init_state to final_state (or zeros without one); B = 0 is a no-op."""
    Dn, N = 256, 16
    wl = _wl("f32", 2, 0, Dn, N)
    prm = synth.s6_params(wl, 6)
    A = prm["A"].to(DEV)
    x = torch.empty(2, 0, Dn, device=DEV)
    bm = torch.empty(2, 0, N, device=DEV)
    h0 = torch.randn(2, Dn, N, device=DEV)
    fs = torch.full((2, Dn, N), 7.0, device=DEV)
    gpu_lib.ssd_s6_scan_fwd(x, x, A, bm, bm, init_state=h0, final_state=fs)
    torch.cuda.synchronize()
    assert torch.equal(fs, h0)
    gpu_lib.ssd_s6_scan_fwd(x, x, A, bm, bm, final_state=fs)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fs).item() == 0
    e = torch.empty(0, 5, Dn, device=DEV)
    gpu_lib.ssd_s6_scan_fwd(e, e, A, torch.empty(0, 5, N, device=DEV), torch.empty(0, 5, N, device=DEV))


def test_s6_refusals(gpu_lib):
    Dn, N, B, L = 256, 64, 1, 8
    A = torch.zeros(Dn, N, device=DEV)
    x = torch.zeros(B, L, Dn, device=DEV)
    bm = torch.zeros(B, L, N, device=DEV)
    with pytest.raises(gpu_lib.SSDError, match="N=64 is not supported"):
        gpu_lib.ssd_s6_scan_fwd(x, x, A, bm, bm)
    A16 = torch.zeros(Dn, 16, device=DEV)
    b16 = torch.zeros(B, L, 17, device=DEV)[:, :, 1:]    # misaligned base
    with pytest.raises(gpu_lib.SSDError, match="Bm=.*not 16-byte aligned"):
        gpu_lib.ssd_s6_scan_fwd(x, x, A16, b16, b16)
    big = torch.zeros(2, 4096, 512, device=DEV)
    bb = torch.zeros(2, 4096, 16, device=DEV)
    need = gpu_lib.ssd_s6_workspace_size(2, 4096, 512, 16)
    assert need > 0
    with pytest.raises(gpu_lib.SSDError, match="workspace_bytes"):
        gpu_lib.ssd_s6_scan_fwd(big, big, torch.zeros(512, 16, device=DEV), bb, bb,
                                workspace=torch.empty(need // 8, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("split", [False, True], ids=["single_pass", "seq_split"])
def test_s6_full_workload_sampled_channels(gpu_lib, split):
    """The Mamba-1 workload (B=5, L=8192, D=2048, N=16, bf16, gate), as the benchmark launches it (with the
    split), on 96 sampled channels spread over every workgroup, with documents and a carried state."""
    wl = synth.WORKLOADS["s6_bf16"].with_(h0=True)
    _say(f"s6 full workload split={split}")
    prm = synth.s6_params(wl, 0)
    inp = synth.s6_inputs(wl, 0, device=DEV)
    ids = synth.doc_ids(wl, 0)
    y, fs = _run(gpu_lib, inp, prm, docs=ids, h0=inp["h0"], split=split)
    rng = np.random.default_rng(7)
    chan = np.sort(rng.choice(wl.H * wl.P, 96, replace=False))
    chan[0], chan[-1] = 0, wl.H * wl.P - 1
    ct = torch.as_tensor(chan)
    yr, fr = _oracle(inp, prm, docs=ids, h0=inp["h0"], chan=ct)
    hp.assert_bf16(y[:, :, ct.to(DEV)], yr, "y sampled channels")
    hp.assert_bf16(fs[:, ct.to(DEV)], fr, "final state sampled channels")
