"""GPU: ragged batches (lengths) in ssd_chunk_scan_fwd and ssd_mixer_fwd.

The mojolearn.Mamba3Block forward(): row b is real at positions t < lengths[b]; every padding output is exactly
+0.0 and every real output equals the row run alone at its own length.  Checked: padding is +0.0 bit for bit (sign
included); real outputs equal the same call without lengths bit for bit, and the row run alone at its length bit
for bit on the sequential path (no workspace) and within the bf16 bar (0.03125) with the sequence split; and the
fp64 oracle on each row at its length.
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


def _mixer(lib, wl, prm, raw, L, lengths=None, ws=None, plan_bytes=None, rows=None):
    g = lambda t: None if t is None else t.to(DEV)
    sl = (lambda t: t) if rows is None else (lambda t: None if t is None else t[rows])
    cut = lambda t: None if t is None else sl(t)[:, :L].contiguous()
    return lib.ssd_mixer_fwd(g(cut(raw["xbc_raw"])), g(cut(raw["dt_raw"])), g(prm["conv_w"]), g(prm["A"]), H=wl.H,
                             P=wl.P, N=wl.N, G=wl.G, conv_b=g(prm.get("conv_b")), dt_bias=g(prm["dt_bias"]),
                             D=g(prm["D"]), z=g(cut(raw["z"])), lengths=g(lengths), workspace=ws)


def _ws(lib, wl, L, B, staged=True):
    f = lib.ssd_mixer_workspace_size if staged else lib.ssd_chunk_scan_workspace_size
    n = f(B, L, wl.H, wl.P, wl.N, wl.G, lib.SSD_BF16 if wl.dtype == "bf16" else lib.SSD_F32)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=DEV) if n else None


@pytest.mark.parametrize("plan", ["sequential", "staged_split", "fused"])
def test_mixer_ragged(gpu_lib, plan):
    wl = synth.Workload("ragged_mix", 4, 700, 8, 64, 64, 2, "bf16")
    _say(f"ragged mixer {plan}")
    prm = synth.params(wl, 21, conv_bias=True)
    raw = synth.raw_inputs(wl, 21)
    lens = torch.tensor([700, 1, 333, 64], dtype=torch.int32)
    ws = None
    if plan == "staged_split":
        ws = _ws(gpu_lib, wl, 700, 4)
    elif plan == "fused":
        ws = _ws(gpu_lib, wl, 700, 4, staged=False)
    y = _mixer(gpu_lib, wl, prm, raw, 700, lens, ws)
    y_full = _mixer(gpu_lib, wl, prm, raw, 700, None, ws)
    torch.cuda.synchronize()
    for b, n in enumerate(lens.tolist()):
        pad = y[b, n:]
        assert torch.equal(pad, torch.zeros_like(pad)) and not torch.signbit(pad).any(), f"row {b}: padding not +0.0"
        assert torch.equal(y[b, :n], y_full[b, :n]), f"row {b}: real outputs changed by lengths"
        alone_ws = None if plan == "sequential" else _ws(gpu_lib, wl, n, 1, staged=plan != "fused")
        ya = _mixer(gpu_lib, wl, prm, raw, n, None, alone_ws, rows=slice(b, b + 1))
        torch.cuda.synchronize()
        if plan == "sequential":
            assert torch.equal(ya[0], y[b, :n]), f"row {b}: differs from the row run alone"
        else:
            hp.assert_bf16(y[b, :n], ya[0], f"row {b} vs alone")
        # the oracle on the row at its length
        prm_c = {k: (None if v is None else v.cpu()) for k, v in prm.items()}
        cut = lambda t: t[b:b + 1, :n]
        yr, _, _, xr, _ = oracle.forward(cut(raw["xbc_raw"]), prm_c["conv_w"], prm_c["conv_b"], cut(raw["dt_raw"]),
                                         prm_c["dt_bias"], prm_c["A"], prm_c["D"], cut(raw["z"]), H=wl.H, P=wl.P,
                                         N=wl.N, G=wl.G, round_bf16=True)
        hp.assert_pipeline(y[b:b + 1, :n], yr, xr[..., :wl.H * wl.P], cut(raw["z"]), prm_c["D"], wl.H, wl.P,
                           f"row {b} vs oracle")


def test_scan_ragged_fp32(gpu_lib):
    """The scan call alone (fp32), lengths 0..L including 0 (all padding) and L."""
    wl = synth.Workload("ragged_scan", 4, 300, 4, 64, 32, 1, "f32", conv=False)
    _say("ragged scan fp32")
    inp = synth.scan_inputs(wl, 22)
    prm = synth.params(wl, 22)
    lens = torch.tensor([0, 300, 65, 129], dtype=torch.int32)
    g = lambda t: None if t is None else t.to(DEV)
    call = lambda L, rows, ln: gpu_lib.ssd_chunk_scan_fwd(
        g(inp["x"][rows, :L].contiguous()), g(inp["Bm"][rows, :L].contiguous()), g(inp["Cm"][rows, :L].contiguous()),
        g(inp["dt_raw"][rows, :L].contiguous()), g(prm["A"]), H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=g(prm["D"]),
        z=g(inp["z"][rows, :L].contiguous()), lengths=g(ln), dt_softplus=True, dt_bias=g(prm["dt_bias"]))
    y = call(300, slice(0, 4), lens)
    torch.cuda.synchronize()
    for b, n in enumerate(lens.tolist()):
        pad = y[b, n:]
        assert torch.equal(pad, torch.zeros_like(pad)) and not torch.signbit(pad).any()
        if n:
            ya = call(n, slice(b, b + 1), None)
            torch.cuda.synchronize()
            assert torch.equal(ya[0], y[b, :n]), f"row {b}"
            yr, _ = oracle.scan(hp.np64(inp["x"][b:b + 1, :n]), hp.np64(inp["Bm"][b:b + 1, :n]),
                                hp.np64(inp["Cm"][b:b + 1, :n]), hp.np64(inp["dt_raw"][b:b + 1, :n]),
                                hp.np64(prm["A"]), hp.np64(prm["D"]), hp.np64(inp["z"][b:b + 1, :n]), H=wl.H, P=wl.P,
                                N=wl.N, G=wl.G, dt_softplus=True, dt_bias=hp.np64(prm["dt_bias"]))
            hp.assert_fp32(y[b:b + 1, :n], yr, f"row {b} vs oracle")


def test_ragged_refusals(gpu_lib):
    wl = synth.Workload("ragged_ref", 1, 64, 4, 64, 32, 1, "bf16")
    prm = {k: (None if v is None else v.to(DEV)) for k, v in synth.params(wl, 1).items()}
    raw = {k: (None if v is None else v.to(DEV)) for k, v in synth.raw_inputs(wl, 1).items()}
    lens = torch.tensor([10], dtype=torch.int32, device=DEV)
    fs = torch.zeros(1, 4, 64, 32, device=DEV)
    with pytest.raises(gpu_lib.SSDError, match="lengths cannot be combined"):
        gpu_lib.ssd_mixer_fwd(raw["xbc_raw"], raw["dt_raw"], prm["conv_w"], prm["A"], H=4, P=64, N=32, G=1,
                              lengths=lens, final_state=fs)
