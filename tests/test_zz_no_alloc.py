"""GPU: ssd_chunk_scan_fwd_static (the scan's split workspace in the library's static scratch) against
ssd_chunk_scan_fwd with a caller workspace of ssd_chunk_scan_workspace_size() bytes: bit for bit, on two calls
in a row (the second smaller, so it runs over what the first left in the scratch), plus the sizes that need no
workspace and an in-place state."""
import pytest
import torch

import synth
from tests import helpers as hp

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _inputs(wl, seed, docs, h0):
    inp = {k: (None if v is None else v.to(DEV)) for k, v in synth.scan_inputs(wl, seed).items()}
    prm = {k: (None if v is None else v.to(DEV)) for k, v in synth.params(wl, seed).items()}
    ids = synth.doc_ids(wl, seed, mean_len=700.0).to(DEV) if docs else None
    if not h0:
        inp["h0"] = None
    return inp, prm, ids


def _run(lib, wl, inp, prm, ids, static, in_place=False):
    fs = torch.full((wl.B, wl.H, wl.P, wl.N), 7.0, device=DEV)
    h0 = inp["h0"]
    if in_place:
        fs.copy_(h0)
        h0 = fs
    kw = dict(H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=prm["D"], z=inp["z"], doc_ids=ids, init_state=h0, final_state=fs,
              dt_softplus=True, dt_bias=prm["dt_bias"])
    if static:
        y = lib.ssd_chunk_scan_fwd_static(inp["x"], inp["Bm"], inp["Cm"], inp["dt_raw"].float(), prm["A"], **kw)
    else:
        n = lib.ssd_chunk_scan_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, 1 if wl.dtype == "bf16" else 0)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
        y = lib.ssd_chunk_scan_fwd(inp["x"], inp["Bm"], inp["Cm"], inp["dt_raw"].float(), prm["A"], workspace=ws,
                                   **kw)
    torch.cuda.synchronize()
    return y, fs


def _check(lib, wl, seed, docs, h0, in_place=False, expect_split=True):
    code = 1 if wl.dtype == "bf16" else 0
    need = lib.ssd_chunk_scan_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, code)
    assert (need > 0) == expect_split and need <= lib.SSD_STATIC_SCRATCH_BYTES, need
    _say(f"static scratch {wl.dtype} B={wl.B} L={wl.L} H={wl.H} N={wl.N} G={wl.G} workspace={need}")
    inp, prm, ids = _inputs(wl, seed, docs, h0)
    y1, f1 = _run(lib, wl, inp, prm, ids, static=True, in_place=in_place)
    y0, f0 = _run(lib, wl, inp, prm, ids, static=False, in_place=in_place)
    assert torch.equal(y1, y0), hp.report("static vs caller workspace y", y1, y0)
    assert torch.equal(f1, f0), hp.report("static vs caller workspace final_state", f1, f0)


def test_static_scratch_two_calls_second_smaller(gpu_lib):
    """The Mini-K3 workload (B=5, L=8192, H=32, N=64, G=8, bf16; 15.7 MB of workspace), then a smaller packed
    call with an initial state (a different split over less of the scratch)."""
    _check(gpu_lib, synth.WORKLOADS["mini_k3_bf16"], 41, docs=False, h0=False)
    _check(gpu_lib, synth.Workload("static_small", 2, 3000, 8, 64, 64, 2, "bf16", docs=True, h0=True), 42,
           docs=True, h0=True)


def test_static_scratch_fp32_in_place_and_no_split(gpu_lib):
    """fp32 with the split and final_state aliasing init_state; then sizes that need no workspace."""
    _check(gpu_lib, synth.Workload("static_f32", 2, 2048, 4, 64, 64, 1, "f32", h0=True), 43, docs=True, h0=True,
           in_place=True)
    _check(gpu_lib, synth.Workload("static_short", 2, 64, 4, 64, 32, 2, "bf16", h0=True), 44, docs=False, h0=True,
           expect_split=False)


def test_static_scratch_refuses_oversized_workspace(gpu_lib):
    """Sizes whose split workspace exceeds the static scratch are refused before any launch."""
    B, L, H, N, G = 5, 8192, 64, 128, 8
    need = gpu_lib.ssd_chunk_scan_workspace_size(B, L, H, 64, N, G, 1)
    assert need > gpu_lib.SSD_STATIC_SCRATCH_BYTES
    x = torch.zeros(B, L, H * 64, dtype=torch.bfloat16, device=DEV)
    bm = torch.zeros(B, L, G * N, dtype=torch.bfloat16, device=DEV)
    dt = torch.zeros(B, L, H, device=DEV)
    A = -torch.ones(H, device=DEV)
    with pytest.raises(gpu_lib.SSDError, match="static scratch"):
        gpu_lib.ssd_chunk_scan_fwd_static(x, bm, bm, dt, A, H=H, P=64, N=N, G=G)
