"""GPU parity: the backward (VJP) calls against the fp64 oracle's backward.

Bars, per gradient tensor:
  * inputs the two sides read identically (fp32 inputs, or bf16 inputs fed to the scan or the conv directly):
    max |gpu - oracle| <= 1e-3 * RMS(oracle) -- fp32 arithmetic throughout on the GPU.
  * ssd_mixer_bwd with bf16 inputs, element-wise at the same bar against the oracle's backward fed the GPU's
    own conv output (the bf16 [x | B | C] rows and fp32 dt of ssd_conv_fwd, which ssd_mixer_bwd recomputes bit
    for bit): oracle.scan_bwd on those rows, then oracle.conv_bwd on its gradient.  Against the oracle's own
    end-to-end backward (oracle.mixer_bwd, which rounds its fp64 conv output to bf16) the relative L2 error
    is also held under 1e-3 per tensor: the two conv outputs can round to adjacent bf16 values (about 1 in
    10^4), and each such one-ulp (2^-8 relative) change of a scan input moves that token's gradients by up
    to the same relative amount -- sparse, so an L2 bar and not an element-wise one.
Document isolation is bitwise: a loss on a later document gives exactly 0.0 gradient on every earlier-document
input.  Two calls on the same inputs give identical bits.
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


def _np(t):
    return None if t is None else hp.np64(t)


def _check(got, ref, name, rel=hp.FP32_REL):
    got, ref = hp.np64(got), hp.np64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    bound = rel * hp.rms(ref)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= bound, hp.report(name, got, ref) + f" > {rel:g}*rms = {bound:.3e}"


def _scan_case(dtype, B, L, H, N, G, seed, docs, gate, softplus, mean_len=90.0):
    wl = synth.Workload(f"bwd_{dtype}_{B}_{L}_{H}_{N}_{G}", B, L, H, 64, N, G, dtype, gate=gate)
    inp = synth.scan_inputs(wl, seed)
    prm = synth.params(wl, seed)
    gen = torch.Generator().manual_seed(seed + 99)
    gy = torch.randn(B, L, H * 64, generator=gen)
    dt = inp["dt_raw"] if softplus else torch.nn.functional.softplus(inp["dt_raw"] + prm["dt_bias"])
    ids = synth.doc_ids(wl, seed, L=L, mean_len=mean_len) if docs else None
    return wl, inp, prm, gy, dt, ids


SCAN_CASES = [
    # dtype, B, L, H, N, G, docs, gate, softplus
    ("f32", 2, 200, 4, 64, 2, True, True, True),      # three chunks and an 8-token tail
    ("f32", 1, 64, 2, 16, 1, False, False, False),    # one full chunk
    ("f32", 2, 331, 4, 32, 4, True, True, False),
    ("bf16", 2, 257, 8, 64, 2, True, True, True),     # four heads per group
    ("bf16", 1, 130, 2, 16, 2, False, True, True),
    # N = 128: the state dimension in two blocks of 64 that take turns in LDS
    ("f32", 2, 200, 4, 128, 2, True, True, True),     # two heads per group
    ("bf16", 1, 270, 6, 128, 1, True, True, False),   # six heads: the resident block alternates
    ("f32", 1, 64, 1, 128, 1, False, False, True),    # one head, one chunk
]


@pytest.mark.parametrize("dtype,B,L,H,N,G,docs,gate,softplus", SCAN_CASES)
def test_scan_bwd_vs_oracle(gpu_lib, dtype, B, L, H, N, G, docs, gate, softplus):
    _say(f"scan bwd {dtype} B={B} L={L} H={H} N={N} G={G} docs={docs} gate={gate} softplus={softplus}")
    wl, inp, prm, gy, dt, ids = _scan_case(dtype, B, L, H, N, G, 3, docs, gate, softplus)
    g = lambda t: None if t is None else t.to(DEV)
    z = inp["z"] if gate else None
    got = gpu_lib.ssd_chunk_scan_bwd(g(inp["x"]), g(inp["Bm"]), g(inp["Cm"]), g(dt), g(prm["A"]), g(gy), H=H, P=64,
                                     N=N, G=G, D=g(prm["D"]), z=g(z), doc_ids=g(ids), dt_softplus=softplus,
                                     dt_bias=g(prm["dt_bias"]) if softplus else None)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(_np(inp["x"]), _np(inp["Bm"]), _np(inp["Cm"]), _np(dt), _np(prm["A"]), _np(gy),
                          _np(prm["D"]), _np(z), None if ids is None else ids.numpy(), H=H, P=64, N=N, G=G,
                          dt_softplus=softplus, dt_bias=_np(prm["dt_bias"]) if softplus else None)
    assert set(got) == set(ref), (sorted(got), sorted(ref))
    for k in ref:
        _check(got[k], ref[k], f"d{k}")


@pytest.mark.parametrize("dtype,act,docs", [("f32", 0, True), ("bf16", 0, True), ("f32", 1, False)])
def test_conv_bwd_vs_oracle(gpu_lib, dtype, act, docs):
    _say(f"conv bwd {dtype} act={act} docs={docs}")
    wl = synth.Workload(f"cbwd_{dtype}", 2, 300, 4, 64, 32, 2, dtype)
    prm = synth.params(wl, 4, conv_bias=True)
    raw = synth.raw_inputs(wl, 4)["xbc_raw"]
    ids = synth.doc_ids(wl, 4, mean_len=40.0) if docs else None
    gx = torch.randn(2, 300, wl.conv_dim, generator=torch.Generator().manual_seed(5))
    g = lambda t: None if t is None else t.to(DEV)
    got = gpu_lib.ssd_conv_bwd(g(raw), g(prm["conv_w"]), g(gx), H=wl.H, P=64, N=wl.N, G=wl.G, conv_b=g(prm["conv_b"]),
                               doc_ids=g(ids), act=act)
    torch.cuda.synchronize()
    ref = oracle.conv_bwd(_np(raw), _np(prm["conv_w"]), _np(gx), _np(prm["conv_b"]),
                          doc_ids=None if ids is None else ids.numpy(), act=act)
    for k in ("raw", "w", "bias"):
        _check(got[k], ref[k], f"d{k}")


def test_conv_bwd_document_starts_at_mask_edges(gpu_lib):
    """Document starts at the rows whose flags sit at bits 31, 32, 63 and 64 of the conv backward's per-tile
    start mask (local rows 28, 29, 60, 61), and at a tile's first row."""
    wl = synth.Workload("cbwd_edges", 1, 320, 4, 64, 32, 2, "f32")
    prm = synth.params(wl, 12, conv_bias=True)
    raw = synth.raw_inputs(wl, 12)["xbc_raw"]
    ids = torch.zeros(1, 320, dtype=torch.int32)
    for t in (28, 64 + 29, 128 + 60, 192 + 61, 256):
        ids[0, t:] += 1
    gx = torch.randn(1, 320, wl.conv_dim, generator=torch.Generator().manual_seed(13))
    g = lambda t: t.to(DEV)
    got = gpu_lib.ssd_conv_bwd(g(raw), g(prm["conv_w"]), g(gx), H=wl.H, P=64, N=wl.N, G=wl.G, conv_b=g(prm["conv_b"]),
                               doc_ids=g(ids))
    torch.cuda.synchronize()
    ref = oracle.conv_bwd(_np(raw), _np(prm["conv_w"]), _np(gx), _np(prm["conv_b"]), doc_ids=ids.numpy())
    for k in ("raw", "w", "bias"):
        _check(got[k], ref[k], f"d{k}")


def _mixer_inputs(wl, seed, docs, mean_len=1024.0, L=None):
    prm = synth.params(wl, seed, conv_bias=True)
    raw = synth.raw_inputs(wl, seed, L=L)
    Lr = raw["xbc_raw"].shape[1]
    ids = synth.doc_ids(wl, seed, L=Lr, mean_len=mean_len) if docs else None
    gy = torch.randn(wl.B, Lr, wl.H * wl.P, generator=torch.Generator().manual_seed(seed + 7))
    return prm, raw, ids, gy


def _mixer_gpu(lib, wl, prm, raw, ids, gy):
    g = lambda t: None if t is None else t.to(DEV)
    out = lib.ssd_mixer_bwd(g(raw["xbc_raw"]), g(raw["dt_raw"]), g(prm["conv_w"]), g(prm["A"]), g(gy), H=wl.H, P=wl.P,
                            N=wl.N, G=wl.G, conv_b=g(prm.get("conv_b")), dt_bias=g(prm["dt_bias"]), D=g(prm["D"]),
                            z=g(raw["z"]), doc_ids=g(ids))
    torch.cuda.synchronize()
    return out


def _mixer_oracle(wl, prm, raw, ids, gy, rows=None):
    sl = (lambda t: t) if rows is None else (lambda t: t[rows])
    return oracle.mixer_bwd(_np(sl(raw["xbc_raw"])), _np(prm["conv_w"]), _np(prm.get("conv_b")),
                            _np(sl(raw["dt_raw"])), _np(prm["dt_bias"]), _np(prm["A"]), _np(prm["D"]),
                            _np(sl(raw["z"])), _np(sl(gy)), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                            doc_ids=None if ids is None else sl(ids).numpy(), round_bf16=wl.dtype == "bf16")


def _mixer_oracle_on_gpu_conv(lib, wl, prm, raw, ids, gy, rows=None):
    """The oracle's mixer backward with its conv step replaced by the GPU's ssd_conv_fwd output: oracle.scan_bwd
    on the GPU's [x | B | C] rows and dt, then oracle.conv_bwd on the resulting conv-output gradient."""
    g = lambda t: None if t is None else t.to(DEV)
    xbc, dt = lib.ssd_conv_fwd(g(raw["xbc_raw"]), g(prm["conv_w"]), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                               conv_b=g(prm.get("conv_b")), dt_raw=g(raw["dt_raw"]), dt_bias=g(prm["dt_bias"]),
                               doc_ids=g(ids))
    torch.cuda.synchronize()
    sl = (lambda t: t) if rows is None else (lambda t: t[rows])
    HP, GN = wl.H * wl.P, wl.G * wl.N
    xg, dg = _np(sl(xbc.cpu())), _np(sl(dt.cpu()))
    idn = None if ids is None else sl(ids).numpy()
    gs = oracle.scan_bwd(xg[..., :HP], xg[..., HP:HP + GN], xg[..., HP + GN:], dg, _np(prm["A"]), _np(sl(gy)),
                         _np(prm["D"]), _np(sl(raw["z"])), idn, H=wl.H, P=wl.P, N=wl.N, G=wl.G)
    dxbc = np.concatenate([gs["x"], gs["Bm"], gs["Cm"]], axis=2)
    gc = oracle.conv_bwd(_np(sl(raw["xbc_raw"])), _np(prm["conv_w"]), dxbc, _np(prm.get("conv_b")),
                         _np(sl(raw["dt_raw"])), _np(prm["dt_bias"]), gs["dt"], idn)
    out = {"raw": gc["raw"], "w": gc["w"], "dt_raw": gc["dt_raw"], "A": gs["A"]}
    for k, src in (("bias", gc), ("dt_bias", gc), ("D", gs), ("z", gs)):
        if k in src:
            out[k] = src[k]
    return out


@pytest.mark.parametrize("dtype,N", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_mixer_bwd_vs_oracle(gpu_lib, dtype, N):
    wl = synth.Workload(f"mbwd_{dtype}_{N}", 2, 333, 8, 64, N, 2, dtype)
    _say(f"mixer bwd {dtype} N={N}")
    prm, raw, ids, gy = _mixer_inputs(wl, 6, True, mean_len=100.0)
    got = _mixer_gpu(gpu_lib, wl, prm, raw, ids, gy)
    ref = _mixer_oracle(wl, prm, raw, ids, gy)
    for k in ref:
        if dtype == "f32":
            _check(got[k], ref[k], f"d{k}")
        else:
            hp.assert_rel_l2(got[k], ref[k], f"d{k}")
    if dtype == "bf16":
        same = _mixer_oracle_on_gpu_conv(gpu_lib, wl, prm, raw, ids, gy)
        assert set(same) == set(ref)
        for k in same:
            _check(got[k], same[k], f"d{k} (oracle fed the GPU conv output)")


def test_bwd_document_isolation_and_determinism(gpu_lib):
    """A loss on the last document of a row gives exactly zero gradient on every earlier input of that row (and
    on the other row); two calls agree bit for bit."""
    wl = synth.Workload("iso_bwd", 2, 400, 4, 64, 32, 2, "bf16")
    _say("bwd isolation")
    prm, raw, ids, gy = _mixer_inputs(wl, 8, True, mean_len=70.0)
    for b in range(2):
        k = int(ids[b, -1])
        start = int(torch.nonzero(ids[b] == k)[0])
        assert start > 0
        gk = torch.zeros_like(gy)
        gk[b, start:] = gy[b, start:]
        out = _mixer_gpu(gpu_lib, wl, prm, raw, ids, gk)
        for name in ("raw", "dt_raw", "z"):
            t = out[name].cpu()
            assert torch.count_nonzero(t[b, :start]).item() == 0, f"d{name} before the document, row {b}"
            assert torch.count_nonzero(t[1 - b]).item() == 0, f"d{name} on the other row"
        again = _mixer_gpu(gpu_lib, wl, prm, raw, ids, gk)
        for name in out:
            assert torch.equal(out[name], again[name]), f"d{name} differs between two calls"


def test_mixer_bwd_equals_composition(gpu_lib):
    """ssd_mixer_bwd equals ssd_conv_fwd -> ssd_chunk_scan_bwd -> ssd_conv_bwd on the same inputs: bit for bit
    for every gradient the composition produces the same way, and within fp32 rounding for dt_raw (the chain
    through the softplus is applied in a different place)."""
    wl = synth.Workload("comp_bwd", 2, 260, 8, 64, 32, 2, "bf16")
    _say("bwd composition")
    prm, raw, ids, gy = _mixer_inputs(wl, 9, True, mean_len=80.0)
    g = lambda t: None if t is None else t.to(DEV)
    out = _mixer_gpu(gpu_lib, wl, prm, raw, ids, gy)
    HP, GN = wl.H * wl.P, wl.G * wl.N
    xbc, dt = gpu_lib.ssd_conv_fwd(g(raw["xbc_raw"]), g(prm["conv_w"]), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                                   conv_b=g(prm["conv_b"]), dt_raw=g(raw["dt_raw"]), dt_bias=g(prm["dt_bias"]),
                                   doc_ids=g(ids))
    sb = gpu_lib.ssd_chunk_scan_bwd(xbc[..., :HP], xbc[..., HP:HP + GN], xbc[..., HP + GN:], dt, g(prm["A"]), g(gy),
                                    H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=g(prm["D"]), z=g(raw["z"]), doc_ids=g(ids))
    dxbc = torch.cat([sb["x"], sb["Bm"], sb["Cm"]], dim=2).contiguous()
    cb = gpu_lib.ssd_conv_bwd(g(raw["xbc_raw"]), g(prm["conv_w"]), dxbc, H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                              conv_b=g(prm["conv_b"]), doc_ids=g(ids))
    torch.cuda.synchronize()
    for a, b in (("raw", cb["raw"]), ("w", cb["w"]), ("bias", cb["bias"]), ("A", sb["A"]), ("D", sb["D"]),
                 ("z", sb["z"])):
        assert torch.equal(out[a], b), hp.report(f"d{a} mixer vs composition", out[a], b)
    ddt_raw = sb["dt"] * (-torch.expm1(-dt))
    hp.assert_fp32(out["dt_raw"], ddt_raw, "ddt_raw mixer vs composition")


def test_bwd_empty_and_refusals(gpu_lib):
    wl = synth.Workload("bwd_ref", 1, 0, 2, 64, 16, 1, "f32")
    prm = {k: (None if v is None else v.to(DEV)) for k, v in synth.params(wl, 1).items()}
    e = lambda w: torch.empty(1, 0, w, device=DEV)
    got = gpu_lib.ssd_chunk_scan_bwd(e(128), e(16), e(16), e(2), prm["A"], e(128), H=2, P=64, N=16, G=1, D=prm["D"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(got["A"]).item() == 0 and torch.count_nonzero(got["D"]).item() == 0
    x = torch.zeros(1, 8, 128, device=DEV)
    b256 = torch.zeros(1, 8, 256, device=DEV)
    with pytest.raises(gpu_lib.SSDError, match="N=256"):
        gpu_lib.ssd_chunk_scan_bwd(x, b256, b256, torch.zeros(1, 8, 2, device=DEV), prm["A"], x, H=2, P=64, N=256,
                                   G=1)
    with pytest.raises(gpu_lib.SSDError, match="workspace_bytes"):
        gpu_lib.ssd_chunk_scan_bwd(x, x[..., :16].contiguous(), x[..., :16].contiguous(),
                                   torch.zeros(1, 8, 2, device=DEV), prm["A"], x, H=2, P=64, N=16, G=1,
                                   workspace=torch.empty(64, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["mini_k3_packed", "mini_k3_bf16"])
def test_mixer_bwd_full_workload(gpu_lib, name, dtype):
    """The Mini-K3 mixer shape (B=5, L=8192, H=32, N=64, G=8) end to end against the oracle's backward on all
    five rows, every gradient (parameter gradients included): element-wise with fp32 inputs; with bf16 inputs
    element-wise against the oracle fed the GPU's conv output, and relative L2 against the oracle's own
    end-to-end backward (see the module doc)."""
    wl = synth.WORKLOADS[name].with_(dtype=dtype)
    _say(f"mixer bwd full workload {name} {dtype}")
    prm, raw, ids, gy = _mixer_inputs(wl, 0, wl.docs)
    got = _mixer_gpu(gpu_lib, wl, prm, raw, ids, gy)
    ref = _mixer_oracle(wl, prm, raw, ids, gy)
    for k in ref:
        if dtype == "f32":
            _check(got[k], ref[k], f"d{k}")
        else:
            hp.assert_rel_l2(got[k], ref[k], f"d{k}")
    if dtype == "bf16":
        del ref
        same = _mixer_oracle_on_gpu_conv(gpu_lib, wl, prm, raw, ids, gy)
        for k in same:
            _check(got[k], same[k], f"d{k} (oracle fed the GPU conv output)")


def test_scan_bwd_full_workload_bf16(gpu_lib):
    """ssd_chunk_scan_bwd at the Mini-K3 shape with bf16 x, B, C read identically by both sides (packed
    documents, gate, softplus on dt): element-wise against the oracle on all five rows."""
    wl = synth.WORKLOADS["mini_k3_packed"]
    _say("scan bwd full workload bf16")
    inp = synth.scan_inputs(wl, 1)
    prm = synth.params(wl, 1)
    ids = synth.doc_ids(wl, 1)
    gy = torch.randn(wl.B, wl.L, wl.H * wl.P, generator=torch.Generator().manual_seed(11))
    g = lambda t: None if t is None else t.to(DEV)
    got = gpu_lib.ssd_chunk_scan_bwd(g(inp["x"]), g(inp["Bm"]), g(inp["Cm"]), g(inp["dt_raw"]), g(prm["A"]), g(gy),
                                     H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=g(prm["D"]), z=g(inp["z"]), doc_ids=g(ids),
                                     dt_softplus=True, dt_bias=g(prm["dt_bias"]))
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(_np(inp["x"]), _np(inp["Bm"]), _np(inp["Cm"]), _np(inp["dt_raw"]), _np(prm["A"]), _np(gy),
                          _np(prm["D"]), _np(inp["z"]), ids.numpy(), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                          dt_softplus=True, dt_bias=_np(prm["dt_bias"]))
    for k in ref:
        _check(got[k], ref[k], f"d{k}")


def test_scan_bwd_large_layer_f32(gpu_lib):
    """ssd_chunk_scan_bwd at the large-layer shape (B=4, L=4096, H=128, P=64, N=128, G=8) with fp32 inputs,
    documents, gate and softplus on dt: every per-token gradient of rows 0 and 3 of the full-batch call
    element-wise against the oracle on those rows, and the parameter gradients of a call on those two rows
    alone against the oracle's."""
    wl = synth.WORKLOADS["large_layer_bf16"].with_(dtype="f32")
    rows = [0, wl.B - 1]
    _say("scan bwd large layer f32")
    inp = synth.scan_inputs(wl, 2)
    prm = synth.params(wl, 2)
    ids = synth.doc_ids(wl, 2, mean_len=1024.0)
    gy = torch.randn(wl.B, wl.L, wl.H * wl.P, generator=torch.Generator().manual_seed(12))
    g = lambda t: None if t is None else t.to(DEV)

    def run(sl):
        out = gpu_lib.ssd_chunk_scan_bwd(g(sl(inp["x"])), g(sl(inp["Bm"])), g(sl(inp["Cm"])), g(sl(inp["dt_raw"])),
                                         g(prm["A"]), g(sl(gy)), H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=g(prm["D"]),
                                         z=g(sl(inp["z"])), doc_ids=g(sl(ids)), dt_softplus=True,
                                         dt_bias=g(prm["dt_bias"]))
        torch.cuda.synchronize()
        return {k: v.cpu() for k, v in out.items()}

    full = run(lambda t: t)
    part = run(lambda t: t[rows].contiguous())
    _say("scan bwd large layer f32: oracle rows")
    sl = lambda t: t[rows]
    ref = oracle.scan_bwd(_np(sl(inp["x"])), _np(sl(inp["Bm"])), _np(sl(inp["Cm"])), _np(sl(inp["dt_raw"])),
                          _np(prm["A"]), _np(sl(gy)), _np(prm["D"]), _np(sl(inp["z"])), sl(ids).numpy(), H=wl.H,
                          P=wl.P, N=wl.N, G=wl.G, dt_softplus=True, dt_bias=_np(prm["dt_bias"]))
    assert set(full) == set(ref), (sorted(full), sorted(ref))
    for k in ref:
        if full[k].dim() == 3:                     # per token: rows of the full-batch call
            _check(full[k][rows], ref[k], f"d{k} (rows {rows} of the full batch)")
            assert torch.equal(full[k][rows], part[k]), f"d{k}: the two-row call differs from the full batch"
        else:                                      # per head: summed over the two rows
            _check(part[k], ref[k], f"d{k} (rows {rows} alone)")
