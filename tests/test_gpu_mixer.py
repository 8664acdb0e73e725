"""GPU parity of ssd_mixer_fwd -- the conv prologue fused into the scan -- through the C ABI.

Two bars on seeded synthetic inputs:
  * bit identity with the two-call path ssd_conv_fwd -> ssd_chunk_scan_fwd (dt_softplus = 0 on the conv's
    dt) with the same workspace choice: the fused kernels convolve each chunk in LDS with the conv
    kernel's fp32 arithmetic, so y, the final state and the conv state must agree exactly;
  * the fp64 oracle, call by call on identical inputs: the conv (run alone on the GPU; the mixer equals the
    two-call path bit for bit) within one bf16 ulp of the oracle conv, and the scan within the flat 0.03125
    (bf16) or 1e-3 * RMS (fp32) of the oracle scan fed that conv's exact output; the outgoing conv state (raw
    rows) exactly.
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


def mix_wl(dtype, H, N, G, L, B=2, **kw):
    return synth.Workload("mix_" + dtype, B, L, H, 64, N, G, dtype, **kw)


def _g(t):
    return None if t is None else t.to(DEV)


def run_mixer(lib, wl, raw, prm, ids=None, cs_in=None, h0=None, act=0, split=False, plan="fused"):
    """ssd_mixer_fwd.  plan "staged": a workspace of ssd_mixer_workspace_size() bytes (the split is then
    always on when the sizes call for one); "fused" (bf16): no workspace, or the scan's split workspace."""
    B, L = raw["xbc_raw"].shape[:2]
    code = 1 if wl.dtype == "bf16" else 0
    cs_out = torch.full((B, 3, wl.conv_dim), 7.0, dtype=wl.torch_dtype, device=DEV)
    fs = torch.full((B, wl.H, wl.P, wl.N), 7.0, dtype=torch.float32, device=DEV)
    ws = None
    if plan == "staged" or wl.dtype == "f32":
        n = lib.ssd_mixer_workspace_size(B, L, wl.H, wl.P, wl.N, wl.G, code)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    elif split:
        n = lib.ssd_chunk_scan_workspace_size(B, L, wl.H, wl.P, wl.N, wl.G, code)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)
    y = lib.ssd_mixer_fwd(_g(raw["xbc_raw"]), _g(raw["dt_raw"]), _g(prm["conv_w"]), _g(prm["A"]), H=wl.H, P=wl.P,
                          N=wl.N, G=wl.G, conv_b=_g(prm.get("conv_b")), dt_bias=_g(prm["dt_bias"]), D=_g(prm["D"]),
                          z=_g(raw["z"]), doc_ids=_g(ids), conv_state_in=_g(cs_in), conv_state_out=cs_out,
                          init_state=_g(h0), final_state=fs, act=act, workspace=ws)
    torch.cuda.synchronize()
    return y, fs, cs_out


def run_two_call(lib, wl, raw, prm, ids=None, cs_in=None, h0=None, act=0, split=False, plan=None):
    split = split or plan == "staged"
    B, L = raw["xbc_raw"].shape[:2]
    HP, GN = wl.H * wl.P, wl.G * wl.N
    cs_out = torch.full((B, 3, wl.conv_dim), 7.0, dtype=wl.torch_dtype, device=DEV)
    xbc, dt = lib.ssd_conv_fwd(_g(raw["xbc_raw"]), _g(prm["conv_w"]), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                               conv_b=_g(prm.get("conv_b")), dt_raw=_g(raw["dt_raw"]), dt_bias=_g(prm["dt_bias"]),
                               doc_ids=_g(ids), conv_state_in=_g(cs_in), conv_state_out=cs_out, act=act)
    fs = torch.full((B, wl.H, wl.P, wl.N), 7.0, dtype=torch.float32, device=DEV)
    ws = None
    if split or wl.dtype == "f32":
        n = lib.ssd_chunk_scan_workspace_size(B, L, wl.H, wl.P, wl.N, wl.G, 1 if wl.dtype == "bf16" else 0)
        ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
    y = lib.ssd_chunk_scan_fwd(xbc[..., :HP], xbc[..., HP:HP + GN], xbc[..., HP + GN:], dt, _g(prm["A"]), H=wl.H,
                               P=wl.P, N=wl.N, G=wl.G, D=_g(prm["D"]), z=_g(raw["z"]), doc_ids=_g(ids),
                               init_state=_g(h0), final_state=fs, workspace=ws)
    torch.cuda.synchronize()
    return y, fs, cs_out


def gpu_conv(lib, wl, raw, prm, ids=None, cs_in=None, act=0):
    """ssd_conv_fwd alone: the [x | B | C] rows and dt that the mixer's scan reads (the mixer equals the
    two-call path bit for bit)."""
    xbc, dt = lib.ssd_conv_fwd(_g(raw["xbc_raw"]), _g(prm["conv_w"]), H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                               conv_b=_g(prm.get("conv_b")), dt_raw=_g(raw["dt_raw"]), dt_bias=_g(prm["dt_bias"]),
                               doc_ids=_g(ids), conv_state_in=_g(cs_in), act=act)
    torch.cuda.synchronize()
    return xbc, dt


def check_oracle(lib, wl, raw, prm, ids, cs_in, h0, act, y, fs, cs_out, rows=None):
    """Call by call against the oracle on identical inputs (module doc), on whole batch rows."""
    rows = range(raw["xbc_raw"].shape[0]) if rows is None else rows
    bf = wl.dtype == "bf16"
    HP, GN = wl.H * wl.P, wl.G * wl.N
    xbc, dt = gpu_conv(lib, wl, raw, prm, ids, cs_in, act)
    for b in rows:
        sl = slice(b, b + 1)
        cpu = lambda t: None if t is None else t[sl].cpu()
        ids_b = None if ids is None else ids[sl].cpu()
        ref, dref, cr = oracle.conv(cpu(raw["xbc_raw"]), prm["conv_w"], prm.get("conv_b"), cpu(raw["dt_raw"]),
                                    prm["dt_bias"], ids_b, cpu(cs_in), act=act, want_state=True)
        xg, dg = xbc[sl].cpu(), dt[sl].cpu()
        if bf:
            ab = lambda t: None if t is None else hp.np64(t).__abs__()
            mag, _, _ = oracle.conv(ab(cpu(raw["xbc_raw"])), ab(prm["conv_w"]), ab(prm.get("conv_b")), doc_ids=ids_b,
                                    state_in=ab(cpu(cs_in)), act=1)
            hp.assert_within_ulp(xg, ref, f"conv row {b}", mag)
        else:
            hp.assert_fp32(xg, ref, f"conv row {b}")
        hp.assert_fp32(dg, dref, f"dt row {b}")
        yr, fr = oracle.scan(xg[..., :HP], xg[..., HP:HP + GN], xg[..., HP + GN:], dg, prm["A"], prm["D"],
                             cpu(raw["z"]), ids_b, cpu(h0), H=wl.H, P=wl.P, N=wl.N, G=wl.G, dt_softplus=False,
                             want_state=True)
        check = hp.assert_bf16 if bf else hp.assert_fp32
        check(y[sl], yr, f"y row {b}")
        check(fs[sl], fr, f"final_state row {b}")
        np.testing.assert_array_equal(hp.np64(cs_out[sl]), cr, err_msg=f"conv_state_out row {b}")


def inputs(wl, seed, docs, cs, h0, bias, mean_len=40.0):
    prm = synth.params(wl, seed, conv_bias=bias)
    raw = synth.raw_inputs(wl, seed)
    if not h0:
        raw["h0"] = None
    elif raw["h0"] is None:
        raw["h0"] = torch.randn(wl.B, wl.H, wl.P, wl.N, generator=torch.Generator().manual_seed(seed)) * 0.3
    ids = synth.doc_ids(wl, seed, mean_len=mean_len) if docs else None
    cs_in = (torch.randn(wl.B, 3, wl.conv_dim, generator=torch.Generator().manual_seed(seed + 100))
             .to(wl.torch_dtype) if cs else None)
    return prm, raw, ids, cs_in


MIX_CASES = [
    # dtype, N, G, H, L, docs, conv state in, h0, gate, act, conv bias
    ("bf16", 64, 2, 8, 333, True, True, True, True, 0, True),       # four heads per workgroup
    ("bf16", 64, 8, 8, 200, False, False, False, True, 0, False),   # one head per workgroup
    ("bf16", 64, 2, 4, 130, True, True, True, False, 1, True),      # two heads per workgroup, no act
    ("bf16", 16, 1, 4, 190, True, True, True, True, 0, True),
    ("bf16", 32, 2, 8, 129, True, False, True, False, 0, True),
    ("bf16", 128, 1, 4, 100, True, True, True, True, 0, True),
    ("bf16", 128, 4, 8, 64, False, True, False, True, 0, False),
    ("bf16", 64, 1, 2, 1, True, True, True, True, 0, True),
    ("bf16", 64, 1, 4, 2, True, True, True, True, 0, True),
    ("bf16", 64, 1, 4, 3, True, True, True, True, 0, True),
    ("bf16", 32, 1, 4, 67, True, True, True, True, 0, True),
    ("f32", 32, 2, 4, 130, True, True, True, True, 0, True),
    ("f32", 64, 1, 2, 65, False, False, True, True, 1, False),
]


@pytest.mark.parametrize("plan", ["fused", "staged"])
@pytest.mark.parametrize("dtype,N,G,H,L,docs,cs,h0,gate,act,bias", MIX_CASES)
def test_mixer_small(gpu_lib, dtype, N, G, H, L, docs, cs, h0, gate, act, bias, plan):
    if dtype == "f32" and plan == "fused":
        pytest.skip("fp32 has only the staged plan")
    wl = mix_wl(dtype, H, N, G, L, gate=gate)
    _say(f"mixer small {plan} {dtype} N={N} G={G} H={H} L={L} docs={docs} cs={cs} h0={h0} gate={gate} act={act}")
    prm, raw, ids, cs_in = inputs(wl, 21, docs, cs, h0, bias, mean_len=20.0)
    y, fs, co = run_mixer(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, plan=plan)
    y2, fs2, co2 = run_two_call(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, plan=plan)
    assert torch.equal(y, y2), hp.report("mixer vs two-call y", y, y2)
    assert torch.equal(fs, fs2), hp.report("mixer vs two-call final_state", fs, fs2)
    assert torch.equal(co, co2), "mixer vs two-call conv_state_out"
    check_oracle(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, y, fs, co)


SPLIT_CASES = [
    # dtype, N, G, H, L, docs, conv state in, h0   (long enough for the sequence split)
    ("bf16", 64, 2, 4, 2000, True, True, True),
    ("bf16", 64, 1, 4, 3000, True, False, True),
    ("bf16", 128, 1, 4, 3000, True, True, True),
    ("bf16", 16, 2, 8, 1800, True, True, False),
    ("bf16", 32, 1, 4, 2500, False, True, True),
    ("f32", 64, 1, 2, 1100, True, True, True),
]


@pytest.mark.parametrize("dtype,N,G,H,L,docs,cs,h0", SPLIT_CASES)
def test_mixer_split(gpu_lib, dtype, N, G, H, L, docs, cs, h0):
    """The split path of the fused plan (fp32: the staged plan): the state-only pre-pass plus the main pass,
    both convolving on chip."""
    wl = mix_wl(dtype, H, N, G, L)
    _say(f"mixer split {dtype} N={N} G={G} H={H} L={L} docs={docs} cs={cs} h0={h0}")
    prm, raw, ids, cs_in = inputs(wl, 22, docs, cs, h0, True, mean_len=300.0)
    n = gpu_lib.ssd_chunk_scan_workspace_size(wl.B, L, H, 64, N, G, 1 if dtype == "bf16" else 0)
    assert n > 0
    y, fs, co = run_mixer(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], split=True)
    y2, fs2, co2 = run_two_call(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], split=True)
    assert torch.equal(y, y2), hp.report("mixer vs two-call y", y, y2)
    assert torch.equal(fs, fs2), hp.report("mixer vs two-call final_state", fs, fs2)
    assert torch.equal(co, co2), "mixer vs two-call conv_state_out"
    check_oracle(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], 0, y, fs, co)


def test_mixer_strided_views(gpu_lib):
    """xbc_raw, dt_raw and z as column slices of one wider in_proj-like row (row strides > widths)."""
    wl = mix_wl("bf16", 8, 64, 2, 300, docs=True)
    _say("mixer strided views")
    prm, raw, ids, cs_in = inputs(wl, 23, True, True, True, True)
    HP, C, H = wl.H * wl.P, wl.conv_dim, wl.H
    width = HP + C + H + 8          # [z | xbc | dt | pad], an even row stride
    row = torch.zeros(wl.B, wl.L, width, dtype=torch.bfloat16)
    row[..., :HP] = raw["z"]
    row[..., HP:HP + C] = raw["xbc_raw"]
    row[..., HP + C:HP + C + H] = raw["dt_raw"]
    row = row.to(DEV)
    view = {"z": row[..., :HP], "xbc_raw": row[..., HP:HP + C], "dt_raw": row[..., HP + C:HP + C + H],
            "h0": raw["h0"]}
    y, fs, co = run_mixer(gpu_lib, wl, view, prm, ids, cs_in, raw["h0"])
    y2, fs2, co2 = run_mixer(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"])
    assert torch.equal(y, y2) and torch.equal(fs, fs2) and torch.equal(co, co2)


def test_mixer_empty_sequence_passes_states_through(gpu_lib):
    wl = mix_wl("bf16", 4, 32, 1, 0)
    cs_in = torch.randn(wl.B, 3, wl.conv_dim, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(DEV)
    h0 = torch.randn(wl.B, wl.H, wl.P, wl.N, generator=torch.Generator().manual_seed(5)).to(DEV)
    co = torch.zeros_like(cs_in)
    fs = torch.zeros_like(h0)
    raw = torch.empty(wl.B, 0, wl.conv_dim, dtype=torch.bfloat16, device=DEV)
    dtr = torch.empty(wl.B, 0, wl.H, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(wl.conv_dim, 4, device=DEV)
    A = -torch.ones(wl.H, device=DEV)
    gpu_lib.ssd_mixer_fwd(raw, dtr, w, A, H=wl.H, P=wl.P, N=wl.N, G=wl.G, conv_state_in=cs_in, conv_state_out=co,
                          init_state=h0, final_state=fs)
    torch.cuda.synchronize()
    assert torch.equal(co, cs_in) and torch.equal(fs, h0)


@pytest.mark.parametrize("plan", ["fused", "staged"])
@pytest.mark.parametrize("name", ["mini_k3_packed", "large_layer_bf16"])
def test_mixer_full_workload(gpu_lib, name, plan):
    """The full-size workloads with the split: bit-identical to the two-call path on every output, and call by
    call within the flat bars of the oracle on the first and last batch rows."""
    wl = synth.WORKLOADS[name]
    _say(f"mixer full {name} {plan}")
    prm = synth.params(wl, 0)
    raw = synth.raw_inputs(wl, 0, device=DEV)
    ids = synth.doc_ids(wl, 0) if wl.docs else None
    y, fs, co = run_mixer(gpu_lib, wl, raw, prm, ids, None, raw["h0"], split=True, plan=plan)
    y2, fs2, co2 = run_two_call(gpu_lib, wl, raw, prm, ids, None, raw["h0"], split=True)
    assert torch.equal(y, y2), hp.report("mixer vs two-call y", y, y2)
    assert torch.equal(fs, fs2) and torch.equal(co, co2)
    del y2, fs2
    check_oracle(gpu_lib, wl, raw, prm, ids, None, raw["h0"], 0, y, fs, co, rows=(0, wl.B - 1))


@pytest.mark.parametrize("cut", [64, 1024, 1984])
def test_mixer_prefill_split_bitwise(gpu_lib, cut):
    """A prefill cut at a multiple of 64, both states carried, equals one sequential call bit for bit."""
    wl = synth.WORKLOADS["mini_k3_packed"].with_(L=2048, B=2)
    _say(f"mixer prefill cut at {cut}")
    prm = synth.params(wl, 7)
    raw = synth.raw_inputs(wl, 7, device=DEV)
    # documents start next to every cut but not on one (a call's t = 0 always continues the carried state)
    ids = torch.zeros(wl.B, wl.L, dtype=torch.int32)
    for cpos in (1, 62, 63, 65, 130, 1000, 1022, 1023, 1025, 1500, 1982, 1983, 1985, 2040):
        ids[0, cpos:] += 1
    for cpos in (3, 66, 1021, 1986):
        ids[1, cpos:] += 1
    ids = ids.to(DEV)
    y, fs, co = run_mixer(gpu_lib, wl, raw, prm, ids)
    a = {n: (None if v is None else v[:, :cut].contiguous()) for n, v in raw.items() if n != "h0"}
    c = {n: (None if v is None else v[:, cut:].contiguous()) for n, v in raw.items() if n != "h0"}
    a["h0"] = c["h0"] = None
    ya, fa, ca = run_mixer(gpu_lib, wl.with_(L=cut), a, prm, ids[:, :cut].contiguous())
    yc, fc, cc = run_mixer(gpu_lib, wl.with_(L=wl.L - cut), c, prm, ids[:, cut:].contiguous(), cs_in=ca, h0=fa)
    assert torch.equal(torch.cat([ya, yc], 1), y)
    assert torch.equal(fc, fs)
    assert torch.equal(cc, co)


@pytest.mark.parametrize("split", [False, True], ids=["single_pass", "seq_split"])
def test_mixer_doc_isolation_bitwise(gpu_lib, split):
    """Replacing every input of a row's earlier documents leaves every later output bit unchanged."""
    wl = synth.WORKLOADS["mini_k3_packed"].with_(L=2048, B=2)
    _say(f"mixer doc isolation split={split}")
    prm = synth.params(wl, 8)
    raw = synth.raw_inputs(wl, 8)
    ids = torch.zeros(wl.B, wl.L, dtype=torch.int32)
    splits = {0: [1, 2, 3, 64, 65, 700, 1023, 1024], 1: [62, 63, 127, 1500, 2047]}
    for b, cuts in splits.items():
        for cpos in cuts:
            ids[b, cpos:] += 1
    base, fbase, cbase = run_mixer(gpu_lib, wl, raw, prm, ids, split=split)
    gen = torch.Generator().manual_seed(12)
    for b, cuts in splits.items():
        for k in (cuts[0], cuts[len(cuts) // 2], cuts[-1]):
            pert = {n: (None if v is None else v.clone()) for n, v in raw.items()}
            pert["xbc_raw"][b, :k] = (torch.randn(k, wl.conv_dim, generator=gen) * 100.0).to(wl.torch_dtype)
            pert["dt_raw"][b, :k] = (torch.randn(k, wl.H, generator=gen) * 3.0).to(wl.torch_dtype)
            pert["z"][b, :k] = (torch.randn(k, wl.H * wl.P, generator=gen) * 100.0).to(wl.torch_dtype)
            y, fs, co = run_mixer(gpu_lib, wl, pert, prm, ids, split=split)
            assert torch.equal(base[b, k:], y[b, k:]), f"row {b}: outputs after boundary {k} changed"
            assert torch.equal(fbase[b], fs[b]), f"row {b}: final state changed (boundary {k})"
            assert torch.equal(cbase[b], co[b]), f"row {b}: conv state changed (boundary {k})"
            assert not torch.equal(base[b, :k], y[b, :k])
            other = 1 - b
            assert torch.equal(base[other], y[other])
