"""GPU parity of ssd_chunk_scan_fwd, ssd_chunk_scan_bwd, ssd_mixer_fwd, ssd_s6_scan_fwd and the two decode
calls (ssd_step against the oracle, ssd_resume_fwd bit for bit against the forward) over seeded random
configurations: state sizes,
group layouts (heads per group 1, 2, 3, 4, 6, 8, so every workgroup plan the library picks), lengths from one
token to several superchunks, documents, carried states, the gate, both dt forms, and the sequence split where
the sizes take it.  Inputs reach both sides identically, so the bars are the per-call ones: fp32 1e-3 * RMS,
bf16 0.03125 absolute, the backward 1e-3 * RMS per gradient; the split result is held to the same bars."""
import random

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import helpers as hp
from tests.test_gpu_bwd import DEV, _check, _np
from tests.test_gpu_conv_scan import run_scan, small_wl, workspace
from tests.test_gpu_mixer import check_oracle, inputs, mix_wl, run_mixer, run_two_call
from tests.test_gpu_resume import Resumer, forward as resume_forward, setup as resume_setup
from tests.test_gpu_s6 import _check as s6_check, _docs, _oracle as s6_oracle, _run as s6_run, _wl as s6_wl
from tests.test_gpu_step import decode_run, oracle_single_pass

pytestmark = pytest.mark.gpu


def _configs(n, seed=2024):
    r = random.Random(seed)
    out = []
    for i in range(n):
        dtype = r.choice(["bf16", "bf16", "f32"])
        N = r.choice([16, 32, 64, 128])
        G = r.choice([1, 2, 4])
        hpg = r.choice([1, 2, 3, 4, 6, 8])
        if G * hpg > 16:
            hpg = max(1, 16 // G)
        L = r.choice([1, 2, 63, 64, 65, r.randint(3, 600), r.randint(600, 2600)])
        B = r.choice([1, 2, 3])
        docs = r.random() < 0.5
        h0 = r.random() < 0.5
        gate = r.random() < 0.7
        softplus = r.random() < 0.7
        out.append((i, dtype, N, G, G * hpg, L, B, docs, h0, gate, softplus))
    return out


@pytest.mark.parametrize("i,dtype,N,G,H,L,B,docs,h0,gate,softplus", _configs(48))
def test_scan_random_config(gpu_lib, i, dtype, N, G, H, L, B, docs, h0, gate, softplus):
    print(f"random scan #{i}: {dtype} N={N} G={G} H={H} L={L} B={B} docs={docs} h0={h0} gate={gate} "
          f"softplus={softplus}", flush=True)
    wl = small_wl(dtype, H=H, N=N, G=G, L=L, B=B, docs=docs, h0=h0, gate=gate)
    prm = synth.params(wl, 100 + i)
    inp = synth.scan_inputs(wl, 100 + i)
    if not softplus:        # dt given directly (positive), as the conv prologue would deliver it
        inp["dt_raw"] = torch.nn.functional.softplus(inp["dt_raw"] + prm["dt_bias"])
    ids = synth.doc_ids(wl, 100 + i, mean_len=float(max(2, L // 3))) if docs else None
    check = hp.assert_fp32 if dtype == "f32" else hp.assert_bf16
    y, fs = run_scan(gpu_lib, wl, inp, prm, ids, dt_softplus=softplus)
    yr, fr = oracle.scan(inp["x"], inp["Bm"], inp["Cm"], inp["dt_raw"].float(), prm["A"], prm["D"], inp["z"], ids,
                          inp["h0"], H=wl.H, P=wl.P, N=wl.N, G=wl.G, dt_softplus=softplus,
                          dt_bias=prm["dt_bias"] if softplus else None, want_state=True)
    check(y, yr, "y")
    check(fs, fr, "final_state")
    if workspace(gpu_lib, wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, wl.dtype) is not None:
        ys, fss = run_scan(gpu_lib, wl, inp, prm, ids, dt_softplus=softplus, split=True)
        check(ys, yr, "y (sequence split)")
        check(fss, fr, "final_state (sequence split)")


@pytest.mark.parametrize("i,dtype,N,G,H,L,B,docs,h0,gate,softplus", _configs(16, seed=4048))
def test_scan_bwd_random_config(gpu_lib, i, dtype, N, G, H, L, B, docs, h0, gate, softplus):
    """The backward from a zero state (h0 unused) on the same kind of random configurations."""
    print(f"random scan bwd #{i}: {dtype} N={N} G={G} H={H} L={L} B={B} docs={docs} gate={gate} "
          f"softplus={softplus}", flush=True)
    wl = small_wl(dtype, H=H, N=N, G=G, L=L, B=B, docs=docs, gate=gate)
    prm = synth.params(wl, 200 + i)
    inp = synth.scan_inputs(wl, 200 + i)
    dt = inp["dt_raw"] if softplus else torch.nn.functional.softplus(inp["dt_raw"] + prm["dt_bias"])
    ids = synth.doc_ids(wl, 200 + i, mean_len=float(max(2, L // 3))) if docs else None
    gy = torch.randn(B, L, H * 64, generator=torch.Generator().manual_seed(300 + i))
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


def _mixer_configs(n, seed=7077):
    r = random.Random(seed)
    out = []
    for i in range(n):
        dtype = r.choice(["bf16", "bf16", "bf16", "f32"])
        N = r.choice([16, 32, 64, 128])
        G = r.choice([1, 2, 4])
        H = G * r.choice([1, 2, 3, 4])
        if dtype == "bf16" and H % 2:
            H *= 2                    # bf16 dt_raw rows are read in 4-byte words: an even row stride
        L = r.choice([1, 3, 64, 65, r.randint(4, 500), r.randint(500, 2400)])
        B = r.choice([1, 2])
        out.append((i, dtype, N, G, H, L, B, r.random() < 0.5, r.random() < 0.5, r.random() < 0.5,
                    r.random() < 0.8, r.choice([0, 0, 1]), r.random() < 0.5))
    return out


@pytest.mark.parametrize("i,dtype,N,G,H,L,B,docs,cs,h0,gate,act,bias", _mixer_configs(16))
def test_mixer_random_config(gpu_lib, i, dtype, N, G, H, L, B, docs, cs, h0, gate, act, bias):
    """ssd_mixer_fwd in both plans (fp32: the staged one) bit-identical to ssd_conv_fwd + ssd_chunk_scan_fwd,
    and call by call against the oracle (the conv within one bf16 ulp, the scan at the flat bar on the GPU
    conv's output, the outgoing conv state exactly)."""
    print(f"random mixer #{i}: {dtype} N={N} G={G} H={H} L={L} B={B} docs={docs} cs={cs} h0={h0} gate={gate} "
          f"act={act} bias={bias}", flush=True)
    wl = mix_wl(dtype, H, N, G, L, B=B, gate=gate)
    prm, raw, ids, cs_in = inputs(wl, 400 + i, docs, cs, h0, bias, mean_len=float(max(2, L // 3)))
    plans = ["staged"] if dtype == "f32" else ["fused", "staged"]
    for plan in plans:
        y, fs, co = run_mixer(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, plan=plan)
        y2, fs2, co2 = run_two_call(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, plan=plan)
        assert torch.equal(y, y2), hp.report(f"{plan}: mixer vs two-call y", y, y2)
        assert torch.equal(fs, fs2), hp.report(f"{plan}: mixer vs two-call final_state", fs, fs2)
        assert torch.equal(co, co2), f"{plan}: mixer vs two-call conv_state_out"
    check_oracle(gpu_lib, wl, raw, prm, ids, cs_in, raw["h0"], act, y, fs, co)


def _s6_configs(n, seed=9099):
    r = random.Random(seed)
    out = []
    for i in range(n):
        out.append((i, r.choice(["bf16", "f32"]), r.choice([1, 2, 3]),
                    r.choice([1, 2, 63, 64, 65, r.randint(3, 700), r.randint(700, 2100)]),
                    # channels: rows of 16-byte multiples (the call's stride rule), ragged workgroups included
                    r.choice([8, 64, 248, 256, 264, 8 * r.randint(2, 90)]), r.choice([8, 16, 32]),
                    r.random() < 0.5, r.random() < 0.5, r.random() < 0.7, r.random() < 0.7, r.random() < 0.5))
    return out


@pytest.mark.parametrize("i,dtype,B,L,Dn,N,docs,h0,gate,softplus,split", _s6_configs(20))
def test_s6_random_config(gpu_lib, i, dtype, B, L, Dn, N, docs, h0, gate, softplus, split):
    """ssd_s6_scan_fwd against the oracle's S6 routine: any channel count (ragged 256-channel workgroups),
    N = 8 / 16 / 32, documents, carried state, gate, both dt forms, with and without the sequence split."""
    print(f"random s6 #{i}: {dtype} B={B} L={L} D={Dn} N={N} docs={docs} h0={h0} gate={gate} softplus={softplus} "
          f"split={split}", flush=True)
    wl = s6_wl(dtype, B, L, Dn, N, h0=h0, gate=gate)
    prm = synth.s6_params(wl, 500 + i)
    inp = synth.s6_inputs(wl, 500 + i)
    if not softplus:
        inp["dt_raw"] = torch.nn.functional.softplus(inp["dt_raw"].float() - 2.5).to(inp["dt_raw"].dtype)
    ids = _docs(wl, 600 + i, L, float(max(2, L // 3))) if docs else None
    y, fs = s6_run(gpu_lib, inp, prm, softplus=softplus, gate=gate, docs=ids, h0=inp["h0"], split=split)
    yr, fr = s6_oracle(inp, prm, softplus=softplus, gate=gate, docs=ids, h0=inp["h0"])
    s6_check(dtype, y, yr, "y")
    s6_check(dtype, fs, fr, "final_state")


def _decode_configs(n, seed=1312):
    r = random.Random(seed)
    out = []
    for i in range(n):
        dtype = r.choice(["bf16", "f32"])
        N = r.choice([16, 32, 64, 128])
        G = r.choice([1, 2])
        H = G * r.choice([1, 2, 3, 4])
        if dtype == "bf16" and H % 2:
            H *= 2
        out.append((i, dtype, N, G, H, 64 * r.randint(1, 4), r.randint(20, 140), r.choice([1, 2, 3])))
    return out


@pytest.mark.parametrize("i,dtype,N,G,H,L0,steps,B", _decode_configs(12))
def test_resume_random_config(gpu_lib, i, dtype, N, G, H, L0, steps, B):
    """ssd_resume_fwd after a prefill of L0 tokens, appending random runs of tokens (crossing chunk ends): every
    output equals the one-call forward over the whole sequence bit for bit, and so does the state at every chunk
    end."""
    print(f"random resume #{i}: {dtype} N={N} G={G} H={H} prefill={L0} steps={steps} B={B}", flush=True)
    wl = synth.Workload("rresume_" + dtype, B, L0, H, 64, N, G, dtype)
    prm, raw, h0 = resume_setup(wl, 700 + i, L0 + steps, h0=i % 2 == 0)
    y_ref, _, _ = resume_forward(gpu_lib, wl, raw, prm, L0 + steps, h0=h0)
    _, fs, cs = resume_forward(gpu_lib, wl, raw, prm, L0, h0=h0)
    rs = Resumer(gpu_lib, wl, prm, B, fs, cs)
    r = random.Random(800 + i)
    ys, t = [], L0
    while t < L0 + steps:
        n = min(r.choice([1, 1, 1, 2, 5, 17]), 64 - rs.pos, L0 + steps - t)
        ys.append(rs.append(raw, t, n))
        t += n
        if rs.pos == 0:
            _, f_at, _ = resume_forward(gpu_lib, wl, raw, prm, t, h0=h0)
            assert torch.equal(rs.state, f_at), f"state after the chunk ending at token {t}"
    torch.cuda.synchronize()
    y = torch.cat(ys, 1)
    assert torch.equal(y, y_ref[:, L0:]), hp.report("resumed y vs one forward", y, y_ref[:, L0:])


def r_off(i):
    """A ragged prefill length for the step tests (the step itself needs no chunk alignment)."""
    return (37 * i) % 64


@pytest.mark.parametrize("i,dtype,N,G,H,L0,steps,B", _decode_configs(12, seed=2626))
def test_step_random_config(gpu_lib, i, dtype, N, G, H, L0, steps, B):
    """ssd_step after a GPU prefill, against the oracle's single pass over prefill and steps (fp32: 1e-3 * RMS;
    bf16: the conv -> scan pipeline bound), the conv state exactly."""
    print(f"random step #{i}: {dtype} N={N} G={G} H={H} prefill={L0} steps={steps} B={B}", flush=True)
    L = L0 + r_off(i)
    wl = synth.Workload("rstep_" + dtype, B, L, H, 64, N, G, dtype, steps=steps)
    prm = synth.params(wl, 900 + i, conv_bias=i % 2 == 1)
    raw = synth.raw_inputs(wl, 900 + i)
    y, ys, fs, cs = decode_run(gpu_lib, wl, prm, raw, steps, 900 + i, "cpu")
    yr, fr, cr, xr, _ = oracle_single_pass(wl, prm, raw, steps, 900 + i, list(range(B)), "cpu")
    yall = torch.cat([y.cpu()] + [s.cpu()[:, None] for s in ys], 1)
    if dtype == "f32":
        hp.assert_fp32(yall, yr, "prefill ++ decode y")
        hp.assert_fp32(fs, fr, "ssm state")
    else:
        z = torch.cat([raw["z"]] + [synth.step_inputs(wl, s, 900 + i)["z"][:, None] for s in range(steps)], 1)
        hp.assert_pipeline(yall, yr, xr[..., :H * 64], z, prm["D"], H, 64, "prefill ++ decode y")
        hp.assert_bf16(fs, fr, "ssm state")
    np.testing.assert_array_equal(hp.np64(cs), cr)
