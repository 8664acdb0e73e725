#!/usr/bin/env python3
"""Benchmark of the SSD mixer core on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
ssd_conv_fwd (causal conv + SiLU + dt softplus) then ssd_chunk_scan_fwd
(chunked scan, groups, D skip, z gate, final state), at the Mini-K3 mixer
shape B=5, L=8192, H=32, P=64, N=64, G=8, bf16 inputs, fp32 state and y.
Inputs are resident in HBM before the timed region; two input sets alternate
so no step runs out of the 256 MB last-level cache.  From a cold start the
first ~40 steps run up to 10% slower than the steady state while the GPU ramps
up from idle, so the headline step runs ~30 ms untimed (settle) before its W
warm-up steps; every other timed loop follows it on a GPU already busy.

Prints ONE JSON line: value = head-tokens (B*L*H) per second over the whole
step; "roofline" = the scan call's algorithmic bytes / its average duration
against 8 TB/s, the duration measured over back-to-back launches of that call
alone, bracketed by one pair of HIP events on the launch stream;
"cpu_baseline" = the fp64 oracle (conv + scan) timed on this host.  Under
"extra": ssd_mixer_fwd on the same workload in both plans (staged: the same
two kernels behind one call; fused: the conv computed inside the scan
kernels), the other workloads (packed documents, the large layer, the decode
step), the chunk-resume decode (ssd_resume_fwd) and the fp32 4096-token
prefill (conv + scan) on the decode workload, the
Mamba-1 selective scan (ssd_s6_scan_fwd) priced against the VALU rate, and
the backward of the mixer (ssd_mixer_bwd) on the Mini-K3 batch and on the
large layer.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD scan tokens/sec (B×L×H/s) and % HBM roofline at 1 MI355X"
HBM_PEAK_GBS = 8000.0
# measured HBM traffic of the scan call (rocprofv3 FETCH_SIZE / WRITE_SIZE passes)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_mini_k3_bf16_traffic.txt")
SCAN_SOURCES = ("selective_state_space_14_amd/csrc/scan.hip", "selective_state_space_14_amd/csrc/ssd_device.hpp",
                "selective_state_space_14_amd/csrc/ssd_launch.hpp")


def scan_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per scan call from the committed counter summary, or None once the kernel sources changed."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != scan_source_hash():
            return None
        return float(kv["traffic_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def scan_bytes(wl, docs=False, h0=False):
    """Algorithmic bytes of one ssd_chunk_scan_fwd: every input read once, every output written once."""
    es = 2 if wl.dtype == "bf16" else 4
    tok = wl.B * wl.L
    b = tok * wl.H * wl.P * es            # x
    b += 2 * tok * wl.G * wl.N * es       # B, C
    b += tok * wl.H * 4                   # dt (fp32)
    b += tok * wl.H * wl.P * es if wl.gate else 0   # z
    b += tok * wl.H * wl.P * 4            # y (fp32)
    st = wl.B * wl.H * wl.P * wl.N * 4
    b += st                               # final state
    b += st if h0 else 0                  # initial state
    b += tok * 4 if docs else 0           # doc ids
    return b


def conv_bytes(wl, docs=False):
    """Algorithmic bytes of one ssd_conv_fwd: raw in, conv out, dt_raw in, dt out (fp32)."""
    es = 2 if wl.dtype == "bf16" else 4
    tok = wl.B * wl.L
    b = 2 * tok * wl.conv_dim * es + tok * wl.H * es + tok * wl.H * 4
    b += tok * 4 if docs else 0
    return b


def mixer_bytes(wl, docs=False, h0=False):
    """Algorithmic bytes of one ssd_mixer_fwd: the raw [x | B | C] columns, dt_raw and z read once, y and
    the final state written once (the conv output and dt never reach memory)."""
    es = 2 if wl.dtype == "bf16" else 4
    tok = wl.B * wl.L
    b = tok * wl.conv_dim * es            # raw x | B | C
    b += tok * wl.H * es                  # dt_raw
    b += tok * wl.H * wl.P * es if wl.gate else 0   # z
    b += tok * wl.H * wl.P * 4            # y (fp32)
    st = wl.B * wl.H * wl.P * wl.N * 4
    b += st                               # final state
    b += st if h0 else 0                  # initial state
    b += tok * 4 if docs else 0           # doc ids
    b += wl.B * 3 * wl.conv_dim * es      # conv state out
    return b


def step_bytes(wl):
    """Algorithmic bytes of one ssd_step: state and conv buffer read + written, row inputs, y."""
    es = 2 if wl.dtype == "bf16" else 4
    b = 2 * wl.B * wl.H * wl.P * wl.N * 4
    b += 2 * wl.B * 3 * wl.conv_dim * es
    b += wl.B * wl.conv_dim * es + wl.B * wl.H * es + (wl.B * wl.H * wl.P * es if wl.gate else 0)
    b += wl.B * wl.H * wl.P * 4
    return b


def resume_bytes(wl):
    """Bytes one ssd_resume_fwd call at working-chunk position pos must move, averaged over pos = 0 .. 63: the new
    token's conv (raw row, conv state read and written, its chunk row), the rescan of rows 0 .. pos (convolved row,
    dt and gate row read, chunk_y row written), the state at the chunk's start (read every call, written on the
    chunk's last token) and the new token's y copied out."""
    es = 2 if wl.dtype == "bf16" else 4
    C, HP, B = wl.conv_dim, wl.H * wl.P, wl.B
    conv = B * (C * es + 2 * 3 * C * es + C * es + wl.H * (es + 4))
    rows = 32.5                                   # mean of pos + 1 over a chunk
    scan = B * rows * (C * es + wl.H * 4 + (HP * es if wl.gate else 0) + HP * 4)
    state = B * wl.H * wl.P * wl.N * 4 * (1 + 1 / 64)
    return conv + scan + state + 2 * B * HP * 4


def loop_ms(torch, calls, n):
    """Mean duration in ms of one call when `n` calls run back to back on the launch stream (cycling through
    `calls`, e.g. one per input set), bracketed by ONE pair of HIP events: no event or host work sits between
    the kernels, so the figure is the calls' own device time plus the launch gaps between them."""
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(n):
        calls[i % len(calls)]()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def mixer_bench(ssd, synth, torch, wl, steps, warmup, docs=False, h0=False, seed=0, plan="staged"):
    """ssd_mixer_fwd as the step: plan "staged" (a workspace of ssd_mixer_workspace_size() bytes) or "fused"
    (the scan's split workspace only)."""
    dev = "cuda"
    HP = wl.H * wl.P
    prm = synth.params(wl, seed, device=dev)
    sets = []
    for k in range(2):
        raw = synth.raw_inputs(wl, seed + k, device=dev)
        ids = synth.doc_ids(wl, seed + k).to(dev) if docs else None
        sets.append((raw, ids))
    code = ssd.SSD_BF16 if wl.dtype == "bf16" else ssd.SSD_F32
    size = ssd.ssd_mixer_workspace_size if plan == "staged" else ssd.ssd_chunk_scan_workspace_size
    ws_bytes = size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, code)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty(wl.B, wl.L, HP, dtype=torch.float32, device=dev)
    fs = torch.empty(wl.B, wl.H, wl.P, wl.N, dtype=torch.float32, device=dev)
    cs = torch.empty(wl.B, 3, wl.conv_dim, dtype=wl.torch_dtype, device=dev)
    calls = []
    for k in range(2):
        raw, ids = sets[k]
        calls.append(lambda raw=raw, ids=ids: ssd.ssd_mixer_fwd(
            raw["xbc_raw"], raw["dt_raw"], prm["conv_w"], prm["A"], H=wl.H, P=wl.P, N=wl.N, G=wl.G,
            dt_bias=prm["dt_bias"], D=prm["D"], z=raw["z"], doc_ids=ids, conv_state_out=cs,
            init_state=raw["h0"] if h0 else None, final_state=fs, y=y, workspace=ws))
    for i in range(warmup):
        calls[i % 2]()
    ms = loop_ms(torch, calls, steps)
    mb = mixer_bytes(wl, docs, h0)
    return {"ms_per_step": ms, "value": wl.B * wl.L * wl.H / (ms * 1e-3), "mixer_us": ms * 1e3,
            "mixer_bytes": mb, "mixer_GBs": mb / (ms * 1e-3) / 1e9, "mixer_workspace_bytes": ws_bytes}


def settle(torch, fns, ms=30.0):
    """Run fns round-robin, untimed, for about `ms` of wall time (at least 4 calls), so that the timed loop that
    follows does not start on a GPU still ramping up from idle."""
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while i < 4 or (time.perf_counter() - t0) * 1e3 < ms:
        fns[i % len(fns)]()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def prefill_bench(ssd, synth, torch, wl, steps, warmup, docs=False, h0=False, seed=0):
    """The two-call path: ssd_conv_fwd then ssd_chunk_scan_fwd."""
    dev = "cuda"
    HP, GN = wl.H * wl.P, wl.G * wl.N
    prm = synth.params(wl, seed, device=dev)
    sets = []
    for k in range(2):
        raw = synth.raw_inputs(wl, seed + k, device=dev)
        ids = synth.doc_ids(wl, seed + k).to(dev) if docs else None
        sets.append((raw, ids))
    ws_bytes = ssd.ssd_chunk_scan_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G,
                                                 ssd.SSD_BF16 if wl.dtype == "bf16" else ssd.SSD_F32)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty(wl.B, wl.L, HP, dtype=torch.float32, device=dev)
    fs = torch.empty(wl.B, wl.H, wl.P, wl.N, dtype=torch.float32, device=dev)
    convs, scans = [], []
    for k in range(2):   # each input set has its own conv output, so the scan-only loop reads real data
        raw, ids = sets[k]
        xbc = torch.empty(wl.B, wl.L, wl.conv_dim, dtype=wl.torch_dtype, device=dev)
        dt = torch.empty(wl.B, wl.L, wl.H, dtype=torch.float32, device=dev)
        convs.append(lambda raw=raw, ids=ids, xbc=xbc, dt=dt: ssd.ssd_conv_fwd(
            raw["xbc_raw"], prm["conv_w"], H=wl.H, P=wl.P, N=wl.N, G=wl.G, dt_raw=raw["dt_raw"],
            dt_bias=prm["dt_bias"], doc_ids=ids, xbc_out=xbc, dt_out=dt))
        scans.append(lambda raw=raw, ids=ids, xbc=xbc, dt=dt: ssd.ssd_chunk_scan_fwd(
            xbc[..., :HP], xbc[..., HP:HP + GN], xbc[..., HP + GN:], dt, prm["A"], H=wl.H, P=wl.P, N=wl.N, G=wl.G,
            D=prm["D"], z=raw["z"], doc_ids=ids, init_state=raw["h0"] if h0 else None, final_state=fs, y=y,
            workspace=ws))
    steps_fn = [lambda k=k: (convs[k](), scans[k]()) for k in range(2)]
    settle(torch, steps_fn)
    for i in range(warmup):
        steps_fn[i % 2]()
    # the step (conv then scan, back to back), then each call alone over as many launches
    ms = loop_ms(torch, steps_fn, steps)
    conv_ms = loop_ms(torch, convs, steps)
    scan_ms = loop_ms(torch, scans, steps)
    sb, cb = scan_bytes(wl, docs, h0), conv_bytes(wl, docs)
    return {
        "ms_per_step": ms,
        "value": wl.B * wl.L * wl.H / (ms * 1e-3),
        "scan_us": scan_ms * 1e3, "conv_us": conv_ms * 1e3,
        "scan_bytes": sb, "conv_bytes": cb,
        "scan_GBs": sb / (scan_ms * 1e-3) / 1e9, "conv_GBs": cb / (conv_ms * 1e-3) / 1e9,
        "scan_head_tokens_per_s": wl.B * wl.L * wl.H / (scan_ms * 1e-3),
        "scan_workspace_bytes": ws_bytes,
    }


def decode_bench(ssd, synth, torch, wl, steps, warmup, seed=0):
    dev = "cuda"
    prm = synth.params(wl, seed, device=dev)
    g = torch.Generator(device=dev).manual_seed(seed)
    ssm = torch.randn(wl.B, wl.H, wl.P, wl.N, generator=g, device=dev) * 0.1
    conv = torch.randn(wl.B, 3, wl.conv_dim, generator=g, device=dev).to(wl.torch_dtype)
    ins = [synth.step_inputs(wl, s, seed, device=dev) for s in range(2)]
    y = torch.empty(wl.B, wl.H * wl.P, dtype=torch.float32, device=dev)
    calls = [lambda st=st: ssd.ssd_step(st["xbc_raw"], st["dt_raw"], prm["conv_w"], prm["A"], conv, ssm, H=wl.H,
                                        P=wl.P, N=wl.N, G=wl.G, z=st["z"], dt_bias=prm["dt_bias"], D=prm["D"], y=y)
             for st in ins]
    for i in range(warmup):
        calls[i % 2]()
    ms = loop_ms(torch, calls, steps)
    kb = step_bytes(wl)
    return {"ms_per_step": ms, "value": wl.B * wl.H / (ms * 1e-3), "step_us": ms * 1e3, "step_bytes": kb,
            "step_GBs": kb / (ms * 1e-3) / 1e9}


def f32_prefill_bench(ssd, synth, torch, wl, steps, warmup, seed=0):
    """The fp32 prefill of the decode workload (conv then scan with its split workspace, one input set: 36 GB of
    inputs, far beyond any cache), each call timed alone over back-to-back launches."""
    dev = "cuda"
    HP, GN = wl.H * wl.P, wl.G * wl.N
    prm = synth.params(wl, seed, device=dev)
    raw = synth.raw_inputs(wl, seed, device=dev)
    ws_bytes = ssd.ssd_chunk_scan_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, ssd.SSD_F32)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    xbc = torch.empty(wl.B, wl.L, wl.conv_dim, dtype=torch.float32, device=dev)
    dt = torch.empty(wl.B, wl.L, wl.H, dtype=torch.float32, device=dev)
    y = torch.empty(wl.B, wl.L, HP, dtype=torch.float32, device=dev)
    fs = torch.empty(wl.B, wl.H, wl.P, wl.N, dtype=torch.float32, device=dev)
    conv = lambda: ssd.ssd_conv_fwd(raw["xbc_raw"], prm["conv_w"], H=wl.H, P=wl.P, N=wl.N, G=wl.G,
                                    dt_raw=raw["dt_raw"], dt_bias=prm["dt_bias"], xbc_out=xbc, dt_out=dt)
    scan = lambda: ssd.ssd_chunk_scan_fwd(xbc[..., :HP], xbc[..., HP:HP + GN], xbc[..., HP + GN:], dt, prm["A"],
                                          H=wl.H, P=wl.P, N=wl.N, G=wl.G, D=prm["D"], z=raw["z"], final_state=fs,
                                          y=y, workspace=ws)
    for _ in range(warmup):
        conv()
        scan()
    conv_ms, scan_ms = loop_ms(torch, [conv], steps), loop_ms(torch, [scan], steps)
    sb = scan_bytes(wl)
    del raw, xbc, y
    return {"workload": wl.name + " prefill (fp32 ssd_conv_fwd + ssd_chunk_scan_fwd, B=%d L=%d H=%d N=%d)"
            % (wl.B, wl.L, wl.H, wl.N), "ms_per_step": conv_ms + scan_ms, "conv_ms": conv_ms, "scan_ms": scan_ms,
            "scan_bytes": sb, "scan_GBs": sb / (scan_ms * 1e-3) / 1e9,
            "scan_frac": sb / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "value": wl.B * wl.L * wl.H / (scan_ms * 1e-3), "unit": "head-tokens/s (scan)"}


def resume_bench(ssd, synth, torch, wl, warmup, seed=0):
    """ssd_resume_fwd one token at a time over one full working chunk (64 steps, pos 0..63): the decode that
    continues the forward bit for bit.  Returns the mean per step."""
    dev = "cuda"
    prm = synth.params(wl, seed, device=dev)
    g = torch.Generator(device=dev).manual_seed(seed)
    B, C, HP = wl.B, wl.conv_dim, wl.H * wl.P
    state = torch.randn(B, wl.H, wl.P, wl.N, generator=g, device=dev) * 0.1
    conv = torch.randn(B, 3, C, generator=g, device=dev).to(wl.torch_dtype)
    cx = torch.zeros(B, 64, C, dtype=wl.torch_dtype, device=dev)
    cdt = torch.zeros(B, 64, wl.H, dtype=torch.float32, device=dev)
    cz = torch.zeros(B, 64, HP, dtype=wl.torch_dtype, device=dev)
    cy = torch.empty(B, 64, HP, dtype=torch.float32, device=dev)
    y = torch.empty(B, 1, HP, dtype=torch.float32, device=dev)
    ins = [synth.step_inputs(wl, s, seed, device=dev) for s in range(2)]
    ins = [{k: v[:, None].contiguous() for k, v in st.items()} for st in ins]

    def one(pos):
        st = ins[pos % 2]
        ssd.ssd_resume_fwd(st["xbc_raw"], st["dt_raw"], prm["conv_w"], prm["A"], conv, cx, cdt, state, cy, pos=pos,
                           H=wl.H, P=wl.P, N=wl.N, G=wl.G, z=st["z"], chunk_z=cz, dt_bias=prm["dt_bias"], D=prm["D"],
                           y=y)

    for i in range(warmup):
        one(i % 64)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for pos in range(64):
        one(pos)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / 64
    nb = resume_bytes(wl)
    return {"workload": wl.name + " (ssd_resume_fwd, one token per call, mean over a 64-token chunk)",
            "ms_per_step": ms, "value": wl.B * wl.H / (ms * 1e-3), "unit": "head-tokens/s (B*H per step)",
            "hbm_bytes": nb, "hbm_GBs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


# fp32 VALU lane-operations per second this build can issue on MI355X: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz = 39.3e12, i.e. one wave64 instruction per SIMD every 4 cycles.  The 157.3 TFLOP/s headline counts an
# fma as two flops AND assumes packed fp32 (two lanes per instruction slot), which the build turns off; the SQ
# counters of the scan kernels show 4.3 cycles per VALU instruction.  One S6 state update costs 8 issue slots:
# exp2 (a transcendental, quarter rate: 4 slots), dt*A, dt*x*B, the fma into h and the fma into y (4 slots).
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
S6_SLOTS_PER_UPDATE = 8


def s6_bytes(wl, h0=False, docs=False):
    """Algorithmic bytes of one ssd_s6_scan_fwd: x, dt, z (T) and B, C rows read once, y (fp32) and the final
    state written once."""
    es = 2 if wl.dtype == "bf16" else 4
    tok, Dn = wl.B * wl.L, wl.H * wl.P
    b = tok * Dn * (2 + (1 if wl.gate else 0)) * es + 2 * tok * wl.N * es + tok * Dn * 4
    st = wl.B * Dn * wl.N * 4
    return b + st + (st if h0 else 0) + (tok * 4 if docs else 0)


def s6_bench(ssd, synth, torch, wl, steps, warmup, seed=0):
    """ssd_s6_scan_fwd (the Mamba-1 selective scan) with its split workspace; the value is channel-tokens
    (B*L*D) per second, and the kernel is priced against the VALU issue rate (bound "alu")."""
    dev = "cuda"
    Dn = wl.H * wl.P
    prm = synth.s6_params(wl, seed, device=dev)
    sets = [synth.s6_inputs(wl, seed + k, device=dev) for k in range(2)]
    ws_bytes = ssd.ssd_s6_workspace_size(wl.B, wl.L, Dn, wl.N, ssd.SSD_BF16 if wl.dtype == "bf16" else ssd.SSD_F32)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    y = torch.empty(wl.B, wl.L, Dn, dtype=torch.float32, device=dev)
    fs = torch.empty(wl.B, Dn, wl.N, dtype=torch.float32, device=dev)
    calls = [lambda a=a: ssd.ssd_s6_scan_fwd(a["x"], a["dt_raw"], prm["A"], a["Bm"], a["Cm"], D_skip=prm["D_skip"],
                                             z=a["z"], final_state=fs, y=y, dt_softplus=True,
                                             dt_bias=prm["dt_bias"], workspace=ws)
             for a in sets]
    for i in range(warmup):
        calls[i % 2]()
    ms = loop_ms(torch, calls, steps)
    upd = wl.B * wl.L * Dn * wl.N
    peak = VALU_LANE_OPS / S6_SLOTS_PER_UPDATE
    nb = s6_bytes(wl)
    return {"workload": wl.name + " (ssd_s6_scan_fwd: B=%d L=%d D=%d N=%d)" % (wl.B, wl.L, Dn, wl.N),
            "ms_per_step": ms, "value": wl.B * wl.L * Dn / (ms * 1e-3), "unit": "channel-tokens/s (B*L*D)",
            "roofline": {"bound": "alu", "achieved": upd / (ms * 1e-3) / 1e12, "peak": peak / 1e12,
                         "unit": "T state-updates/s", "frac": upd / (ms * 1e-3) / peak},
            "hbm_GBs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nb, "workspace_bytes": ws_bytes}


def bwd_flops(wl):
    """Algorithmic fp32 flops of one ssd_mixer_bwd's scan passes: per (batch row, head, 64-token chunk) the chunk
    kernel's products (M X, C Hin, dyr X^T, M^T dyr, B Gout: 64x64x64 or 64xNx64 each, and the four 64x64xN
    products of dB and dC) and the first pass's two 64xNx64 products, plus C B^T once per group."""
    nc = (wl.L + 63) // 64
    Q, P, N = 64, wl.P, wl.N
    per_bhc = 3 * Q * Q * P + 2 * Q * N * P + 4 * Q * Q * N + 2 * Q * N * P
    per_bgc = Q * Q * N
    return 2.0 * (wl.B * wl.H * nc * per_bhc + wl.B * wl.G * nc * per_bgc)


def bwd_bench(ssd, synth, torch, wl, steps, warmup, seed=0):
    """ssd_mixer_bwd (conv recompute, the scan's backward passes, the conv's backward) on one batch."""
    dev = "cuda"
    prm = synth.params(wl, seed, device=dev)
    raw = synth.raw_inputs(wl, seed, device=dev)
    g = torch.Generator(device=dev).manual_seed(seed + 7)
    gy = torch.randn(wl.B, wl.L, wl.H * wl.P, generator=g, device=dev)
    code = ssd.SSD_BF16 if wl.dtype == "bf16" else ssd.SSD_F32
    ws = torch.empty(ssd.ssd_mixer_bwd_workspace_size(wl.B, wl.L, wl.H, wl.P, wl.N, wl.G, code), dtype=torch.uint8,
                     device=dev)
    call = lambda: ssd.ssd_mixer_bwd(raw["xbc_raw"], raw["dt_raw"], prm["conv_w"], prm["A"], gy, H=wl.H, P=wl.P,
                                     N=wl.N, G=wl.G, dt_bias=prm["dt_bias"], D=prm["D"], z=raw["z"], workspace=ws)
    for _ in range(warmup):
        call()
    ms = loop_ms(torch, [call], steps)
    fl = bwd_flops(wl)
    return {"workload": wl.name + " (ssd_mixer_bwd: conv recompute + scan backward + conv backward)",
            "ms_per_step": ms, "value": wl.B * wl.L * wl.H / (ms * 1e-3), "unit": "head-tokens/s",
            "scan_bwd_TFLOPs_over_call": fl / (ms * 1e-3) / 1e12, "algorithmic_flops": fl,
            "workspace_bytes": ws.numel()}


def oracle_seconds(synth, wl, rows):
    """Seconds the fp64 oracle (conv + scan, as it stands) takes on `rows` batch rows of the workload, with the
    OpenMP threads of this process."""
    import oracle
    prm = synth.params(wl, 0)
    raw = synth.raw_inputs(wl, 0, B=rows)
    oracle.build()
    t0 = time.perf_counter()
    oracle.forward(raw["xbc_raw"], prm["conv_w"], None, raw["dt_raw"], prm["dt_bias"], prm["A"], prm["D"], raw["z"],
                   H=wl.H, P=wl.P, N=wl.N, G=wl.G, round_bf16=True)
    return time.perf_counter() - t0


def cpu_baseline(synth, wl, rows, rows_1t=1):
    """The fp64 oracle on `rows` batch rows with every OpenMP thread of the host (OMP_NUM_THREADS or the CPU
    count), and on `rows_1t` rows with one thread (a child process started with OMP_NUM_THREADS=1)."""
    import subprocess
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    sec = oracle_seconds(synth, wl, rows)
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    out = {"value": rows * wl.L * wl.H / sec, "unit": "head-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows} of {wl.B} batch rows of the {wl.name} workload (L={wl.L}, all {wl.H} heads), "
                     f"conv + scan in fp64, {sec:.2f} s on {threads} threads of {model}"}
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-seconds", str(rows_1t)], env=env,
                       capture_output=True, text=True)
    if r.returncode == 0 and r.stdout.strip():
        sec1 = float(r.stdout.strip().split()[-1])
        out["single_thread"] = {"value": rows_1t * wl.L * wl.H / sec1, "unit": "head-tokens/s", "cores": 1,
                                "sample": f"{rows_1t} of {wl.B} batch rows, {sec1:.2f} s on 1 thread"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=5)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (hardware-counter calibration)")
    ap.add_argument("--oracle-seconds", type=int, default=0, help=argparse.SUPPRESS)   # the single-thread child
    args = ap.parse_args()
    if args.oracle_seconds:
        import synth
        print(oracle_seconds(synth, synth.WORKLOADS["mini_k3_bf16"], args.oracle_seconds))
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this build runs on one GPU only (the scan shards by batch row and "
              "head with no exchange; multi-GPU runs are not part of it)", file=sys.stderr)
        sys.exit(2)

    import torch

    import selective_state_space_14_amd as ssd
    import synth

    ssd.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    wl = synth.WORKLOADS["mini_k3_bf16"]
    main_r = prefill_bench(ssd, synth, torch, wl, args.steps, args.warmup)

    def mixer_extra(w, r, plan):
        return {"workload": w.name, "path": f"ssd_mixer_fwd ({plan} plan)", "value": r["value"],
                "ms_per_step": r["ms_per_step"], "mixer_us": r["mixer_us"], "mixer_GBs": r["mixer_GBs"],
                "mixer_frac": r["mixer_GBs"] / HBM_PEAK_GBS, "unit": "head-tokens/s"}

    def two_call_extra(w, r):
        return {"workload": w.name, "path": "ssd_conv_fwd + ssd_chunk_scan_fwd",
                **{k: r[k] for k in ("value", "ms_per_step", "scan_us", "conv_us", "scan_GBs", "conv_GBs")},
                "scan_frac": r["scan_GBs"] / HBM_PEAK_GBS, "conv_frac": r["conv_GBs"] / HBM_PEAK_GBS,
                "unit": "head-tokens/s"}

    extras = []
    if not args.no_extras:
        for plan in ("staged", "fused"):
            extras.append(mixer_extra(wl, mixer_bench(ssd, synth, torch, wl, args.steps, args.warmup, plan=plan),
                                      plan))
        pk = synth.WORKLOADS["mini_k3_packed"]
        extras.append(two_call_extra(pk, prefill_bench(ssd, synth, torch, pk, args.steps, args.warmup, docs=True)))
        ll = synth.WORKLOADS["large_layer_bf16"]
        ls = max(5, args.steps // 2)
        extras.append(two_call_extra(ll, prefill_bench(ssd, synth, torch, ll, ls, args.warmup, h0=True)))
        extras.append(mixer_extra(ll, mixer_bench(ssd, synth, torch, ll, ls, args.warmup, h0=True, plan="fused"),
                                  "fused"))
        dw = synth.WORKLOADS["decode_fp32"]
        r = decode_bench(ssd, synth, torch, dw, max(20, args.steps * 2), args.warmup)
        extras.append({"workload": dw.name + " (ssd_step)", **r, "step_frac": r["step_GBs"] / HBM_PEAK_GBS,
                       "unit": "head-tokens/s (B*H per step)"})
        extras.append(resume_bench(ssd, synth, torch, dw, args.warmup))
        extras.append(f32_prefill_bench(ssd, synth, torch, dw, 3, 2))
        torch.cuda.empty_cache()
        extras.append(s6_bench(ssd, synth, torch, synth.WORKLOADS["s6_bf16"], args.steps, args.warmup))
        extras.append(bwd_bench(ssd, synth, torch, wl, max(5, args.steps // 5), args.warmup))
        torch.cuda.empty_cache()
        extras.append(bwd_bench(ssd, synth, torch, synth.WORKLOADS["large_layer_bf16"], max(3, args.steps // 10),
                                min(args.warmup, 5)))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, wl, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": main_r["value"],
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "L": wl.L, "H": wl.H, "P": wl.P, "N": wl.N, "G": wl.G,
                   "chunk": 64, "conv_k": 4, "gate": True, "step": "ssd_conv_fwd + ssd_chunk_scan_fwd",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": "ssd_chunk_scan_fwd (ssd_scan_bf16_kernel: state-only pre-pass + full pass)",
                     "achieved": main_r["scan_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": main_r["scan_GBs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "launch_us": main_r["scan_us"], "algorithmic_bytes": main_r["scan_bytes"]},
        "kernels": {"scan_us": main_r["scan_us"], "conv_us": main_r["conv_us"], "scan_GBs": main_r["scan_GBs"],
                    "conv_GBs": main_r["conv_GBs"], "conv_frac": main_r["conv_GBs"] / HBM_PEAK_GBS,
                    "scan_head_tokens_per_s": main_r["scan_head_tokens_per_s"],
                    "scan_workspace_bytes": main_r["scan_workspace_bytes"]},
        "cpu_baseline": cpu,
        "extra": extras,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
