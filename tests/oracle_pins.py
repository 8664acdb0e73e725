"""Pins for the fp64 oracle: each function checks the oracle against something
other than itself (a hand-worked special case, an independent closed form, a
library routine, or an invariant the definition forces).

Every pin takes an ``oracle.Oracle`` so the same checks can run against
deliberately mutated builds (test_oracle_pins.py::test_pins_catch_planted_mistakes).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
from scipy.special import expit

from oracle import closed_forms as cf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_scan_case(seed, *, B=2, L=37, H=4, P=3, N=5, G=2, docs=False, h0=False, gate=False, D=True):
    r = _rng(seed)
    case = dict(
        x=r.standard_normal((B, L, H * P)),
        Bm=r.standard_normal((B, L, G * N)) / math.sqrt(N),
        Cm=r.standard_normal((B, L, G * N)) / math.sqrt(N),
        dt=np.log1p(np.exp(r.standard_normal((B, L, H)) + r.uniform(-4, -1, H))),
        A=-np.exp(r.uniform(0, math.log(16), H)),
        D=r.standard_normal(H) if D else None,
        z=r.standard_normal((B, L, H * P)) if gate else None,
        doc_ids=None,
        init_state=r.standard_normal((B, H, P, N)) * 0.3 if h0 else None,
    )
    if docs:
        ids = np.zeros((B, L), np.int32)
        for b in range(B):
            cuts = sorted(r.choice(np.arange(1, L), size=4, replace=False))
            for c in cuts:
                ids[b, c:] += 1
        # a length-1 document and back-to-back boundaries
        ids[0, 5:] += 1
        ids[0, 6:] += 1
        case["doc_ids"] = ids
    return case, dict(H=H, P=P, N=N, G=G)


# ----------------------------------------------------------------------------- hand vectors
def pin_hand_vectors(o):
    """Scalar worked examples (tests/golden/hand_vectors.json), exact in binary."""
    with open(os.path.join(GOLDEN, "hand_vectors.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L = len(c["x"])
        x = np.array(c["x"], float).reshape(1, L, 1)
        Bm = np.array(c["B"], float).reshape(1, L, 1)
        Cm = np.ones((1, L, 1))
        dt = np.array(c["dt"], float).reshape(1, L, 1)
        doc = None if c["doc"] is None else np.array(c["doc"], np.int32).reshape(1, L)
        h0 = None if c["h0"] is None else np.full((1, 1, 1, 1), float(c["h0"]))
        y, fs = o.scan(x, Bm, Cm, dt, np.array([c["A"]]), np.array([float(c["D"])]), None, doc, h0,
                       H=1, P=1, N=1, G=1, want_state=True)
        np.testing.assert_allclose(y.ravel(), c["y"], rtol=1e-15, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(fs.ravel(), [c["final"]], rtol=1e-15, atol=1e-15, err_msg=c["name"])


# ----------------------------------------------------------------------------- closed forms
def pin_quadratic_form(o, seed=1):
    """Sequential recurrence == materialised (L o C B^T)(dt X) form, with groups, D,
    gate, documents (incl. a length-1 document) and a carried initial state."""
    for variant in (dict(), dict(docs=True), dict(h0=True, gate=True), dict(docs=True, h0=True, gate=True),
                    dict(H=4, G=4, P=2, N=3), dict(H=6, G=1, docs=True, h0=True)):
        case, dims = _tiny_scan_case(seed, **variant)
        y, fs = o.scan(**case, **dims, want_state=True)
        yq, fq = cf.quadratic_form(**case, **dims)
        np.testing.assert_allclose(y, yq, rtol=1e-11, atol=1e-12, err_msg=str(variant))
        np.testing.assert_allclose(fs, fq, rtol=1e-11, atol=1e-12, err_msg=str(variant))


def pin_zero_decay(o, seed=2):
    """A = 0: the state is a running sum (np.cumsum form)."""
    case, dims = _tiny_scan_case(seed)
    case["A"] = np.zeros_like(case["A"])
    y, _ = o.scan(**case, **dims)
    yc = cf.zero_decay_form(case["x"], case["Bm"], case["Cm"], case["dt"], case["D"], **dims)
    np.testing.assert_allclose(y, yc, rtol=1e-12, atol=1e-12)


def pin_softplus_silu_bf16(o):
    """softplus(0) = ln 2; softplus against numpy's logaddexp; the inverse-softplus
    reparameterisation log(exp(sp(v)) - 1) = v; silu against v * expit(v); bf16
    rounding against torch's (round-to-nearest-even) conversion."""
    assert abs(o.softplus(0.0) - math.log(2.0)) < 1e-16
    for v in np.linspace(-30, 30, 61):
        sp = o.softplus(v)
        assert abs(sp - np.logaddexp(0.0, v)) <= 1e-15 * max(1.0, abs(sp))
        if -20 < v < 20:
            assert abs(math.log(math.expm1(sp)) - v) < 1e-9
        assert abs(o.silu(v) - v * expit(v)) <= 1e-15 * max(1.0, abs(v))
    r = _rng(3)
    vals = np.concatenate([r.standard_normal(2000) * s for s in (1e-3, 1.0, 30.0, 1e5)])
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = np.array([o.round_bf16(float(np.float32(v))) for v in vals])
    np.testing.assert_array_equal(got, ref)


def pin_conv_library(o, seed=4):
    """Conv without documents or history == per-channel np.convolve (+bias, +SiLU or none)."""
    r = _rng(seed)
    raw = r.standard_normal((2, 29, 7))
    w = r.standard_normal((7, 4)) * 0.5
    b = r.standard_normal(7) * 0.5
    for act in (0, 1):
        out, _, _ = o.conv(raw, w, b, act=act)
        np.testing.assert_allclose(out, cf.conv_reference(raw, w, b, act_silu=(act == 0)), rtol=1e-13, atol=1e-14)


def pin_conv_impulse(o):
    """Unit impulse at (t0, c) gives w[c,3], w[c,2], w[c,1], w[c,0] at t0..t0+3 (no act):
    the last tap multiplies the current token."""
    L, C = 12, 3
    w = np.arange(1, 13, dtype=float).reshape(C, 4)
    raw = np.zeros((1, L, C))
    raw[0, 4, 1] = 1.0
    out, _, _ = o.conv(raw, w, None, act=1)
    expect = np.zeros((L, C))
    expect[4:8, 1] = w[1, ::-1]
    np.testing.assert_array_equal(out[0], expect)


def pin_conv_documents(o, seed=5):
    """An impulse on a document's last token leaves the next document's conv outputs
    unchanged; packed documents == each document convolved alone (bitwise)."""
    r = _rng(seed)
    L, C = 40, 6
    raw = r.standard_normal((1, L, C))
    w = r.standard_normal((C, 4))
    b = r.standard_normal(C)
    ids = np.zeros((1, L), np.int32)
    ids[0, 17:] = 1
    ids[0, 18:] = 2           # a length-1 document
    ids[0, 30:] = 3
    base, _, _ = o.conv(raw, w, b, doc_ids=ids)
    bumped = raw.copy()
    bumped[0, 16, :] += 100.0
    out2, _, _ = o.conv(bumped, w, b, doc_ids=ids)
    np.testing.assert_array_equal(out2[0, 17:], base[0, 17:])
    assert np.all(out2[0, 16] != base[0, 16])
    for s, e in ((0, 17), (17, 18), (18, 30), (30, L)):
        alone, _, _ = o.conv(raw[:, s:e], w, b)
        np.testing.assert_array_equal(base[:, s:e], alone)


def pin_conv_state_carry(o, seed=6):
    """Conv split at any point, carrying the conv state, == one call (bitwise); a carried
    state feeds only the first document of the next call."""
    r = _rng(seed)
    raw = r.standard_normal((2, 23, 5))
    w = r.standard_normal((5, 4))
    b = r.standard_normal(5)
    s0 = r.standard_normal((2, 3, 5))
    whole, _, st = o.conv(raw, w, b, state_in=s0, want_state=True)
    for cut in (1, 2, 3, 7, 22):
        a, _, sa = o.conv(raw[:, :cut], w, b, state_in=s0, want_state=True)
        c, _, sc = o.conv(raw[:, cut:], w, b, state_in=sa, want_state=True)
        np.testing.assert_array_equal(np.concatenate([a, c], 1), whole)
        np.testing.assert_array_equal(sc, st)
    # documents: a boundary at t = 2 cuts the carried history off from t = 2 onwards
    ids = np.zeros((2, 23), np.int32)
    ids[:, 2:] = 1
    d1, _, _ = o.conv(raw, w, b, doc_ids=ids, state_in=s0)
    d0, _, _ = o.conv(raw, w, b, doc_ids=ids, state_in=np.zeros_like(s0))
    np.testing.assert_array_equal(d1[:, 2:], d0[:, 2:])
    assert np.all(d1[:, :2] != d0[:, :2])


# ----------------------------------------------------------------------------- invariants
def pin_packed_equals_separate(o, seed=7):
    """Packed documents == each document run alone from a zero state (bitwise), and
    the first document alone carries the initial state."""
    case, dims = _tiny_scan_case(seed, B=1, L=50, docs=True, h0=True, gate=True)
    ids = case["doc_ids"][0]
    y, fs = o.scan(**case, **dims, want_state=True)
    starts = [0] + [t for t in range(1, len(ids)) if ids[t] != ids[t - 1]] + [len(ids)]
    for k in range(len(starts) - 1):
        s, e = starts[k], starts[k + 1]
        sub = {n: (None if v is None else v) for n, v in case.items()}
        for n in ("x", "Bm", "Cm", "dt", "z"):
            sub[n] = case[n][:, s:e]
        sub["doc_ids"] = None
        if k > 0:
            sub["init_state"] = None
        ya, fa = o.scan(**sub, **dims, want_state=True)
        np.testing.assert_array_equal(y[:, s:e], ya)
    np.testing.assert_array_equal(fs, fa)


def pin_split_equals_single(o, seed=8):
    """Scan split at any point with the final state carried into the next call == one
    call (bitwise)."""
    case, dims = _tiny_scan_case(seed, L=41, h0=True, gate=True)
    y, fs = o.scan(**case, **dims, want_state=True)
    for cut in (1, 16, 40):
        a = dict(case)
        c = dict(case)
        for n in ("x", "Bm", "Cm", "dt", "z"):
            a[n] = case[n][:, :cut]
            c[n] = case[n][:, cut:]
        ya, fa = o.scan(**a, **dims, want_state=True)
        c["init_state"] = fa
        yc, fc = o.scan(**c, **dims, want_state=True)
        np.testing.assert_array_equal(np.concatenate([ya, yc], 1), y)
        np.testing.assert_array_equal(fc, fs)


def pin_step_equals_prefill(o, seed=9):
    """A prefill of L0 tokens followed by single-token steps == one prefill over all
    tokens (bitwise): y, the SSM state and the conv state, in fp64 and with the bf16
    storage rounding of the conv output."""
    r = _rng(seed)
    B, H, P, N, G, K = 2, 4, 3, 5, 2, 4
    C = H * P + 2 * G * N
    L0, S = 9, 6
    raw = r.standard_normal((B, L0 + S, C))
    dt_raw = r.standard_normal((B, L0 + S, H))
    z = r.standard_normal((B, L0 + S, H * P))
    w = r.standard_normal((C, K)) * 0.5
    bias = r.standard_normal(C) * 0.5
    dt_bias = r.uniform(-4, -1, H)
    A = -np.exp(r.uniform(0, math.log(16), H))
    D = r.standard_normal(H)
    for rb in (False, True):
        kw = dict(H=H, P=P, N=N, G=G, round_bf16=rb)
        y_all, fs_all, cs_all, _, _ = o.forward(raw, w, bias, dt_raw, dt_bias, A, D, z, **kw)
        y0, fs0, cs0, _, _ = o.forward(raw[:, :L0], w, bias, dt_raw[:, :L0], dt_bias, A, D, z[:, :L0], **kw)
        np.testing.assert_array_equal(y0, y_all[:, :L0])
        conv_state = np.ascontiguousarray(cs0)
        ssm_state = np.ascontiguousarray(fs0)
        for s in range(S):
            t = L0 + s
            ys = o.step(raw[:, t], dt_raw[:, t], z[:, t], w, bias, dt_bias, A, D, conv_state, ssm_state, **kw)
            np.testing.assert_array_equal(ys, y_all[:, t])
        np.testing.assert_array_equal(ssm_state, fs_all)
        np.testing.assert_array_equal(conv_state, cs_all)


def pin_linearity_and_decay_only(o, seed=10):
    """With no gate and zero h0, y is linear in x; with x = 0, y_t = exp(cs_t) C_t . h0
    (the carried state only decays)."""
    case, dims = _tiny_scan_case(seed)
    x1 = case["x"]
    x2 = _rng(seed + 100).standard_normal(x1.shape)
    ya, _ = o.scan(**{**case, "x": x1}, **dims)
    yb, _ = o.scan(**{**case, "x": x2}, **dims)
    yab, _ = o.scan(**{**case, "x": 2.0 * x1 - 3.0 * x2}, **dims)
    np.testing.assert_allclose(yab, 2.0 * ya - 3.0 * yb, rtol=1e-11, atol=1e-11)
    case, dims = _tiny_scan_case(seed, h0=True)
    case["x"] = np.zeros_like(case["x"])
    y, _ = o.scan(**case, **dims)
    H, P, N, G = dims["H"], dims["P"], dims["N"], dims["G"]
    for b in range(case["x"].shape[0]):
        for h in range(H):
            g = h // (H // G)
            cs = np.cumsum(case["dt"][b, :, h] * case["A"][h])
            Cg = case["Cm"][b, :, g * N:(g + 1) * N]
            expect = np.exp(cs)[:, None] * (Cg @ case["init_state"][b, h].T)
            np.testing.assert_allclose(y[b, :, h * P:(h + 1) * P], expect, rtol=1e-11, atol=1e-13)


def pin_groups_and_batch(o, seed=11):
    """G groups holding identical B and C == one group; permuting batch rows permutes y."""
    case, dims = _tiny_scan_case(seed, B=3, H=4, G=2, docs=True, h0=True, gate=True)
    N = dims["N"]
    Bm1, Cm1 = case["Bm"][..., :N], case["Cm"][..., :N]
    c2 = {**case, "Bm": np.concatenate([Bm1, Bm1], -1), "Cm": np.concatenate([Cm1, Cm1], -1)}
    y2, f2 = o.scan(**c2, **dims, want_state=True)
    y1, f1 = o.scan(**{**case, "Bm": Bm1, "Cm": Cm1}, **{**dims, "G": 1}, want_state=True)
    np.testing.assert_array_equal(y2, y1)
    np.testing.assert_array_equal(f2, f1)
    perm = [2, 0, 1]
    yp, fp = o.scan(**{k: (v[perm] if isinstance(v, np.ndarray) and v.ndim >= 2 and k != "A" else v)
                       for k, v in case.items()}, **dims, want_state=True)
    y, f = o.scan(**case, **dims, want_state=True)
    np.testing.assert_array_equal(yp, y[perm])
    np.testing.assert_array_equal(fp, f[perm])


def pin_dt_softplus_inside(o, seed=12):
    """dt_softplus = 1 with raw dt and bias == dt activated beforehand with numpy's logaddexp."""
    case, dims = _tiny_scan_case(seed)
    r = _rng(seed)
    raw = r.standard_normal(case["dt"].shape)
    bias = r.uniform(-4, -1, dims["H"])
    y1, _ = o.scan(**{**case, "dt": raw}, **dims, dt_softplus=True, dt_bias=bias)
    y2, _ = o.scan(**{**case, "dt": np.logaddexp(0.0, raw + bias)}, **dims)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- Mamba-1 S6
def _tiny_s6_case(seed, *, B=2, L=29, D=5, N=4, docs=False, h0=False, gate=False, Dskip=True):
    r = _rng(seed)
    case = dict(
        x=r.standard_normal((B, L, D)),
        dt=np.log1p(np.exp(r.standard_normal((B, L, D)) + r.uniform(-4, -1, D))),
        A=-np.exp(r.uniform(-1.0, math.log(16), (D, N))),
        Bm=r.standard_normal((B, L, N)) / math.sqrt(N),
        Cm=r.standard_normal((B, L, N)) / math.sqrt(N),
        D=r.standard_normal(D) if Dskip else None,
        z=r.standard_normal((B, L, D)) if gate else None,
        doc_ids=None,
        init_state=r.standard_normal((B, D, N)) * 0.3 if h0 else None,
    )
    if docs:
        ids = np.zeros((B, L), np.int32)
        for b in range(B):
            for c in sorted(r.choice(np.arange(1, L), size=3, replace=False)):
                ids[b, c:] += 1
        ids[0, 4:] += 1
        ids[0, 5:] += 1                                   # a length-1 document
        case["doc_ids"] = ids
    return case


def pin_s6_quadratic_form(o, seed=20):
    """S6 recurrence == per-(d, n) materialised decay-matrix form, with D skip, gate, documents and a carried
    initial state (per-n decay rates, so a decay taken from the wrong state index is caught)."""
    for variant in (dict(), dict(docs=True), dict(h0=True, gate=True), dict(docs=True, h0=True, gate=True),
                    dict(D=1, N=7), dict(N=1, h0=True)):
        case = _tiny_s6_case(seed, **variant)
        y, fs = o.s6(**case, want_state=True)
        yq, fq = cf.s6_quadratic_form(**case)
        np.testing.assert_allclose(y, yq, rtol=1e-11, atol=1e-12, err_msg=str(variant))
        np.testing.assert_allclose(fs, fq, rtol=1e-11, atol=1e-12, err_msg=str(variant))


def pin_s6_equals_ssd(o, seed=21):
    """With A[d, n] equal to its head's A for every n and dt equal across a head's P channels, the S6 scan is
    the SSD scan with one group (both run through their own oracle routines)."""
    B, L, H, P, N = 2, 33, 3, 4, 5
    case, dims = _tiny_scan_case(seed, B=B, L=L, H=H, P=P, N=N, G=1, docs=True, h0=True, gate=True)
    y_ssd, f_ssd = o.scan(**case, **dims, want_state=True)
    dt6 = np.repeat(case["dt"], P, axis=2)                # [B, L, H*P]
    A6 = np.repeat(case["A"], P)[:, None] * np.ones((1, N))
    h06 = case["init_state"].reshape(B, H * P, N)         # [B][H][P][N] -> channels h*P + p
    y6, f6 = o.s6(case["x"], dt6, A6, case["Bm"], case["Cm"], np.repeat(case["D"], P), case["z"],
                  case["doc_ids"], h06, want_state=True)
    np.testing.assert_allclose(y6, y_ssd, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f6.reshape(B, H, P, N), f_ssd, rtol=1e-12, atol=1e-13)


def pin_s6_zero_decay_and_carry(o, seed=22):
    """A = 0: the state is a running sum (np.cumsum); a prefill split anywhere with the state carried equals one
    pass bit for bit; raw dt with its bias through the softplus equals dt activated with numpy's logaddexp."""
    case = _tiny_s6_case(seed, Dskip=True)
    case["A"] = np.zeros_like(case["A"])
    y, _ = o.s6(**case)
    hsum = np.cumsum(case["dt"][..., None] * case["Bm"][:, :, None, :] * case["x"][..., None], axis=1)
    expect = (hsum * case["Cm"][:, :, None, :]).sum(-1) + case["D"] * case["x"]
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)
    case = _tiny_s6_case(seed + 1, docs=True, h0=True, gate=True)
    y, f = o.s6(**case, want_state=True)
    for cut in (1, 13, 28):
        sl = lambda v, a, b: None if v is None else v[:, a:b]
        ya, fa = o.s6(case["x"][:, :cut], case["dt"][:, :cut], case["A"], case["Bm"][:, :cut], case["Cm"][:, :cut],
                      case["D"], sl(case["z"], 0, cut), sl(case["doc_ids"], 0, cut), case["init_state"],
                      want_state=True)
        ids_c = sl(case["doc_ids"], cut, None)
        # the second call's t = 0 continues its state: a cut on a document start passes a zero state
        yc, fc = o.s6(case["x"][:, cut:], case["dt"][:, cut:], case["A"], case["Bm"][:, cut:], case["Cm"][:, cut:],
                      case["D"], sl(case["z"], cut, None), ids_c,
                      np.where((case["doc_ids"][:, cut] != case["doc_ids"][:, cut - 1])[:, None, None], 0.0, fa),
                      want_state=True)
        np.testing.assert_array_equal(np.concatenate([ya, yc], 1), y)
        np.testing.assert_array_equal(fc, f)
    r = _rng(seed + 2)
    raw = r.standard_normal(case["dt"].shape)
    bias = r.uniform(-4, -1, case["x"].shape[2])
    y1, _ = o.s6(**{**case, "dt": raw}, dt_softplus=True, dt_bias=bias)
    y2, _ = o.s6(**{**case, "dt": np.logaddexp(0.0, raw + bias)})
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- backward (VJP)
def _fd_check(f, grad, X, seed, name, eps=1e-5, rtol=1e-6, ndir=3):
    """<grad, V> against the central difference (f(X + eps V) - f(X - eps V)) / (2 eps) along random V.
    f is fp64 and smooth, so the two agree to ~1e-9 relative; the bar is 1e-6 of the summed term sizes."""
    r = _rng(seed)
    X = np.asarray(X, np.float64)
    for k in range(ndir):
        V = r.standard_normal(X.shape)
        lhs = float(np.sum(grad * V))
        rhs = (f(X + eps * V) - f(X - eps * V)) / (2 * eps)
        scale = float(np.sum(np.abs(grad * V))) + 1e-300
        assert abs(lhs - rhs) <= rtol * scale, f"{name} direction {k}: <g,v>={lhs!r} fd={rhs!r} scale={scale!r}"


def _scan_bwd_case(seed, *, softplus, **kw):
    case, dims = _tiny_scan_case(seed, **kw)
    r = _rng(seed + 1000)
    case.pop("init_state")
    if softplus:
        case["dt"] = r.standard_normal(case["dt"].shape)
        case["dt_bias"] = r.uniform(-4, -1, dims["H"])
    gy = r.standard_normal(case["x"].shape)
    return case, dims, gy


def pin_scan_bwd_finite_differences(o, seed=30):
    """Every gradient of the scan's backward against central differences of the forward oracle, with and
    without documents, gate, D skip, groups and the softplus on dt."""
    for variant in (dict(softplus=False), dict(softplus=True, docs=True, gate=True),
                    dict(softplus=True, G=1, H=2, docs=True), dict(softplus=False, gate=True, D=False, N=1, P=2)):
        case, dims, gy = _scan_bwd_case(seed, **variant)
        sp = variant["softplus"]
        g = o.scan_bwd(case["x"], case["Bm"], case["Cm"], case["dt"], case["A"], gy, case["D"], case["z"],
                       case["doc_ids"], dt_softplus=sp, dt_bias=case.get("dt_bias"), **dims)
        names = ["x", "Bm", "Cm", "dt", "A"] + (["D"] if case["D"] is not None else []) + \
                (["z"] if case["z"] is not None else []) + (["dt_bias"] if sp else [])
        for i, nm in enumerate(names):
            def f(v, nm=nm):
                c = dict(case)
                c[nm] = v
                y, _ = o.scan(c["x"], c["Bm"], c["Cm"], c["dt"], c["A"], c["D"], c["z"], c["doc_ids"],
                              dt_softplus=sp, dt_bias=c.get("dt_bias"), **dims)
                return float(np.sum(gy * y))
            _fd_check(f, g[nm], case[nm], seed + 7 * i, f"{variant} d{nm}")


def _conv_bwd_case(seed, *, B=2, L=23, C=7, K=4, H=3, docs=True):
    r = _rng(seed)
    case = dict(raw=r.standard_normal((B, L, C)), w=r.standard_normal((C, K)) * 0.5, bias=r.standard_normal(C),
                dt_raw=r.standard_normal((B, L, H)), dt_bias=r.uniform(-4, -1, H), doc_ids=None)
    if docs:
        ids = np.zeros((B, L), np.int32)
        for b in range(B):
            for c in sorted(r.choice(np.arange(1, L), size=3, replace=False)):
                ids[b, c:] += 1
        ids[0, 9:] += 1
        ids[0, 10:] += 1                                   # a length-1 document
        case["doc_ids"] = ids
    return case, r.standard_normal((B, L, C)), r.standard_normal((B, L, H))


def pin_conv_bwd_finite_differences(o, seed=31):
    """Every gradient of the conv's backward (SiLU and identity activations, documents) against central
    differences of the forward conv."""
    for act in (0, 1):
        case, dout, ddt = _conv_bwd_case(seed + act)
        g = o.conv_bwd(case["raw"], case["w"], dout, case["bias"], case["dt_raw"], case["dt_bias"], ddt,
                       case["doc_ids"], act=act)
        for i, nm in enumerate(["raw", "w", "bias", "dt_raw", "dt_bias"]):
            def f(v, nm=nm):
                c = dict(case)
                c[nm] = v
                out, dt, _ = o.conv(c["raw"], c["w"], c["bias"], c["dt_raw"], c["dt_bias"], c["doc_ids"], act=act)
                return float(np.sum(dout * out) + np.sum(ddt * dt))
            _fd_check(f, g[nm], case[nm], seed + 11 * i, f"act={act} d{nm}")


def _mixer_case(seed, *, B=2, L=21, H=2, P=3, N=4, G=1, docs=True):
    r = _rng(seed)
    C = H * P + 2 * G * N
    case = dict(raw=r.standard_normal((B, L, C)), w=r.standard_normal((C, 4)) * 0.5, bias=r.standard_normal(C) * 0.5,
                dt_raw=r.standard_normal((B, L, H)), dt_bias=r.uniform(-4, -1, H), A=-np.exp(r.uniform(0, 2.7, H)),
                D=r.standard_normal(H), z=r.standard_normal((B, L, H * P)))
    ids = None
    if docs:
        ids = np.zeros((B, L), np.int32)
        for b in range(B):
            for c in sorted(r.choice(np.arange(1, L), size=3, replace=False)):
                ids[b, c:] += 1
    return case, ids, dict(H=H, P=P, N=N, G=G), r.standard_normal((B, L, H * P))


def pin_mixer_bwd_finite_differences(o, seed=32):
    """The composed backward (conv -> scan) against central differences of forward() end to end."""
    case, ids, dims, gy = _mixer_case(seed)
    g = o.mixer_bwd(*[case[k] for k in ("raw", "w", "bias", "dt_raw", "dt_bias", "A", "D", "z")], gy, doc_ids=ids,
                    **dims)
    keys = ("raw", "w", "bias", "dt_raw", "dt_bias", "A", "D", "z")
    for i, nm in enumerate(keys):
        def f(v, nm=nm):
            c = dict(case)
            c[nm] = v
            y = o.forward(*[c[k] for k in keys], doc_ids=ids, **dims)[0]
            return float(np.sum(gy * y))
        _fd_check(f, g[nm], case[nm], seed + 13 * i, f"mixer d{nm}")


def pin_bwd_document_isolation(o, seed=33):
    """A loss on a later document gives exactly zero gradient on every earlier-document input (scan and
    conv -> scan), and the per-token gradients of a packed row's document equal, bit for bit, those of the
    document run alone."""
    case, dims, gy = _scan_bwd_case(seed, softplus=True, docs=True, gate=True)
    ids = case["doc_ids"]
    for b in range(ids.shape[0]):
        k = ids[b, -1]
        start = int(np.argmax(ids[b] == k))
        assert start > 0
        gk = np.zeros_like(gy)
        gk[b, start:] = gy[b, start:]
        g = o.scan_bwd(case["x"], case["Bm"], case["Cm"], case["dt"], case["A"], gk, case["D"], case["z"], ids,
                       dt_softplus=True, dt_bias=case["dt_bias"], **dims)
        for nm in ("x", "Bm", "Cm", "dt", "z"):
            assert np.all(g[nm][:, :start] == 0.0) and np.all(g[nm][1 - b] == 0.0), f"scan d{nm} row {b}"
        # the same document alone
        sl = lambda t: t[b:b + 1, start:]
        ga = o.scan_bwd(sl(case["x"]), sl(case["Bm"]), sl(case["Cm"]), sl(case["dt"]), case["A"], sl(gy),
                        case["D"], sl(case["z"]), None, dt_softplus=True, dt_bias=case["dt_bias"], **dims)
        for nm in ("x", "Bm", "Cm", "dt", "z"):
            assert np.array_equal(g[nm][b:b + 1, start:], ga[nm]), f"packed vs alone d{nm} row {b}"
    mcase, mids, mdims, mgy = _mixer_case(seed + 1)
    for b in range(mids.shape[0]):
        k = mids[b, -1]
        start = int(np.argmax(mids[b] == k))
        gk = np.zeros_like(mgy)
        gk[b, start:] = mgy[b, start:]
        g = o.mixer_bwd(*[mcase[k] for k in ("raw", "w", "bias", "dt_raw", "dt_bias", "A", "D", "z")], gk,
                        doc_ids=mids, **mdims)
        for nm in ("raw", "dt_raw", "z"):
            assert np.all(g[nm][:, :start] == 0.0) and np.all(g[nm][1 - b] == 0.0), f"mixer d{nm} row {b}"


ALL_PINS = [
    pin_hand_vectors, pin_quadratic_form, pin_zero_decay, pin_softplus_silu_bf16, pin_conv_library,
    pin_conv_impulse, pin_conv_documents, pin_conv_state_carry, pin_packed_equals_separate,
    pin_split_equals_single, pin_step_equals_prefill, pin_linearity_and_decay_only, pin_groups_and_batch,
    pin_dt_softplus_inside, pin_s6_quadratic_form, pin_s6_equals_ssd, pin_s6_zero_decay_and_carry,
    pin_scan_bwd_finite_differences, pin_conv_bwd_finite_differences, pin_mixer_bwd_finite_differences,
    pin_bwd_document_isolation,
]
