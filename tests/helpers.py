"""Tolerance checks shared by the GPU parity tests.

Bars (each test states which one it uses):
  * fp32 inputs: max |gpu - oracle| <= 1e-3 * RMS(oracle), per tensor.
  * bf16 inputs with fp32 accumulation: max |gpu - oracle| <= 0.03125.
  * a bf16-stored conv output: within one bf16 ulp of the fp64 oracle value
    (the kernel rounds an fp32 value, the oracle an fp64 one, to the same grid)
    plus the fp32 accumulation error of the pre-activation sum, 8 * 2^-24 *
    (|bias| + sum |w x|) -- an output near zero can come from cancelling O(1)
    terms, and fp32 cannot resolve it better than that.
  * the bf16 conv -> scan pipeline end to end: 0.03125 plus, per element, the
    one-ulp storage difference of x that the D skip carries into y
    (|D_h| * ulp(x) * |silu(z)|).
  * gradients through a bf16-stored conv output: relative L2 error
    ||gpu - oracle|| <= 1e-3 ||oracle|| per tensor (assert_rel_l2).  The two
    pipelines round the conv output to bf16 from fp32 and fp64 values, and a
    few of them land on adjacent bf16 values; each such one-ulp input change
    moves that token's gradients by up to 2^-8 relative, sparse in number.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_TOL = 0.03125
FP32_REL = 1e-3


def np64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().double().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def rms(a):
    a = np64(a)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits)."""
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(int))


def report(name, got, ref):
    d = np.abs(np64(got) - np64(ref))
    i = int(np.argmax(d)) if d.size else 0
    return f"{name}: max|d|={d.max() if d.size else 0:.3e} at {np.unravel_index(i, d.shape) if d.size else ()} rms(ref)={rms(ref):.3e}"


def assert_fp32(got, ref, name):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    bound = FP32_REL * rms(ref)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= bound, report(name, got, ref) + f" > 1e-3*rms = {bound:.3e}"
    return err


def assert_bf16(got, ref, name, tol=BF16_TOL):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= tol, report(name, got, ref) + f" > {tol}"
    return err


def assert_within_ulp(got, ref, name, mag=None, ulps=1.0):
    """bf16-stored output vs the fp64 value it rounds: |d| <= ulps * ulp(ref) + 8 * 2^-24 * mag, where mag is
    the magnitude |bias| + sum |w x| of the fp32 pre-activation sum (0 if not given)."""
    got, ref = np64(got), np64(ref)
    d = np.abs(got - ref)
    lim = ulps * bf16_ulp(ref)
    if mag is not None:
        lim = lim + 8.0 * 2.0 ** -24 * np64(mag)
    bad = d > lim
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} elements beyond the bound; first at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {lim[i]!r}")
    return float(d.max()) if d.size else 0.0


def assert_pipeline(y_gpu, y_ref, x_ref, z, D, H, P, name):
    """End-to-end bound for the bf16 conv -> scan pipeline (see module doc)."""
    y_gpu, y_ref, x_ref = np64(y_gpu), np64(y_ref), np64(x_ref)
    gate = np.ones_like(y_ref) if z is None else np.abs(np64(z) / (1.0 + np.exp(-np64(z))))
    Dfull = np.repeat(np.abs(np64(D)), P)[None, None, :] if D is not None else 0.0
    lim = BF16_TOL + Dfull * bf16_ulp(x_ref) * gate
    d = np.abs(y_gpu - y_ref)
    bad = d > lim
    assert not bad.any(), report(name, y_gpu, y_ref) + f"; {int(bad.sum())} elements beyond the pipeline bound"
    return float(d.max())


def assert_rel_l2(got, ref, name, tol=1e-3):
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    den = float(np.sqrt(np.sum(ref ** 2)))
    assert num <= tol * den, report(name, got, ref) + f"; relative L2 {num / max(den, 1e-300):.3e} > {tol:g}"
    return num / max(den, 1e-300)
