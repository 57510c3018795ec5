"""Shared checks of the GPU parity tests: the tolerance rule of every
comparison with the float64 oracle, and progress output."""
import math

import numpy as np


def _say(*a):
    print(*a, flush=True)


BF16_U = 2.0 ** -8  # unit roundoff of bf16: |bf16(x) - x| <= u |x|


def _tol_check(got, ref, io, what="out"):
    """bf16 output: |got - ref| <= 2e-2 RMS(ref) + u_bf16 |ref| element-wise, i.e. the
    stated 2e-2 RMS bound on the computation plus the one rounding of the exact
    result to the output type that every bf16-returning implementation incurs.
    fp32 output: |got - ref| <= 1e-4.  The literal max|d| / RMS is printed too."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite %s" % what
    d = np.abs(got - ref)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    mx = float(d.max()) if d.size else 0.0
    if io == "bf16":
        allow = 2e-2 * rms + BF16_U * np.abs(ref)
        excess = d - BF16_U * np.abs(ref)   # what is left after the output rounding allowance
        worst = float(excess.max() / rms) if d.size else 0.0
    else:
        allow = np.full_like(d, 1e-4)
        worst = mx
    _say("  %s: max|d|/rms=%.3e (literal) max(|d|-u|ref|)/rms=%.3e rel_rms=%.3e rms=%.3e max|ref|/rms=%.1f" % (
        what, mx / max(rms, 1e-30), worst, math.sqrt(float(np.mean(d ** 2))) / max(rms, 1e-30), rms,
        float(np.abs(ref).max()) / max(rms, 1e-30) if d.size else 0.0))
    bad = d > allow
    assert not np.any(bad), "%s: %d elements over the bound, worst excess %.4e" % (
        what, int(bad.sum()), float((d - allow).max()))


def _grad_check(got, ref, io, what):
    """float32 gradients: bf16 inputs |got - ref| <= 2e-2 RMS(ref) + u_bf16 |ref| element-wise (the
    forward's bar); fp32 inputs |got - ref| <= 1e-4 max(1, RMS(ref)) (the forward's 1e-4, relative
    once the gradient's own scale passes 1)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), "non-finite %s" % what
    d = np.abs(got - ref)
    rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
    allow = (2e-2 * rms + BF16_U * np.abs(ref)) if io == "bf16" else np.full_like(d, 1e-4 * max(1.0, rms))
    mx = float(d.max()) if d.size else 0.0
    _say("  %s: max|d|/rms=%.3e rms=%.3e" % (what, mx / max(rms, 1e-30), rms))
    bad = d > allow
    assert not np.any(bad), "%s: %d elements over the bound, worst excess %.4e" % (
        what, int(bad.sum()), float((d - allow).max()))
