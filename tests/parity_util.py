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


class StreamCheck:
    """_tol_check over an output compared block by block (a long head whose oracle runs in pieces,
    each continued from the previous piece's final state).  The element-wise rule
    |d| <= 2e-2 RMS(ref) + u |ref| (bf16) is max(|d| - u |ref|) <= 2e-2 RMS(ref), so the largest
    excess, the sums for the RMS values and the largest |d| and |ref| are all it needs to keep."""

    def __init__(self, io, what):
        self.io, self.what = io, what
        self.n = 0
        self.ss_ref = self.ss_d = 0.0
        self.max_d = self.max_ref = self.max_excess = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape
        assert np.all(np.isfinite(got)), "non-finite %s" % self.what
        if ref.size == 0:
            return
        d = np.abs(got - ref)
        self.n += d.size
        self.ss_ref += float(np.sum(ref ** 2))
        self.ss_d += float(np.sum(d ** 2))
        self.max_d = max(self.max_d, float(d.max()))
        self.max_ref = max(self.max_ref, float(np.abs(ref).max()))
        if self.io == "bf16":
            self.max_excess = max(self.max_excess, float((d - BF16_U * np.abs(ref)).max()))

    def finish(self):
        """Asserts the bar; returns the figures printed (literal max|d|/RMS, excess/RMS, RMS(d)/RMS)."""
        rms = math.sqrt(self.ss_ref / max(self.n, 1))
        r = max(rms, 1e-30)
        stats = {"literal": self.max_d / r, "excess": (self.max_excess if self.io == "bf16" else self.max_d) / r,
                 "rel_rms": math.sqrt(self.ss_d / max(self.n, 1)) / r, "rms": rms, "max_ref_over_rms": self.max_ref / r}
        _say("  %s: max|d|/rms=%.3e (literal) max(|d|-u|ref|)/rms=%.3e rel_rms=%.3e rms=%.3e max|ref|/rms=%.1f" % (
            self.what, stats["literal"], stats["excess"], stats["rel_rms"], rms, stats["max_ref_over_rms"]))
        if self.io == "bf16":
            assert self.max_excess <= 2e-2 * rms, "%s: excess over the rounding allowance %.4e > 2e-2 RMS = %.4e" % (
                self.what, self.max_excess, 2e-2 * rms)
        else:
            assert self.max_d <= 1e-4, "%s: max|d| %.4e > 1e-4" % (self.what, self.max_d)
        return stats
