"""CPU prediction of which Gamma-scaled operands leave the 16-bit range.

TEST INFRASTRUCTURE ONLY.

The pages' claim (first page, "Practical Techniques ...", sec. 3.1-3.3; third
page, "Breaking Through ...", sec. 2.1): with an unbounded log-decay the inverse
cumulative decay 1/Gamma overflows in BF16, forcing an element-wise path for the
diagonal blocks; with g >= g_min = -5 the inverse stays representable inside any
16-token tile, so every tile can be a dense product.

Referencing each 16-token row tile I to its first row (rho_I = G at row 16 I),
the only scale factors above 1 are those of the key operand of the diagonal
tile, k_s * exp(rho_I - G_s) for s in tile I; their exponent is a sum of at most
15 gates, so it is at most 15 * |g_min| = 75 < ln(bf16 max) = 88.72.

`subtile_operand_overflow` counts, exactly as a device computing those factors
as 2^x in float32 and rounding to bf16 would see them, how many of these
operands are +-inf/NaN; `borderline` counts the ones within `band` (in log2
units) of the threshold, where float32 rounding order can flip the outcome.
"""
from __future__ import annotations

import math

import numpy as np

from .reference import SUBTILE, gate

LOG2E = 1.0 / math.log(2.0)
# float -> bf16 round-to-nearest-even overflows at the midpoint between the
# largest bf16 (2^128 - 2^120) and 2^128.
BF16_OVERFLOW_LOG2 = 128.0 + math.log2(1.0 - 2.0 ** -9)
FP32_OVERFLOW_LOG2 = 128.0 + math.log2(1.0 - 2.0 ** -25)


def _chunk_cumsum(g, chunk):
    """Inclusive cumulative sum of g along time, restarted every `chunk` tokens."""
    T = g.shape[-2]
    if T % chunk == 0:  # every chunk at once (the same sequential sums as one chunk at a time)
        s = g.shape
        return np.cumsum(g.reshape(s[:-2] + (T // chunk, chunk, s[-1])), axis=-2).reshape(s)
    G = np.empty_like(g)
    for n0 in range(0, T, chunk):
        G[..., n0:n0 + chunk, :] = np.cumsum(g[..., n0:n0 + chunk, :], axis=-2)
    return G


def subtile_spans(a, g_min=-5.0, chunk=64, gate_mode="bounded"):
    """Largest exponent rho_I - G_s (natural log) over all diagonal sub-tiles."""
    g = gate(a, g_min, gate_mode)
    G = _chunk_cumsum(g, chunk)
    T = g.shape[-2]
    best = 0.0
    for s0 in range(0, T, SUBTILE):
        rho = G[..., s0:s0 + 1, :]
        best = max(best, float(np.max(rho - G[..., s0:s0 + SUBTILE, :])))
    return best


def subtile_operand_overflow(a, k, g_min=-5.0, chunk=64, gate_mode="bounded",
                             operand="bf16", band=0.02):
    """Returns (count, borderline) of non-finite diagonal-sub-tile key operands."""
    thr = BF16_OVERFLOW_LOG2 if operand == "bf16" else FP32_OVERFLOW_LOG2
    g = gate(a, g_min, gate_mode)
    G = _chunk_cumsum(g, chunk) * LOG2E
    k = np.asarray(k, dtype=np.float64)
    T = g.shape[-2]
    count = 0
    border = 0
    with np.errstate(divide="ignore"):
        lk = np.log2(np.abs(k))
    if T % SUBTILE == 0:  # every sub-tile at once, the same element-wise arithmetic as the loop below
        shp = G.shape[:-2] + (T // SUBTILE, SUBTILE, G.shape[-1])
        G4 = G.reshape(shp)
        x = G4[..., 0:1, :] - G4
        y = x + lk.reshape(shp)
        bad = (x >= 128.0) | (y >= thr)
        near = (np.abs(x - 128.0) < band) | (np.abs(y - thr) < band)
        return int(np.count_nonzero(bad)), int(np.count_nonzero(near))
    for s0 in range(0, T, SUBTILE):
        x = G[..., s0:s0 + 1, :] - G[..., s0:s0 + SUBTILE, :]      # log2 of the factor
        y = x + lk[..., s0:s0 + SUBTILE, :]                         # log2 |operand|
        bad = (x >= 128.0) | (y >= thr)
        count += int(np.count_nonzero(bad))
        border += int(np.count_nonzero((np.abs(x - 128.0) < band) | (np.abs(y - thr) < band)))
    return count, border


def whole_chunk_inverse_overflow(a, k, g_min=-5.0, chunk=64, gate_mode="bounded"):
    """Context only: how many k_s / Gamma_s operands would overflow bf16 if the
    inverse decay were referenced to the chunk start instead of the sub-tile."""
    g = gate(a, g_min, gate_mode)
    x = -_chunk_cumsum(g, chunk) * LOG2E
    with np.errstate(divide="ignore"):
        y = x + np.log2(np.abs(np.asarray(k, dtype=np.float64)))
    return int(np.count_nonzero((x >= 128.0) | (y >= BF16_OVERFLOW_LOG2)))
