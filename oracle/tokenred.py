"""Token reduction in numpy fp64 (test infrastructure only; see __init__).

Page "MiniMax H3 Inference Engine voor Mac computers" -- presets and
implementation notes: an optional token-reduction mode pairs adjacent
horizontal target-video tokens after block 3 while text, audio and reference
tokens stay exact; the full-resolution state is kept as a bypass and
restored before block 40 during the first ten noisy evaluations and before
block 30 afterwards.

Readings (listed in the design doc):
  * merge: a pair (r0, r1) becomes one row holding the mean of the two rows,
    stored in bf16; an unpaired row is copied;
  * the merged row sits at the mean of the two positions (w + 1/2);
  * restore: every full-resolution row gets the bypass (the full state saved
    at the merge) plus the change the reduced blocks made to its merged row:
    x[r] = bypass[r] + (xr_after[i] - xr_before[i]) for r in {r0, r1}, stored
    in bf16.
"""
from __future__ import annotations

import numpy as np

from . import bf16_round, bf16_to_f64


def merge(x_bits, src0, src1) -> np.ndarray:
    """Reduced rows [n_reduced, hidden] as bf16 bits."""
    x = bf16_to_f64(np.asarray(x_bits, np.uint16))
    src0 = np.asarray(src0, np.int64)
    src1 = np.asarray(src1, np.int64)
    out = x[src0].copy()
    pair = src1 >= 0
    out[pair] = (x[src0[pair]] + x[src1[pair]]) / 2.0
    return bf16_round(out)


def unmerge(bypass_bits, xr_before_bits, xr_after_bits, src0, src1) -> np.ndarray:
    """Full-resolution rows [L, hidden] as bf16 bits (every row must be named
    by exactly one entry of src0/src1)."""
    byp = bf16_to_f64(np.asarray(bypass_bits, np.uint16))
    delta = bf16_to_f64(np.asarray(xr_after_bits, np.uint16)) - \
        bf16_to_f64(np.asarray(xr_before_bits, np.uint16))
    out = np.full(byp.shape, np.nan)
    src0 = np.asarray(src0, np.int64)
    src1 = np.asarray(src1, np.int64)
    out[src0] = byp[src0] + delta
    pair = src1 >= 0
    out[src1[pair]] = byp[src1[pair]] + delta[pair]
    assert not np.isnan(out).any(), "every full-resolution row needs a reduced row"
    return bf16_round(out)


def merged_positions(pos, src0, src1) -> np.ndarray:
    """Positions [n_reduced, 3] (fp64, full units) of the reduced rows."""
    pos = np.asarray(pos, np.float64)
    src0 = np.asarray(src0, np.int64)
    src1 = np.asarray(src1, np.int64)
    out = pos[src0].copy()
    pair = src1 >= 0
    out[pair] = (pos[src0[pair]] + pos[src1[pair]]) / 2.0
    return out
