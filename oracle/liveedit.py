"""O4: LiveEdit's active-row mask and active-row attention (test
infrastructure only; see the package docstring).

Source: aitrends.kr, "LiveEdit 실시간 Diffusion 기반 스트리밍 비디오 편집",
methodology and technical-detail sections (AR-oriented Mask Cache).  For
chunk k the mask is 1 where the L2 distance between the previous chunk's
edited latent and its source latent, taken per position, exceeds a
threshold tau; tau is set dynamically so that about 70% of the tokens are
pruned.  Active positions get the full computation; the others reuse the
previous chunk's cached features.

Readings (each listed in the design notes):
  * the distance is taken per token over its channel vector;
  * the decision is taken on the squared distance, summed over channels in
    order in float64 with every difference, square and addition rounded on
    its own, against tau * tau in float64 (the same precision on both sides,
    so the integer result is exact);
  * the dynamic threshold is a top-k rule: the `keep` tokens with the largest
    distance are active, equal distances ranked by lower index;
  * a NaN distance counts as -1 (never above a threshold, ranked last);
  * for attention, "reuse the cached feature" means the output rows of
    inactive tokens keep the previous chunk's values: the result is O1 on the
    active rows, copied into the previous output.
"""
from __future__ import annotations

import numpy as np

from .attention import as_f64


def distance_sq(z_src, z_edit) -> np.ndarray:
    """Squared L2 distance per token, float64, channels summed in order."""
    s = as_f64(z_src)
    e = as_f64(z_edit)
    tokens, channels = s.shape
    acc = np.zeros(tokens, dtype=np.float64)
    for c in range(channels):
        d = e[:, c] - s[:, c]
        sq = d * d
        acc = acc + sq
    acc[np.isnan(acc)] = -1.0
    return acc


def active_rows_threshold(z_src, z_edit, tau: float) -> np.ndarray:
    """Indices (ascending) of the tokens whose distance exceeds tau."""
    t = np.float64(np.float32(tau))
    return np.flatnonzero(distance_sq(z_src, z_edit) > t * t).astype(np.int32)


def active_rows_topk(z_src, z_edit, keep: int) -> np.ndarray:
    """Indices (ascending) of the `keep` tokens with the largest distance;
    equal distances are ranked by lower index."""
    dsq = distance_sq(z_src, z_edit)
    order = sorted(range(len(dsq)), key=lambda i: (-dsq[i], i))
    return np.array(sorted(order[:max(0, keep)]), dtype=np.int32)


def rows_output(previous: np.ndarray, full: np.ndarray, rows) -> np.ndarray:
    """The previous chunk's output with the active rows replaced by this
    chunk's attention output (`full` holds that output for every row)."""
    out = np.array(previous, dtype=np.float64, copy=True)
    rows = np.asarray(rows, dtype=np.int64)
    out[rows] = full[rows]
    return out
