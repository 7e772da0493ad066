"""Coverage diagnostic over a selection's output.

HubKV walkthrough page, "Observation" and its motivation: a plain Top-K over
clustered scores spends the budget on many neighbouring tokens of the same
high-scoring stretch (repetition), while the hub-aware correction is meant to
spread it over more distinct stretches (coverage).  With synthetic inputs the
stretches are known -- the planted key bursts -- so coverage is simply the
number of bursts that keep at least one token.

This is a measurement over host copies of the kept indices, not a step of the
path: the path itself (score, refine, select) runs in the library's kernels.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def cluster_coverage(idx: np.ndarray, kept: Sequence[int], spans) -> np.ndarray:
    """Bursts with at least one kept token.

    idx: int32 [L][Hkv][sum kept] positions local to their sequence, the
    sequences' slices back to back (the layout hubkv_select writes).
    kept: kept count per sequence.  spans: per sequence, a list of
    non-overlapping [start, end) bursts in ascending order.
    Returns int64 [L][Hkv][B]: covered bursts per (layer, head, sequence).
    """
    idx = np.asarray(idx)
    L, H, _ = idx.shape
    B = len(kept)
    out = np.zeros((L, H, B), np.int64)
    off = np.concatenate([[0], np.cumsum(np.asarray(kept, np.int64))])
    for b in range(B):
        if not spans[b]:
            continue
        starts = np.array([s for s, _ in spans[b]], np.int64)
        ends = np.array([e for _, e in spans[b]], np.int64)
        for l in range(L):
            for h in range(H):
                p = idx[l, h, off[b]:off[b + 1]].astype(np.int64)
                j = np.searchsorted(starts, p, side="right") - 1
                inside = (j >= 0) & (p < ends[np.maximum(j, 0)])
                out[l, h, b] = np.unique(j[inside]).size
    return out


def tokens_in_clusters(idx: np.ndarray, kept: Sequence[int], spans) -> np.ndarray:
    """Kept tokens that fall inside any burst, per (layer, head, sequence)."""
    idx = np.asarray(idx)
    L, H, _ = idx.shape
    B = len(kept)
    out = np.zeros((L, H, B), np.int64)
    off = np.concatenate([[0], np.cumsum(np.asarray(kept, np.int64))])
    for b in range(B):
        if not spans[b]:
            continue
        starts = np.array([s for s, _ in spans[b]], np.int64)
        ends = np.array([e for _, e in spans[b]], np.int64)
        for l in range(L):
            for h in range(H):
                p = idx[l, h, off[b]:off[b + 1]].astype(np.int64)
                j = np.searchsorted(starts, p, side="right") - 1
                out[l, h, b] = int(((j >= 0) & (p < ends[np.maximum(j, 0)])).sum())
    return out
