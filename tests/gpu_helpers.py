"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import os
import sys

import numpy as np

import synthetic as S


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def note(msg: str) -> None:
    """Write straight to the real stderr (bypassing capture) so a GPU step is
    named before it runs."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def to_dev(x: np.ndarray, dtype: str):
    """float32 host array (bf16-representable when dtype == 'bf16') -> torch GPU tensor."""
    import torch
    if dtype == "bf16":
        bits = S.to_bf16_bits(x).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return S.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def rel_err(a, b, floor=1e-30):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), floor)


def near_tie_sets_ok(idx_gpu, idx_orc, z_orc, seqlens, kept, n_sink, n_recent, tol):
    """Kept sets may differ only in positions whose oracle score lies within
    `tol` (relative) of the oracle's threshold: the smallest kept unprotected
    score of that (layer, head, sequence).  Returns (ok, n_differing)."""
    L, H, _ = idx_gpu.shape
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    ko = np.concatenate([[0], np.cumsum(kept)])
    ndiff = 0
    for l in range(L):
        for h in range(H):
            for b, N in enumerate(seqlens):
                g = idx_gpu[l, h, ko[b]:ko[b + 1]]
                o = idx_orc[l, h, ko[b]:ko[b + 1]]
                if np.array_equal(g, o):
                    continue
                zb = z_orc[l, h, cu[b]:cu[b + 1]].astype(np.float64)
                pos = np.arange(N)
                prot = (pos < n_sink) | (pos >= N - n_recent)
                kept_unprot = np.setdiff1d(o, pos[prot])
                if kept_unprot.size == 0:
                    return False, ndiff
                tau = zb[kept_unprot].min()
                diff = np.setxor1d(g, o)
                ndiff += diff.size
                if np.any(prot[diff]):
                    return False, ndiff
                if np.any(np.abs(zb[diff] - tau) > tol * abs(tau)):
                    return False, ndiff
                # the GPU set must still be a valid kept set
                if g.size != o.size or np.any(np.diff(g) <= 0) or not set(pos[prot]) <= set(g.tolist()):
                    return False, ndiff
    return True, ndiff
