"""Pins for the oracle's protected Top-K selection and K/V compaction.

Sources: HubKV walkthrough page, "Modular vs. Submodular" (Top-K maximises the
modular sum of scores) and "Method" (refined scores go to Top-K pruning); H2O
breakdown page, heavy + recent section (a recent window is protected) and the
per-head section; KV-cache survey page, sections 4.1-4.2 (sink tokens and the
recent window are kept; StreamingLLM keeps only those); H2O breakdown page,
"two code bases" (real drop removes evicted K/V rows).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synthetic as S


def _lexsort_ref(z, N, k, n_sink, n_recent):
    pos = np.arange(N)
    prot = (pos < n_sink) | (pos >= N - n_recent)
    cand = pos[~prot]
    zc = z[cand].astype(np.float64)
    key = np.where(np.isnan(zc), np.inf, -zc)  # NaN last; -0 == +0 as floats
    order = np.lexsort((cand, key))
    chosen = cand[order[:k - prot.sum()]]
    return np.sort(np.concatenate([pos[prot], chosen]))


@pytest.mark.parametrize("seed", range(4))
def test_matches_library_lexsort(seed):
    seqlens = [1000, 517, 164]
    L, Hkv = 2, 3
    z = S.random_scores(seqlens, L, Hkv, seed=seed, ties=(seed % 2 == 1))
    kept = S.budgets(seqlens, 0.2)
    idx = oracle.select(z, seqlens, kept, 4, 16)
    cu = np.cumsum([0] + seqlens)
    ko = np.cumsum([0] + list(kept))
    for l in range(L):
        for h in range(Hkv):
            for b, n in enumerate(seqlens):
                ref = _lexsort_ref(z[l, h, cu[b]:cu[b + 1]], n, kept[b], 4, 16)
                np.testing.assert_array_equal(idx[l, h, ko[b]:ko[b + 1]], ref)


def _brute(z, k, n_sink, n_recent):
    # among all subsets of the unprotected positions of the right size, the
    # kept set maximises the modular sum; ties go to the lexicographically
    # smallest sorted position list
    N = z.size
    prot = [i for i in range(N) if i < n_sink or i >= N - n_recent]
    cand = [i for i in range(N) if i not in prot]
    best, best_set = None, None
    for comb in itertools.combinations(cand, k - len(prot)):
        val = math.fsum(float(z[i]) for i in comb)
        if best is None or val > best:
            best, best_set = val, comb
    return sorted(prot + list(best_set))


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(5, 13))
    n_sink = int(rng.integers(0, 3))
    n_recent = int(rng.integers(0, 3))
    P = oracle.protected_count(N, n_sink, n_recent)
    k = int(rng.integers(P, N + 1))
    if seed % 3 == 0:
        z = rng.integers(0, 4, N).astype(np.float32)  # many exact ties
    else:
        z = rng.random(N).astype(np.float32)
    idx = oracle.select(z[None, None], [N], [k], n_sink, n_recent)[0, 0]
    assert list(idx) == _brute(z, k, n_sink, n_recent)


def test_invariants():
    seqlens = [333, 1024]
    z = S.random_scores(seqlens, 1, 4, seed=9)
    for budget, ns, nr in ((0.1, 4, 64), (0.5, 0, 0), (0.07, 10, 3)):
        kept = S.budgets(seqlens, budget)
        kept = np.maximum(kept, [oracle.protected_count(n, ns, nr) for n in seqlens])
        idx = oracle.select(z, seqlens, kept, ns, nr)
        ko = np.cumsum([0] + list(kept))
        for h in range(4):
            for b, n in enumerate(seqlens):
                x = idx[0, h, ko[b]:ko[b + 1]]
                assert x.size == kept[b]
                assert (np.diff(x) > 0).all() and x[0] >= 0 and x[-1] < n
                prot = set(range(min(ns, n))) | set(range(max(0, n - nr), n))
                assert prot <= set(x.tolist())


def test_streaming_llm_and_full_budget_cases():
    N = 200
    z = S.random_scores([N], 1, 1, seed=10)
    idx = oracle.select(z, [N], [4 + 32], 4, 32)[0, 0]
    np.testing.assert_array_equal(idx, np.r_[0:4, N - 32:N])
    idx = oracle.select(z, [N], [N], 4, 32)[0, 0]
    np.testing.assert_array_equal(idx, np.arange(N))


def test_nan_lowest_signed_zero_equal_infinities():
    z = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 1.0, np.nan, -0.0], np.float32)
    idx = oracle.select(z[None, None], [8], [4], 0, 0)[0, 0]
    # order: inf(3), 1.0(5), -0.0(1) == 0.0(2) -> position order, then -0.0(7), -inf, NaNs
    np.testing.assert_array_equal(idx, [1, 2, 3, 5])
    idx = oracle.select(z[None, None], [8], [6], 0, 0)[0, 0]
    np.testing.assert_array_equal(idx, [1, 2, 3, 4, 5, 7])


def test_rejects_impossible_budgets():
    z = np.ones((1, 1, 20), np.float32)
    with pytest.raises(ValueError):
        oracle.select(z, [20], [5], 4, 4)   # fewer than the protected tokens
    with pytest.raises(ValueError):
        oracle.select(z, [20], [21], 0, 0)  # more than the sequence


@pytest.mark.parametrize("dt", [np.float32, np.uint16])
def test_compact_is_library_fancy_indexing(dt):
    seqlens = [50, 31]
    L, Hkv, d = 2, 3, 16
    T = sum(seqlens)
    rng = np.random.default_rng(11)
    if dt is np.uint16:
        k = rng.integers(0, 65535, (L, Hkv, T, d)).astype(np.uint16)
        v = rng.integers(0, 65535, (L, Hkv, T, d)).astype(np.uint16)
    else:
        k = rng.standard_normal((L, Hkv, T, d)).astype(np.float32)
        v = rng.standard_normal((L, Hkv, T, d)).astype(np.float32)
    z = S.random_scores(seqlens, L, Hkv, seed=12)
    kept = S.budgets(seqlens, 0.3)
    idx = oracle.select(z, seqlens, kept, 2, 5)
    ko, vo = oracle.compact(k, v, idx, seqlens, kept)
    cu = np.cumsum([0] + seqlens)
    kc = np.cumsum([0] + list(kept))
    for l in range(L):
        for h in range(Hkv):
            for b in range(2):
                sel = idx[l, h, kc[b]:kc[b + 1]] + cu[b]
                np.testing.assert_array_equal(ko[l, h, kc[b]:kc[b + 1]], k[l, h][sel])
                np.testing.assert_array_equal(vo[l, h, kc[b]:kc[b + 1]], v[l, h][sel])
