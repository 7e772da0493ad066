"""Pins for the oracle's layer-wide budget allocation (orc_select_layer) and
the compaction of its output.

Sources: NestedKV summary page, head-wise memory allocation (the layer's
budget goes to the globally highest (token, head) pairs, with a per-head
safety minimum); KV-cache survey page, section 4.4 (PyramidKV sets budgets
per layer); HubKV walkthrough page, head calibration (head weights make scores
comparable across heads) and "Modular vs. Submodular" (the kept set maximises
the modular sum of scores).
"""
import itertools

import numpy as np
import pytest

import oracle
import synthetic as S


def _prot(N, n_sink, n_recent):
    pos = np.arange(N)
    return (pos < n_sink) | (pos >= N - n_recent)


def _lexsort_global(zs, N, n_sink, n_recent, R):
    """Library reference for floor 0: the R best non-protected (head, pos)
    pairs of one (layer, sequence) under (z desc, head asc, pos asc), NaN last."""
    H = zs.shape[0]
    prot = _prot(N, n_sink, n_recent)
    hh, pp = np.meshgrid(np.arange(H), np.arange(N), indexing="ij")
    m = ~prot[pp]
    zc = zs[m].astype(np.float64)
    key = np.where(np.isnan(zc), np.inf, -zc)
    order = np.lexsort((pp[m], hh[m], key))
    keep = np.zeros((H, N), bool)
    keep[:, prot] = True
    keep[hh[m][order[:R]], pp[m][order[:R]]] = True
    return keep


def _split(idx, hk, seqlens):
    """idx / head_kept -> keep masks [L][B][Hkv][N_b]."""
    L, B, H = hk.shape
    out, o = [], 0
    for l in range(L):
        row = []
        for b in range(B):
            heads = []
            for h in range(H):
                n = int(hk[l, b, h])
                pos = idx[o:o + n]
                o += n
                assert np.all(np.diff(pos) > 0), "positions ascending"
                m = np.zeros(seqlens[b], bool)
                m[pos] = True
                heads.append(m)
            row.append(heads)
        out.append(row)
    assert o == idx.size
    return out


@pytest.mark.parametrize("seed", range(3))
def test_floor_zero_is_global_lexsort(seed):
    seqlens = [700, 313]
    L, Hkv, ns, nr = 2, 4, 3, 16
    z = S.random_scores(seqlens, L, Hkv, seed=seed, ties=(seed == 1))
    lk = np.array([[int(0.15 * n * Hkv) for n in seqlens] for _ in range(L)])
    idx, hk = oracle.select_layer(z, seqlens, lk, ns, nr, 0)
    masks = _split(idx, hk, seqlens)
    cu = np.cumsum([0] + seqlens)
    for l in range(L):
        for b, n in enumerate(seqlens):
            P = _prot(n, ns, nr).sum()
            ref = _lexsort_global(z[l, :, cu[b]:cu[b + 1]], n, ns, nr, lk[l, b] - Hkv * P)
            np.testing.assert_array_equal(np.array(masks[l][b]), ref)


def _head_lexsort(zh, N, k, n_sink, n_recent):
    prot = _prot(N, n_sink, n_recent)
    pos = np.arange(N)
    cand = pos[~prot]
    zc = zh[cand].astype(np.float64)
    order = np.lexsort((cand, np.where(np.isnan(zc), np.inf, -zc)))
    m = prot.copy()
    m[cand[order[:k - prot.sum()]]] = True
    return m


def test_floor_at_the_even_share_is_per_head_topk():
    # a floor equal to each head's even share leaves nothing to compete for:
    # every head keeps its own Top-K (the library reference per head)
    seqlens = [900]
    Hkv, ns, nr = 5, 4, 32
    z = S.random_scores(seqlens, 1, Hkv, seed=7)
    k = 150
    P = int(_prot(900, ns, nr).sum())
    idx, hk = oracle.select_layer(z, seqlens, [[Hkv * k]], ns, nr, k - P)
    assert (hk == k).all()
    masks = _split(idx, hk, seqlens)
    for h in range(Hkv):
        np.testing.assert_array_equal(masks[0][0][h], _head_lexsort(z[0, h], 900, k, ns, nr))


def test_brute_force_maximises_the_sum_under_floors():
    # distinct scores: the kept set is the unique maximiser of the modular sum
    # among sets with each head at or above |P| + floor and the given total
    rng = np.random.default_rng(5)
    N, H, ns, nr = 7, 3, 1, 1
    prot = _prot(N, ns, nr)
    cands = [(h, p) for h in range(H) for p in range(N) if not prot[p]]
    for trial in range(30):
        z = rng.permutation(H * N).astype(np.float32).reshape(1, H, N) / 7.0
        fl = int(rng.integers(0, 3))
        P = int(prot.sum())
        total = int(rng.integers(H * (P + fl), H * N + 1))
        idx, hk = oracle.select_layer(z, [N], [[total]], ns, nr, fl)
        got = np.array(_split(idx, hk, [N])[0][0])
        R = total - H * P
        best, best_set = -np.inf, None
        for sub in itertools.combinations(range(len(cands)), R):
            per = np.zeros(H, int)
            for i in sub:
                per[cands[i][0]] += 1
            if (per < fl).any():
                continue
            v = sum(float(z[0, cands[i][0], cands[i][1]]) for i in sub)
            if v > best:
                best, best_set = v, sub
        ref = np.zeros((H, N), bool)
        ref[:, prot] = True
        for i in best_set:
            ref[cands[i]] = True
        np.testing.assert_array_equal(got, ref)


def test_invariants_and_monotone_budget():
    seqlens = [1200, 64, 500]
    L, Hkv, ns, nr, fl = 1, 6, 4, 32, 10
    z = S.random_scores(seqlens, L, Hkv, seed=11)
    cu = np.cumsum([0] + seqlens)
    prev = None
    for frac in (0.1, 0.2, 0.35, 0.6):
        lk = []
        for n in seqlens:
            P = int(_prot(n, ns, nr).sum())
            f = min(fl, n - P)
            lk.append(max(Hkv * (P + f), int(frac * n * Hkv)))
        idx, hk = oracle.select_layer(z, seqlens, [lk], ns, nr, fl)
        masks = _split(idx, hk, seqlens)
        for b, n in enumerate(seqlens):
            P = int(_prot(n, ns, nr).sum())
            f = min(fl, n - P)
            assert hk[0, b].sum() == lk[b]
            assert (hk[0, b] >= P + f).all()
            for h in range(Hkv):
                m = masks[0][b][h]
                assert m[_prot(n, ns, nr)].all()
                # each head keeps a prefix of its own order: its own Top-k_h
                np.testing.assert_array_equal(
                    m, _head_lexsort(z[0, h, cu[b]:cu[b + 1]], n, int(hk[0, b, h]), ns, nr))
        if prev is not None:
            for b in range(len(seqlens)):
                for h in range(Hkv):
                    assert not (prev[0][b][h] & ~masks[0][b][h]).any(), "a larger budget drops nothing"
        prev = masks


def test_specials_nan_lowest_signed_zero_equal():
    z = np.array([[[np.nan, 0.0, -0.0, 1.0, np.inf, -np.inf, np.nan, 2.0],
                   [-0.0, np.nan, 3.0, 0.0, -1.0, np.nan, 0.5, 0.0]]], np.float32)
    idx, hk = oracle.select_layer(z, [8], [[10]], 0, 0, 1)
    masks = np.array(_split(idx, hk, [8])[0][0])
    ref = _lexsort_global(np.where(np.isnan(z[0]), np.nan, z[0]), 8, 0, 0, 10)
    # floor 1: head 0's best (+inf at 4) and head 1's (3.0 at 2) are in
    # anyway; the rest is the global order with -0 == +0 and NaN last
    np.testing.assert_array_equal(masks, ref)
    assert not masks[0, 0] and not masks[0, 6] and not masks[1, 1] and not masks[1, 5]


def test_rejects_budget_below_floors():
    z = S.random_scores([100], 1, 3, seed=2)
    P = 4 + 8
    with pytest.raises(ValueError):
        oracle.select_layer(z, [100], [[3 * (P + 5) - 1]], 4, 8, 5)
    with pytest.raises(ValueError):
        oracle.select_layer(z, [100], [[301]], 4, 8, 5)
    oracle.select_layer(z, [100], [[3 * (P + 5)]], 4, 8, 5)


def test_compact_layer_gathers_each_heads_rows():
    seqlens = [40, 25]
    L, Hkv, d = 2, 3, 8
    rng = np.random.default_rng(1)
    T = sum(seqlens)
    K = rng.standard_normal((L, Hkv, T, d)).astype(np.float32)
    V = rng.standard_normal((L, Hkv, T, d)).astype(np.float32)
    z = S.random_scores(seqlens, L, Hkv, seed=3)
    lk = [[30, 24], [45, 21]]
    idx, hk = oracle.select_layer(z, seqlens, lk, 2, 4, 1)
    ko, vo = oracle.compact_layer(K, V, idx, hk, seqlens)
    cu = np.cumsum([0] + seqlens)
    o = 0
    for l in range(L):
        for b in range(2):
            for h in range(Hkv):
                for _ in range(hk[l, b, h]):
                    np.testing.assert_array_equal(ko[o], K[l, h, cu[b] + idx[o]])
                    np.testing.assert_array_equal(vo[o], V[l, h, cu[b] + idx[o]])
                    o += 1
    assert o == ko.shape[0] == sum(map(sum, lk))
