"""Pins for the oracle's head calibration (beta) and HubKV refinement.

Sources: HubKV walkthrough page, "Method" (four steps: width-5 max-pool hubs,
SMD discount of non-hubs by 0.5, selectivity head weight clipped to
[0.8, 1.2], ratio gate z = s + r^2 (beta q - s)) and "Local theoretical
guarantees" (Local Hub Dominance: a hub outranks its discounted neighbours;
Bounded Perturbation: the gate and the clipped weight bound the change).
"""
import math

import numpy as np
import pytest
from numpy.lib.stride_tricks import sliding_window_view
from scipy.stats import entropy

import oracle
import synthetic as S


def _stats_of(s_heads, N):
    s = np.asarray(s_heads, np.float32)[None]  # [1][Hkv][N]
    return oracle.head_stats(s, [N])


# ---------------------------------------------------------------- beta -----
def test_beta_uniform_vs_one_hot_heads():
    # selectivity 0 (uniform) and 1 (one-hot): mean 0.5 -> ratios 0 and 2,
    # clipped to the page's [0.8, 1.2]
    N = 64
    uni = np.full(N, 0.5, np.float32)
    hot = np.zeros(N, np.float32)
    hot[3] = 32.0
    bt = oracle.beta(_stats_of([uni, hot], N), [N])
    np.testing.assert_allclose(bt[0, 0], [0.8, 1.2], rtol=0, atol=1e-7)


def test_beta_identical_heads_is_one():
    N = 100
    s = np.random.default_rng(1).random(N).astype(np.float32)
    bt = oracle.beta(_stats_of([s, s, s], N), [N])
    np.testing.assert_allclose(bt, 1.0, atol=1e-7)


def test_beta_from_library_entropy():
    # selectivity = 1 - H(s / sum s) / ln N with H the Shannon entropy; pick
    # heads whose ratios to the mean stay inside the clip range
    rng = np.random.default_rng(2)
    N = 512
    heads = [rng.pareto(a, N).astype(np.float32) + 0.05 for a in (2.0, 2.2, 2.5, 3.0)]
    sel = np.array([1 - entropy(h.astype(np.float64)) / math.log(N) for h in heads])
    ref = sel / sel.mean()
    assert (ref > 0.8).all() and (ref < 1.2).all()
    bt = oracle.beta(_stats_of(heads, N), [N])
    np.testing.assert_allclose(bt[0, 0], ref, rtol=2e-6)


def test_beta_permutation_equivariant_and_clipped():
    rng = np.random.default_rng(3)
    N = 256
    heads = [rng.pareto(a, N).astype(np.float32) for a in (0.7, 1.0, 2.0, 5.0, 9.0)]
    st = _stats_of(heads, N)
    bt = oracle.beta(st, [N])
    perm = rng.permutation(len(heads))
    bt2 = oracle.beta(np.ascontiguousarray(st[:, :, perm]), [N])
    np.testing.assert_array_equal(bt2[0, 0], bt[0, 0, perm])
    assert (bt >= np.float32(0.8)).all() and (bt <= np.float32(1.2)).all()


def test_beta_all_flat_heads_is_one():
    N = 32
    bt = oracle.beta(_stats_of([np.ones(N, np.float32)] * 4, N), [N])
    np.testing.assert_array_equal(bt, 1.0)


# -------------------------------------------------------------- refine -----
def _hub_mask_library(s, pool):
    h = pool // 2
    p = np.pad(s.astype(np.float64), h, constant_values=-np.inf)
    return sliding_window_view(p, pool).max(axis=1) == s


@pytest.mark.parametrize("pool", [1, 3, 5, 7])
def test_hub_mask_matches_library_max_pool(pool):
    # r = 1, beta = 1: z = q, the SMD-discounted score, so hubs are exactly
    # where z == s (scores > 0)
    seqlens = [97, 41]
    s = S.random_scores(seqlens, 1, 2, seed=4)
    bt = np.ones((1, 2, 2), np.float32)
    z = oracle.refine(s, seqlens, bt, pool=pool, gamma=0.5, r=1.0)
    cu = np.cumsum([0] + seqlens)
    for h in range(2):
        for b in range(2):
            sb = s[0, h, cu[b]:cu[b + 1]]
            zb = z[0, h, cu[b]:cu[b + 1]]
            hub = _hub_mask_library(sb, pool)
            np.testing.assert_array_equal(zb == sb, hub)
            np.testing.assert_array_equal(zb[~hub], sb[~hub] * np.float32(0.5))


@pytest.mark.parametrize("r,bval", [(0.2, 1.13), (0.1, 0.85), (0.05, 1.2), (0.7, 0.8)])
def test_gate_closed_forms(r, bval):
    # hubs: z = s (1 + r^2 (beta - 1)); others: z = s (1 + r^2 (beta gamma - 1))
    seqlens = [400]
    s = S.random_scores(seqlens, 1, 1, seed=5)
    bt = np.full((1, 1, 1), bval, np.float32)
    z = oracle.refine(s, seqlens, bt, 5, 0.5, r).astype(np.float64)[0, 0]
    sb = s[0, 0].astype(np.float64)
    hub = _hub_mask_library(s[0, 0], 5)
    r2 = float(np.float32(r) * np.float32(r))
    b = float(np.float32(bval))
    ref = np.where(hub, sb * (1 + r2 * (b - 1)), sb * (1 + r2 * (b * 0.5 - 1)))
    np.testing.assert_allclose(z, ref, rtol=3e-7)


def test_local_hub_dominance_and_bounded_perturbation():
    # LHD: z_h >= z_i for |i - h| <= 2 around every hub, strictly when r > 0
    # and i is a non-hub with s_i > 0.  Bounded perturbation:
    # |z - s| <= r^2 max(|beta-1|, |beta gamma - 1|) s <= 0.6 r^2 s
    seqlens = [300, 211]
    s = S.random_scores(seqlens, 2, 3, seed=6)
    for r in (0.05, 0.1, 0.2, 0.5, 1.0):
        for bval in (0.8, 0.95, 1.2):
            bt = np.full((2, 2, 3), bval, np.float32)
            z = oracle.refine(s, seqlens, bt, 5, 0.5, r)
            cu = np.cumsum([0] + seqlens)
            for l in range(2):
                for h in range(3):
                    for b in range(2):
                        sb = s[l, h, cu[b]:cu[b + 1]]
                        zb = z[l, h, cu[b]:cu[b + 1]]
                        hub = _hub_mask_library(sb, 5)
                        n = sb.size
                        for c in np.nonzero(hub)[0]:
                            for i in range(max(0, c - 2), min(n, c + 3)):
                                assert zb[c] >= zb[i]
                                if not hub[i] and sb[i] > 0:
                                    assert zb[c] > zb[i]
                        bound = (r * r) * max(abs(bval - 1), abs(bval * 0.5 - 1)) * sb.astype(np.float64)
                        dev = np.abs(zb.astype(np.float64) - sb)
                        # z is an fp32 result: allow two ulps of s for its rounding
                        ulp = 2 * np.spacing(sb).astype(np.float64)
                        assert (dev <= bound * (1 + 1e-6) + ulp).all()
                        assert (dev <= 0.6 * r * r * sb * (1 + 1e-6) + ulp).all()


def test_special_cases_exact():
    seqlens = [128]
    s = S.random_scores(seqlens, 1, 2, seed=7)
    bt = np.array([[[1.1, 0.9]]], np.float32)
    # r = 0: no correction at all
    np.testing.assert_array_equal(oracle.refine(s, seqlens, bt, 5, 0.5, 0.0), s)
    # gamma = 1 and beta = 1: nothing to correct towards
    np.testing.assert_array_equal(
        oracle.refine(s, seqlens, np.ones_like(bt), 5, 1.0, 0.3), s)


def test_constant_scores_are_all_hubs():
    s = np.full((1, 1, 50), 0.25, np.float32)
    z = oracle.refine(s, [50], np.full((1, 1, 1), 1.2, np.float32), 5, 0.5, 0.5)
    np.testing.assert_allclose(z, 0.25 * (1 + 0.25 * 0.2), rtol=1e-7)


def test_strict_ramp_has_one_hub_at_the_top():
    s = np.arange(1, 41, dtype=np.float32)[None, None] / np.float32(8)
    z = oracle.refine(s, [40], np.ones((1, 1, 1), np.float32), 5, 0.5, 1.0)
    assert z[0, 0, -1] == s[0, 0, -1]
    np.testing.assert_array_equal(z[0, 0, :-1], s[0, 0, :-1] * np.float32(0.5))


def test_windows_stop_at_sequence_boundaries():
    # the last token of sequence 0 is its local max even though sequence 1
    # starts with larger values right after it in the packed layout
    s = np.array([[[0.1, 0.2, 0.3, 0.4, 5.0, 6.0, 0.1, 0.1]]], np.float32)
    z = oracle.refine(s, [4, 4], np.ones((1, 2, 1), np.float32), 5, 0.5, 1.0)
    assert z[0, 0, 3] == s[0, 0, 3]      # hub of sequence 0
    assert z[0, 0, 4] == s[0, 0, 4] * 0.5  # 5.0 is within 1 of 6.0 in sequence 1
    assert z[0, 0, 5] == s[0, 0, 5]


def test_rejects_even_pool():
    s = np.ones((1, 1, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.refine(s, [8], np.ones((1, 1, 1), np.float32), 4, 0.5, 0.1)
