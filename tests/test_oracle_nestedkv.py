"""Pins for the oracle's NestedKV key-only score (orc_nestedkv).

Source: NestedKV summary page -- continuum memory state (stable: the global
mean of normalised keys; episodic: a local block mean, block about N/32;
current: a moving mean over a window of 64), cosine anomalies a = -cos(k^, mu),
head-adaptive blending (a softmax over the scales' discriminative power with a
fixed log-prior) and surprise-gated routing (the standard deviation of the
three anomalies; when high, the largest anomaly).  The reference values below
come from library routines: pandas rolling and group means, scipy's cosine
distance and softmax, numpy's population standard deviation.
"""
import numpy as np
import pandas as pd
import pytest
from scipy.spatial.distance import cosine as cos_dist
from scipy.special import softmax

import oracle


def _library_ref(k, nblocks, window, prior, theta):
    """One (layer, head, sequence) unit with library routines."""
    N, d = k.shape
    kh = k.astype(np.float64) / np.linalg.norm(k.astype(np.float64), axis=1, keepdims=True)
    df = pd.DataFrame(kh)
    mu_s = df.mean(axis=0).to_numpy()
    bs = -(-N // nblocks)
    mu_e = df.groupby(np.arange(N) // bs).transform("mean").to_numpy()
    mu_c = df.rolling(window, min_periods=1).mean().to_numpy()
    a = np.empty((N, 3))
    for i in range(N):
        a[i, 0] = -(1.0 - cos_dist(kh[i], mu_s))
        a[i, 1] = -(1.0 - cos_dist(kh[i], mu_e[i]))
        a[i, 2] = -(1.0 - cos_dist(kh[i], mu_c[i]))
    w = softmax(a.max(axis=0) - a.min(axis=0) + np.asarray(prior))
    sg = a.std(axis=1)                       # population (ddof = 0)
    s = np.where(sg > theta, a.max(axis=1), a @ w)
    return s, a, w


@pytest.mark.parametrize("N,d,nblocks,window,theta", [(300, 16, 32, 64, 0.1), (1000, 64, 32, 64, 0.05),
                                                      (257, 8, 7, 10, 0.2), (64, 128, 3, 64, 0.0)])
def test_matches_library_routines(N, d, nblocks, window, theta):
    rng = np.random.default_rng(N + d)
    k = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    # a few bursts of near-identical keys, as in the prefill workloads
    for st in rng.integers(0, N - 20, size=5):
        k[0, :, st:st + 12] = k[0, :, st:st + 1] + 0.1 * rng.standard_normal((2, 12, d))
    prior = (0.3, -0.2, 0.1)
    s, an, wt = oracle.nestedkv(k, [N], nblocks, window, prior, theta, want_parts=True)
    for h in range(2):
        rs, ra, rw = _library_ref(k[0, h], nblocks, window, prior, theta)
        np.testing.assert_allclose(an[0, h], ra, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(wt[0, 0, h], rw, rtol=1e-5)
        np.testing.assert_allclose(s[0, h], rs, rtol=1e-5, atol=1e-6)


def test_ragged_sequences_and_layers_are_independent():
    rng = np.random.default_rng(3)
    seqlens = [200, 77, 130]
    T = sum(seqlens)
    k = rng.standard_normal((2, 3, T, 8)).astype(np.float32)
    s = oracle.nestedkv(k, seqlens)
    cu = np.cumsum([0] + seqlens)
    for l in range(2):
        for h in range(3):
            for b, n in enumerate(seqlens):
                alone = oracle.nestedkv(np.ascontiguousarray(k[l:l + 1, h:h + 1, cu[b]:cu[b + 1]]), [n])
                np.testing.assert_array_equal(s[l, h, cu[b]:cu[b + 1]], alone[0, 0])


def test_one_direction_gives_closed_forms():
    # every key along one direction: every memory is that direction, every
    # anomaly is -1, no scale discriminates (equal weights) and no surprise
    rng = np.random.default_rng(1)
    v = rng.standard_normal(32).astype(np.float32)
    k = (rng.random((1, 1, 150, 1)).astype(np.float32) + 0.5) * v[None, None, None, :]
    s, an, wt = oracle.nestedkv(k, [150], want_parts=True)
    np.testing.assert_allclose(an, -1.0, atol=1e-6)
    np.testing.assert_allclose(wt, 1.0 / 3.0, rtol=1e-6)
    np.testing.assert_allclose(s, -1.0, atol=1e-6)


def test_degenerate_scales():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((1, 1, 90, 16)).astype(np.float32)
    # window 1: the current memory is the token itself
    _, an, _ = oracle.nestedkv(k, [90], window=1, want_parts=True)
    np.testing.assert_allclose(an[..., 2], -1.0, atol=1e-6)
    # blocks of one position: the episodic memory is the token itself
    _, an, _ = oracle.nestedkv(k, [90], nblocks=90, want_parts=True)
    np.testing.assert_allclose(an[..., 1], -1.0, atol=1e-6)
    # one block: episodic == stable
    _, an, _ = oracle.nestedkv(k, [90], nblocks=1, want_parts=True)
    np.testing.assert_allclose(an[..., 1], an[..., 0], atol=1e-6)


def test_scale_invariance_and_zero_keys():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 1, 120, 16)).astype(np.float32)
    c = rng.random((1, 1, 120, 1)).astype(np.float32) * 8 + 0.25
    np.testing.assert_allclose(oracle.nestedkv(k, [120]), oracle.nestedkv(k * c, [120]), atol=2e-6)
    k[0, 0, 40] = 0.0
    _, an, _ = oracle.nestedkv(k, [120], want_parts=True)
    assert (an[0, 0, 40] == 0).all()


def test_routing_thresholds_and_prior():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((1, 1, 200, 16)).astype(np.float32)
    s_hi, an, wt = oracle.nestedkv(k, [200], theta=10.0, want_parts=True)
    np.testing.assert_allclose(s_hi[0, 0], an[0, 0] @ wt[0, 0, 0], rtol=1e-5, atol=1e-6)
    s_lo = oracle.nestedkv(k, [200], theta=-1.0)
    np.testing.assert_allclose(s_lo[0, 0], an[0, 0].max(axis=1), atol=1e-7)
    # a constant added to every prior changes nothing; a dominant prior picks its scale
    np.testing.assert_array_equal(oracle.nestedkv(k, [200], log_prior=(2, 2, 2), theta=10.0), s_hi)
    s_c = oracle.nestedkv(k, [200], log_prior=(-50, -50, 0), theta=10.0)
    np.testing.assert_allclose(s_c[0, 0], an[0, 0, :, 2], atol=1e-6)
