"""Pins for the oracle's base score (accumulated attention mass over an
observation window) and head statistics.

Every expectation here comes from somewhere other than the oracle's own code:
closed forms, a library softmax on special cases, and metamorphic relations.
Sources: H2O breakdown page, "Observation 2" (a token's score is the attention
probability it receives summed over query positions) and "Problem
formalization" (softmax rows are normalised); KV-cache survey page, section 1.1
(decode attention softmax(q K^T / sqrt(d_head))) and section 3.3 (GQA groups).
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_rows_sum_to_one(causal, Hq, Hkv):
    # every softmax row sums to 1, so a KV head's scores sum to G*W per sequence
    seqlens = [37, 64]
    W, d = 5, 16
    T = sum(seqlens)
    q = _rand((2, Hq, len(seqlens) * W, d), 1)
    k = _rand((2, Hkv, T, d), 2)
    s, st = oracle.score(q, k, seqlens, W, 1 / math.sqrt(d), causal)
    G = Hq // Hkv
    cu = np.cumsum([0] + seqlens)
    for b in range(len(seqlens)):
        tot = s[:, :, cu[b]:cu[b + 1]].astype(np.float64).sum(-1)
        np.testing.assert_allclose(tot, G * W, rtol=1e-6)
        np.testing.assert_allclose(st[:, b, :, 0], G * W, rtol=1e-6)
    assert (s >= 0).all()


def test_single_query_is_library_softmax():
    # W = 1, one head per group: the score is the softmax row itself
    N, d = 300, 32
    q = _rand((1, 3, 1, d), 3)
    k = _rand((1, 3, N, d), 4)
    sc = 0.37
    s, _ = oracle.score(q, k, [N], 1, sc, causal=True)
    for h in range(3):
        ref = softmax(sc * (k[0, h].astype(np.float64) @ q[0, h, 0].astype(np.float64)))
        np.testing.assert_allclose(s[0, h], ref, rtol=1e-6, atol=1e-12)


def test_gqa_contiguous_group_mapping():
    # query head h uses KV head h // G; scores add over the group
    N, d, Hq, Hkv = 200, 16, 6, 2
    G = Hq // Hkv
    q = _rand((1, Hq, 1, d), 5)
    k = _rand((1, Hkv, N, d), 6)
    s, _ = oracle.score(q, k, [N], 1, 0.25, causal=False)
    for g in range(Hkv):
        ref = sum(softmax(0.25 * (k[0, g].astype(np.float64) @ q[0, h, 0].astype(np.float64)))
                  for h in range(g * G, (g + 1) * G))
        np.testing.assert_allclose(s[0, g], ref, rtol=1e-6, atol=1e-12)


def test_causal_two_rows_library_softmax():
    # W = 2: the first window row sees N-1 keys, the second sees all N
    N, d = 150, 24
    q = _rand((1, 1, 2, d), 7)
    k = _rand((1, 1, N, d), 8)
    sc = 1 / math.sqrt(d)
    s, _ = oracle.score(q, k, [N], 2, sc, causal=True)
    K = k[0, 0].astype(np.float64)
    r0 = np.zeros(N)
    r0[:N - 1] = softmax(sc * (K[:N - 1] @ q[0, 0, 0].astype(np.float64)))
    r1 = softmax(sc * (K @ q[0, 0, 1].astype(np.float64)))
    np.testing.assert_allclose(s[0, 0], r0 + r1, rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("G", [1, 3])
def test_identical_keys_causal_closed_form(G):
    # all keys equal -> each window row is uniform over the keys it sees:
    # s_i = G * sum_{w : N-W+w >= i} 1 / (N-W+w+1)
    N, W, d = 40, 7, 8
    kv = _rand((d,), 9)
    k = np.broadcast_to(kv, (1, 1, N, d)).copy()
    q = _rand((1, G, W, d), 10)
    s, _ = oracle.score(q, k, [N], W, 0.5, causal=True)
    ref = np.zeros(N)
    for w in range(W):
        p = N - W + w
        ref[:p + 1] += G / (p + 1)
    np.testing.assert_allclose(s[0, 0], ref, rtol=1e-6)


def test_identical_keys_noncausal_uniform():
    N, W, d = 33, 4, 8
    k = np.ones((1, 2, N, d), np.float32)
    q = _rand((1, 2, W, d), 11)
    s, st = oracle.score(q, k, [N], W, 0.3, causal=False)
    np.testing.assert_allclose(s, W / N, rtol=1e-6)
    # head statistics of a uniform head: sum s ln s = S ln(S / N)
    S = float(W)
    np.testing.assert_allclose(st[0, 0, :, 1], S * math.log(S / N), rtol=1e-7)  # s is fp32


def test_scale_zero_is_uniform_over_visible():
    N, W, d = 25, 3, 8
    q = _rand((1, 1, W, d), 12)
    k = _rand((1, 1, N, d), 13)
    s, _ = oracle.score(q, k, [N], W, 0.0, causal=True)
    ref = np.zeros(N)
    for w in range(W):
        p = N - W + w
        ref[:p + 1] += 1.0 / (p + 1)
    np.testing.assert_allclose(s[0, 0], ref, rtol=1e-6)


def test_large_logits_are_stable():
    # a key aligned with every query at a huge logit takes all the mass; no
    # overflow (max subtraction) and the result stays finite
    N, W, d = 64, 4, 16
    q = np.zeros((1, 1, W, d), np.float32)
    q[..., 0] = 50.0
    k = _rand((1, 1, N, d), 14, 0.01)
    k[0, 0, 10, 0] = 40.0  # logit 2000 at scale 1
    s, st = oracle.score(q, k, [N], W, 1.0, causal=True)
    assert np.isfinite(s).all() and np.isfinite(st).all()
    assert abs(s[0, 0, 10] - W) < 1e-6
    # one-hot head: sum s ln s = W ln W
    assert abs(st[0, 0, 0, 1] - W * math.log(W)) < 1e-4


def test_ragged_batch_equals_separate_sequences():
    seqlens = [20, 57, 33]
    W, d, Hq, Hkv = 6, 8, 4, 2
    T = sum(seqlens)
    q = _rand((1, Hq, len(seqlens) * W, d), 15)
    k = _rand((1, Hkv, T, d), 16)
    s, st = oracle.score(q, k, seqlens, W, 0.35, causal=True)
    cu = np.cumsum([0] + seqlens)
    for b, n in enumerate(seqlens):
        sb, stb = oracle.score(np.ascontiguousarray(q[:, :, b * W:(b + 1) * W]),
                               np.ascontiguousarray(k[:, :, cu[b]:cu[b + 1]]), [n], W, 0.35, True)
        np.testing.assert_array_equal(s[:, :, cu[b]:cu[b + 1]], sb)
        np.testing.assert_array_equal(st[:, b], stb[:, 0])


def test_layers_are_independent():
    W, d = 3, 8
    q = _rand((3, 2, W, d), 17)
    k = _rand((3, 2, 30, d), 18)
    s, _ = oracle.score(q, k, [30], W, 0.4, True)
    for l in range(3):
        sl, _ = oracle.score(q[l:l + 1], k[l:l + 1], [30], W, 0.4, True)
        np.testing.assert_array_equal(s[l], sl[0])


def test_head_stats_matches_scores():
    seqlens = [50, 70]
    q = _rand((1, 2, 2 * 4, 8), 19)
    k = _rand((1, 2, 120, 8), 20)
    s, st = oracle.score(q, k, seqlens, 4, 0.5, True)
    st2 = oracle.head_stats(s, seqlens)
    np.testing.assert_array_equal(st, st2)


def test_rejects_bad_shapes():
    q = _rand((1, 3, 4, 8), 21)
    k = _rand((1, 2, 10, 8), 22)
    with pytest.raises(ValueError):
        oracle.score(q, k, [10], 4, 0.5, True)  # Hq % Hkv != 0
    q = _rand((1, 2, 4, 8), 21)
    with pytest.raises(ValueError):
        oracle.score(q, k, [3], 4, 0.5, True)  # W > N
