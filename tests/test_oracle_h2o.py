"""Pins for the oracle's H2O streaming eviction step.

Sources: H2O breakdown page, "Problem formalization" (the kept set has a fixed
size and changes by at most one token per step; evicted tokens leave the
softmax normaliser), "greedy eviction" with its Algorithm 1 description (the
query's softmax over the cache is added to accumulated scores, the new token
enters with score 0, the lowest accumulated score is evicted, which maximises
the remaining set's total score), the heavy + recent section (a new token
would be evicted at once without a protected recent window) and the FlexGen
section (fixed slots; the evicted slot is overwritten in place).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthetic as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run(q, k, v, C, scale, n_sink=0, n_recent=0, include_self=0, hook=None):
    """Drive the oracle's step over a stream: q [steps][B][Hq][d], k/v [steps][B][Hkv][d]."""
    steps, B, Hq, d = q.shape
    Hkv = k.shape[2]
    st = oracle.empty_state(B, Hkv, C, d)
    evs = []
    for t in range(steps):
        before = {kk: vv.copy() for kk, vv in st.items()}
        ev, pr, mg = oracle.h2o_step(st, q[t], k[t], v[t], t, scale, n_sink, n_recent,
                                     include_self, want_probs=True, want_margin=True)
        evs.append(ev.copy())
        if hook:
            hook(t, before, st, ev, pr)
    return st, np.array(evs)


def _stream(steps, B, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((steps, B, Hq, d)).astype(np.float32)
    k = rng.standard_normal((steps, B, Hkv, d)).astype(np.float32)
    v = rng.standard_normal((steps, B, Hkv, d)).astype(np.float32)
    return q, k, v


def test_literal_algorithm1_budget3_keeps_first_three():
    # With no recent window and the new token entering at score 0 after the
    # softmax over the old cache, every later token is evicted at once.
    gold = json.load(open(os.path.join(GOLD, "h2o_alg1_budget3_literal.json")))
    w = S.H2O_TINY
    for seed in range(20):
        q, k, v = _stream(gold["N"], 1, w.Hq, w.Hkv, w.d, seed)
        st, evs = _run(q, k, v, gold["budget"], w.scale)
        for h in range(w.Hkv):
            assert sorted(st["pos"][0, h].tolist()) == gold["final_set"]
        # from step 3 on, the evicted token is the newcomer
        assert (evs[3:, 0, :] == np.arange(3, gold["N"])[:, None]).all()


@pytest.mark.parametrize("variant", [dict(include_self=1, n_recent=0),
                                     dict(include_self=0, n_recent=1),
                                     dict(include_self=1, n_recent=1, n_sink=1)])
def test_budget3_variants_brute_force_each_step(variant):
    # every eviction maximises the accumulated score of the remaining set
    # among all candidate removals (ties: the oldest token goes)
    w = S.H2O_TINY
    C = 3
    ns, nr = variant.get("n_sink", 0), variant["n_recent"]
    for seed in range(10):
        q, k, v = _stream(12, 1, w.Hq, w.Hkv, w.d, 50 + seed)

        def hook(t, before, st, ev, pr):
            for h in range(w.Hkv):
                old = {int(p): float(a) for p, a in zip(before["pos"][0, h], before["acc"][0, h]) if p >= 0}
                new_acc = {int(p): float(a) for p, a in zip(st["pos"][0, h], st["acc"][0, h]) if p >= 0}
                # the kept set changes by at most one token and has min(t+1, C) members
                assert len(new_acc) == min(t + 1, C)
                assert len(set(new_acc) - set(old)) <= 1
                if len(old) < C:
                    assert ev[0, h] == -1
                    continue
                # accumulated scores after the update, before eviction
                upd = {p: float(np.float32(old[p] + sum(pr[0, hh, j] for hh in [h]
                                                          for j in range(C)
                                                          if before["pos"][0, h, j] == p)))
                       for p in old}
                upd[t] = float(pr[0, h, C]) if variant["include_self"] else 0.0
                cands = [p for p in upd if ns <= p <= t - nr]
                best = max(cands, key=lambda u: (math.fsum(upd[x] for x in cands if x != u), -u))
                assert ev[0, h] == best

        _run(q, k, v, C, w.scale, ns, nr, variant["include_self"], hook)


def test_probabilities_and_mass_bookkeeping():
    # each query head's probabilities over the cache sum to 1 (the new token
    # included when it attends to itself); total accumulated mass grows by G
    # per step minus what the evicted token carried
    B, Hq, Hkv, d, C = 2, 4, 2, 16, 9
    G = Hq // Hkv
    for inc in (0, 1):
        q, k, v = _stream(40, B, Hq, Hkv, d, 7 + inc)

        def hook(t, before, st, ev, pr):
            if t == 0 and not inc:
                assert np.allclose(pr, 0)
                return
            np.testing.assert_allclose(pr.astype(np.float64).sum(-1), 1.0, rtol=1e-6)
            for b in range(B):
                for h in range(Hkv):
                    tot_before = before["acc"][b, h][before["pos"][b, h] >= 0].astype(np.float64).sum()
                    tot_after = st["acc"][b, h][st["pos"][b, h] >= 0].astype(np.float64).sum()
                    if ev[b, h] < 0:
                        lost = 0.0
                    elif ev[b, h] == t:
                        lost = pr[b, h * G:(h + 1) * G, C].astype(np.float64).sum()
                    else:
                        j = int(np.nonzero(before["pos"][b, h] == ev[b, h])[0][0])
                        lost = float(before["acc"][b, h, j]) + pr[b, h * G:(h + 1) * G, j].astype(np.float64).sum()
                    assert abs(tot_after - (tot_before + G - lost)) < 1e-4

        _run(q, k, v, C, 0.25, 1, 2, inc, hook)


def test_step_probabilities_are_library_softmax():
    w = S.workload(4).with_(B=2, Hq=2, Hkv=2, heavy=20, recent=12, d=32)
    stt = S.decode_random_state(w, t=200, seed=3)
    stt = {kk: np.ascontiguousarray(vv) for kk, vv in stt.items()}
    state = {kk: stt[kk].copy() for kk in ("K", "V", "acc", "pos")}
    ev, pr = oracle.h2o_step(state, stt["q"], stt["k_new"], stt["v_new"], 200, w.scale, 0,
                             w.recent, 0, want_probs=True)
    for b in range(2):
        for h in range(2):
            ref = softmax(w.scale * (stt["K"][b, h].astype(np.float64) @ stt["q"][b, h].astype(np.float64)))
            np.testing.assert_allclose(pr[b, h, :w.C], ref, rtol=1e-6, atol=1e-12)


def _torch_attention(q, k, v, scale, mask):
    """torch's scaled_dot_product_attention in float64 on the CPU:
    q [H][Lq][d], k/v [H][Lk][d], mask [Lq][Lk] boolean (True = attend)."""
    import torch
    f = torch.nn.functional.scaled_dot_product_attention
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    return f(T(q)[None], T(k)[None], T(v)[None], attn_mask=torch.from_numpy(mask),
             scale=float(scale))[0].numpy()


@pytest.mark.parametrize("include_self", [0, 1])
def test_attention_output_unbounded_is_causal_attention(include_self):
    # KV-cache page, section 1.1: decode attention of token t is the softmax of
    # its scaled query against every key so far, applied to the values.  With
    # room for every token no eviction happens, so the step outputs are the
    # rows of causal attention (strictly causal without self-attention), with
    # KV head h // G serving query head h.
    N, B, Hq, Hkv, d = 40, 2, 4, 2, 16
    G = Hq // Hkv
    q, k, v = _stream(N, B, Hq, Hkv, d, 61 + include_self)
    st = oracle.empty_state(B, Hkv, N, d)
    outs = []
    for t in range(N):
        ev, o = oracle.h2o_step(st, q[t], k[t], v[t], t, 0.3, 0, 0, include_self, want_out=True)
        assert (ev == -1).all()
        outs.append(o)
    outs = np.array(outs)                                 # [N][B][Hq][d]
    mask = np.tril(np.ones((N, N), bool), 0 if include_self else -1)
    if not include_self:
        mask[0, 0] = True                                 # row 0 is checked separately below
    for b in range(B):
        Kr = np.repeat(k[:, b].transpose(1, 0, 2), G, axis=0)   # [Hq][N][d]
        Vr = np.repeat(v[:, b].transpose(1, 0, 2), G, axis=0)
        ref = _torch_attention(q[:, b].transpose(1, 0, 2), Kr, Vr, 0.3, mask)
        got = outs[:, b].transpose(1, 0, 2)
        lo = 0 if include_self else 1
        np.testing.assert_allclose(got[:, lo:], ref[:, lo:], rtol=1e-5, atol=1e-6)
    if not include_self:
        assert (outs[0] == 0).all()                       # nothing to attend to yet


def test_attention_output_over_retained_tokens():
    # H2O page, problem statement: an evicted token drops out of the keys and
    # of the normaliser.  Each step's output is attention over the tokens the
    # cache held before the step (plus the new token when it attends to
    # itself), whatever slots they sit in.
    B, Hq, Hkv, d, C = 2, 4, 2, 8, 11
    G = Hq // Hkv
    for inc in (0, 1):
        q, k, v = _stream(60, B, Hq, Hkv, d, 71 + inc)
        st = oracle.empty_state(B, Hkv, C, d)
        for t in range(60):
            before = {kk: vv.copy() for kk, vv in st.items()}
            _, o = oracle.h2o_step(st, q[t], k[t], v[t], t, 0.4, 1, 3, inc, want_out=True)
            if t == 0 and not inc:
                continue
            for b in range(B):
                for g in range(Hkv):
                    keys = np.concatenate([before["K"][b, g], k[t, b, g][None]])
                    vals = np.concatenate([before["V"][b, g], v[t, b, g][None]])
                    m = np.concatenate([before["pos"][b, g] >= 0, [bool(inc)]])[None]
                    hs = slice(g * G, (g + 1) * G)
                    ref = _torch_attention(q[t, b, hs][:, None], np.repeat(keys[None], G, 0),
                                           np.repeat(vals[None], G, 0), 0.4, m)[:, 0]
                    np.testing.assert_allclose(o[b, hs], ref, rtol=1e-5, atol=1e-6)


def test_attention_output_ignores_empty_slot_contents():
    # empty slots hold no token: their K/V rows (NaN here) never reach the output
    B, Hq, Hkv, d, C = 1, 2, 1, 8, 16
    q, k, v = _stream(6, B, Hq, Hkv, d, 81)
    clean = oracle.empty_state(B, Hkv, C, d)
    dirty = oracle.empty_state(B, Hkv, C, d)
    dirty["K"][:] = np.nan
    dirty["V"][:] = np.nan
    for t in range(6):
        _, oc = oracle.h2o_step(clean, q[t], k[t], v[t], t, 0.3, 0, 0, 1, want_out=True)
        _, od = oracle.h2o_step(dirty, q[t], k[t], v[t], t, 0.3, 0, 0, 1, want_out=True)
        np.testing.assert_array_equal(oc, od)


def test_attention_output_is_convex_combination():
    # probabilities sum to one: identical value rows come back unchanged, and a
    # value ramp over positions returns the expected position under the softmax
    B, Hq, Hkv, d, C = 1, 3, 1, 4, 9
    q, k, _ = _stream(30, B, Hq, Hkv, d, 91)
    vconst = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0], np.float32), (30, B, Hkv, d)).copy()
    st = oracle.empty_state(B, Hkv, C, d)
    for t in range(30):
        _, o = oracle.h2o_step(st, q[t], k[t], vconst[t], t, 0.5, 1, 2, 1, want_out=True)
        np.testing.assert_allclose(o[0], np.broadcast_to(vconst[0, 0, 0], (Hq, d)), rtol=1e-6)
    vramp = np.zeros((30, B, Hkv, d), np.float32)
    vramp[:, 0, 0, 0] = np.arange(30)
    st = oracle.empty_state(B, Hkv, C, d)
    for t in range(30):
        pos_before = st["pos"][0, 0].copy()
        _, pr, o = oracle.h2o_step(st, q[t], k[t], vramp[t], t, 0.5, 1, 2, 1, want_probs=True,
                                   want_out=True)
        w = np.concatenate([np.maximum(pos_before, 0), [t]]).astype(np.float64)
        np.testing.assert_allclose(o[0, :, 0], pr[0].astype(np.float64) @ w, rtol=1e-5, atol=1e-6)
        assert np.all(o[0, :, 1:] == 0)


def test_protected_windows_never_evicted():
    B, Hq, Hkv, d, C, ns, nr = 1, 2, 2, 8, 12, 3, 5
    q, k, v = _stream(80, B, Hq, Hkv, d, 21)

    def hook(t, before, st, ev, pr):
        for h in range(Hkv):
            kept = set(st["pos"][0, h].tolist())
            assert set(range(min(ns, t + 1))) <= kept
            assert set(range(max(0, t - nr + 1), t + 1)) <= kept

    _run(q, k, v, C, 0.3, ns, nr, 0, hook)


def test_unbounded_cache_with_self_equals_full_window_score():
    # with room for every token and self-attention, H2O's accumulated score of
    # token i is the sum over all later queries of their causal softmax at i:
    # the prefill score with the window covering the whole sequence
    N, d, Hq, Hkv = 48, 16, 4, 2
    rng = np.random.default_rng(31)
    Q = rng.standard_normal((1, Hq, N, d)).astype(np.float32)
    K = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    s, _ = oracle.score(Q, K, [N], N, 0.25, causal=True)
    q = np.ascontiguousarray(Q[0].transpose(1, 0, 2))[:, None]       # [N][1][Hq][d]
    kk = np.ascontiguousarray(K[0].transpose(1, 0, 2))[:, None]      # [N][1][Hkv][d]
    st, evs = _run(q, kk, kk, N, 0.25, 0, 0, include_self=1)
    assert (evs == -1).all()
    for h in range(Hkv):
        order = np.argsort(st["pos"][0, h])
        np.testing.assert_allclose(st["acc"][0, h][order], s[0, h], rtol=2e-6)


def test_resume_from_copied_state_is_identical():
    B, Hq, Hkv, d, C = 2, 2, 2, 8, 10
    q, k, v = _stream(60, B, Hq, Hkv, d, 41)
    full, _ = _run(q, k, v, C, 0.3, 1, 3, 0)
    st = oracle.empty_state(B, Hkv, C, d)
    for t in range(30):
        oracle.h2o_step(st, q[t], k[t], v[t], t, 0.3, 1, 3, 0)
    saved = {kk: vv.copy() for kk, vv in st.items()}
    st2 = {kk: vv.copy() for kk, vv in saved.items()}
    for t in range(30, 60):
        oracle.h2o_step(st2, q[t], k[t], v[t], t, 0.3, 1, 3, 0)
    for kk in full:
        np.testing.assert_array_equal(full[kk], st2[kk])


def test_slot_overwrite_keeps_kv_with_position():
    # the slot of an evicted token takes the new token's K and V rows
    B, Hq, Hkv, d, C = 1, 1, 1, 4, 5
    q, k, v = _stream(30, B, Hq, Hkv, d, 43)
    st, _ = _run(q, k, v, C, 0.5, 0, 2, 0)
    for j in range(C):
        p = st["pos"][0, 0, j]
        np.testing.assert_array_equal(st["K"][0, 0, j], k[p, 0, 0])
        np.testing.assert_array_equal(st["V"][0, 0, j], v[p, 0, 0])


def test_eviction_tie_goes_to_oldest():
    # scale 0 makes every probability equal, so equal accumulated scores stay
    # exactly equal; the oldest candidate must be the one evicted
    B, Hq, Hkv, d, C, t = 1, 2, 1, 8, 6, 40
    rng = np.random.default_rng(5)
    for trial in range(5):
        pos = np.sort(rng.choice(np.arange(t - 2), size=C - 2, replace=False)).tolist() + [t - 2, t - 1]
        perm = rng.permutation(C)
        st = oracle.empty_state(B, Hkv, C, d)
        st["pos"][0, 0, perm] = np.array(pos, np.int32)
        st["acc"][0, 0, :] = np.float32(0.75)
        q = rng.standard_normal((B, Hq, d)).astype(np.float32)
        kn = rng.standard_normal((B, Hkv, d)).astype(np.float32)
        ev = oracle.h2o_step(st, q, kn, kn, t, 0.0, n_sink=0, n_recent=3)
        assert ev[0, 0] == min(pos)
        # the evicted slot now holds the new token with a zero score
        j = int(perm[int(np.argmin(pos))])
        assert st["pos"][0, 0, j] == t and st["acc"][0, 0, j] == 0.0


def test_rejects_capacity_below_protected_windows():
    st = oracle.empty_state(1, 1, 4, 4)
    z = np.zeros((1, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.h2o_step(st, z, z, z, 0, 1.0, 3, 2, 0)
