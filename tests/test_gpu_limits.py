"""GPU parity at the boundary's largest batch: 64 sequences (the most one call
takes), through every entry point, against the CPU oracle.

* prefill: a bf16 score of 64 ragged sequences (lengths from the window up
  to 3000, tile edges included) within the score bar; refine, select and
  compaction bit-exact given the oracle's scores;
* the layer-wide budget at its limit of 256 (layer, sequence) pairs
  (4 layers x 64 sequences), bit-exact;
* one decode step over 64 sequences from a drawn mid-stream cache, with the
  same bars as the other decode tests.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic as S
from gpu_helpers import note, rel_err, threads, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import token_scoring_top_amd as hk  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hk.lib()
    oracle.set_threads(threads())


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _lengths(rng, lo, n=64):
    edges = [lo, 63, 64, 65, 1023, 1024, 1025, 2048]
    out = [int(x) for x in rng.integers(lo, 3001, n)]
    out[:len(edges)] = [max(lo, e) for e in edges]
    return out


def test_prefill_ops_at_64_sequences():
    rng = np.random.default_rng(64)
    W, d, Hkv, G, L = 16, 128, 2, 2, 1
    seqlens = _lengths(rng, W)
    T, Hq = sum(seqlens), G * Hkv
    Q = S.round_bf16(rng.standard_normal((L, Hq, len(seqlens) * W, d), dtype=np.float32))
    K = S.round_bf16(rng.standard_normal((L, Hkv, T, d), dtype=np.float32))
    V = S.round_bf16(rng.standard_normal((L, Hkv, T, d), dtype=np.float32))
    scale = 1 / math.sqrt(d)
    note(f"  64 sequences, T={T}")
    s_o, st_o = oracle.score(Q, K, seqlens, W, scale, True)
    s_g, st_g = hk.hubkv_score(to_dev(Q, "bf16"), to_dev(K, "bf16"), seqlens, W, scale, True)
    torch.cuda.synchronize()
    assert rel_err(s_g.cpu().numpy(), s_o, 1e-30).max() < 5e-5
    np.testing.assert_allclose(st_g.cpu().numpy()[..., 0], st_o[..., 0], rtol=1e-5)
    # refine, select and compaction from the oracle's scores: bit-exact
    ns, nr = 4, 16
    kept = np.array([int(rng.integers(oracle.protected_count(n, ns, nr), n + 1))
                     for n in seqlens], dtype=np.int64)
    beta = oracle.beta(oracle.head_stats(s_o, seqlens), seqlens)
    z_o = oracle.refine(s_o, seqlens, beta, 5, 0.5, 0.1)
    idx_o = oracle.select(z_o, seqlens, kept, ns, nr)
    z_g, _ = hk.hubkv_refine(to_dev(s_o, "f32"), seqlens, beta_in=to_dev(beta, "f32"), r=0.1)
    idx_g = hk.hubkv_select(z_g, seqlens, kept, ns, nr)
    ko, vo = hk.hubkv_compact(to_dev(K, "bf16"), to_dev(V, "bf16"), idx_g, seqlens, kept)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z_g.cpu().numpy(), z_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    ko_o, vo_o = oracle.compact(K, V, idx_o, seqlens, kept)
    np.testing.assert_array_equal(to_host(ko), ko_o)
    np.testing.assert_array_equal(to_host(vo), vo_o)


def test_select_layer_at_256_pairs():
    rng = np.random.default_rng(256)
    L, Hkv, ns, nr, floor = 4, 3, 2, 8, 16
    seqlens = _lengths(rng, 1)
    lk = []
    for _ in range(L):
        row = []
        for n in seqlens:
            P = oracle.protected_count(n, ns, nr)
            f = min(floor, n - P)
            row.append(int(rng.integers(Hkv * (P + f), Hkv * n + 1)))
        lk.append(row)
    z = S.random_scores(seqlens, L, Hkv, seed=5, kind="attention", ties=True)
    note(f"  {L} layers x 64 sequences, T={sum(seqlens)}")
    idx_g, hk_g = hk.hubkv_select_layer(to_dev(z, "f32"), seqlens, lk, ns, nr, floor)
    torch.cuda.synchronize()
    idx_o, hk_o = oracle.select_layer(z, seqlens, lk, ns, nr, floor)
    np.testing.assert_array_equal(hk_g.cpu().numpy(), hk_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)


def test_decode_step_at_64_sequences():
    w = S.workload(4).with_(B=64, Hkv=2, Hq=4, d=128, heavy=200, recent=56, dtype="bf16",
                            n_sink=4)
    t = 3 * w.C
    st = S.decode_random_state(w, t=t, seed=9, fill=w.C)
    ds = {"K": to_dev(st["K"], "bf16"), "V": to_dev(st["V"], "bf16"),
          "acc": torch.from_numpy(st["acc"].copy()).cuda(),
          "pos": torch.from_numpy(st["pos"].copy()).cuda()}
    probs = torch.full((w.B, w.Hq, w.C + 1), float("nan"), device="cuda")
    ev_g = hk.h2o_step(to_dev(st["q"], "bf16"), to_dev(st["k_new"], "bf16"),
                       to_dev(st["v_new"], "bf16"), ds["K"], ds["V"], ds["acc"], ds["pos"], t,
                       w.scale, w.n_sink, w.recent, 0, probs=probs)
    torch.cuda.synchronize()
    st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
    ev_o, pr_o, mg = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale,
                                     w.n_sink, w.recent, 0, want_probs=True, want_margin=True)
    np.testing.assert_allclose(probs.cpu().numpy(), pr_o, rtol=2e-2, atol=1e-7)
    ev_g = ev_g.cpu().numpy()
    same = ev_g == ev_o
    assert np.all(same | (mg <= 1e-4))
    pos_g = ds["pos"].cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hkv):
            if same[b, h]:
                np.testing.assert_array_equal(pos_g[b, h], st_o["pos"][b, h])
