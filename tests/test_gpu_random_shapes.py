"""Seeded sweep of random shapes and parameters through every entry point,
against the CPU oracle, through the C ABI.

Each case draws, from its own seed:
- 1 to 5 sequences of 1 to 20000 tokens, including lengths at tile edges;
- 1 to 3 layers and 1 to 8 KV heads;
- sink and recent windows from 0 to beyond the sequence;
- budgets between the protected count and the whole sequence;
- an odd pooling width from 1 to 9, gamma in (0, 1] and r in [0, 1];
- for the score: d 64 or 128, G * W up to 512, bf16 or fp32, causal or not;
- for the decode step: a drawn mid-stream cache of 2 to 500 slots, partly
  empty or full, group sizes 1 to 8, with or without the new token attending
  to itself;
- for the ring slot layout of the decode step: 2 to 100 slots, streamed from
  empty past the capacity;
- for the score and the compaction: packed, token-major or padded views of
  Q, K, V and of the compaction outputs (strided calls).

The bars are those of the dedicated tests:
- integer and bit results (refined scores, kept sets, compaction, the
  layer-wide allocation) are bit-exact given identical inputs;
- scores are within 5e-5 relative for bf16 inputs and 1e-5 for fp32;
- NestedKV anomalies are within 5e-5 absolute;
- decode: probabilities and accumulated scores within 1e-5 relative (fp32
  inputs) or 2e-2 (bf16), the attention output within 1e-5 / 1e-4 of the
  scale of its terms. The evicted slot is identical unless the oracle's two
  best candidates lie within 1e-4, and where it is identical, the slots
  (positions, K and V rows) are bit-exact;
- strided calls return the packed calls' bits; the ring layout retains the
  oracle's positions, scores and rows.
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


EDGE_LENGTHS = [1, 2, 63, 64, 65, 1023, 1024, 1025, 4095, 4096, 4097, 8192]


def _seqlens(rng, lo=1):
    B = int(rng.integers(1, 6))
    out = []
    for _ in range(B):
        if rng.random() < 0.4:
            out.append(max(lo, int(rng.choice(EDGE_LENGTHS))))
        else:
            out.append(int(rng.integers(lo, 20001)))
    return out


def _windows(rng, seqlens):
    nmax = max(seqlens)
    ns = int(rng.choice([0, 1, 4, int(rng.integers(0, nmax + 2))]))
    nr = int(rng.choice([0, 8, 64, int(rng.integers(0, nmax + 2))]))
    return ns, nr


def _view(rng, x):
    """x itself, or the same values in a token-major or padded layout (a
    non-contiguous view of x's shape with a contiguous last axis)."""
    kind = str(rng.choice(["packed", "token-major", "padded"]))
    if kind == "token-major":
        return kind, x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if kind == "padded":
        L, H, R, d = x.shape
        per = 16 // x.element_size()
        buf = torch.zeros((L, H, R + int(rng.integers(0, 40)), d + per * int(rng.integers(1, 4))),
                          dtype=x.dtype, device=x.device)
        v = buf[:, :, :R, :d]
        v.copy_(x)
        return kind, v
    return kind, x


def _kept(rng, seqlens, ns, nr):
    out = []
    for n in seqlens:
        P = oracle.protected_count(n, ns, nr)
        out.append(int(rng.integers(P, n + 1)))
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("seed", range(24))
def test_refine_select_compact(seed):
    rng = np.random.default_rng(1000 + seed)
    seqlens = _seqlens(rng)
    L, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 9))
    ns, nr = _windows(rng, seqlens)
    kept = _kept(rng, seqlens, ns, nr)
    pool = int(rng.choice([1, 3, 5, 7, 9]))
    gamma = float(rng.choice([0.5, 1.0, float(rng.uniform(0.05, 1.0))]))
    r = float(rng.choice([0.0, 0.1, 1.0, float(rng.uniform(0, 1))]))
    kind = str(rng.choice(["attention", "uniform"]))
    s = S.random_scores(seqlens, L, Hkv, seed=seed, kind=kind, ties=bool(rng.random() < 0.3))
    note(f"  seqlens={seqlens} L={L} Hkv={Hkv} sink={ns} recent={nr} pool={pool} "
         f"gamma={gamma:.3f} r={r:.3f} {kind}")
    beta = oracle.beta(oracle.head_stats(s, seqlens), seqlens)
    z_o = oracle.refine(s, seqlens, beta, pool, gamma, r)
    idx_o = oracle.select(z_o, seqlens, kept, ns, nr)
    z_g, b_g = hk.hubkv_refine(to_dev(s, "f32"), seqlens, beta_in=to_dev(beta, "f32"), pool=pool,
                               gamma=gamma, r=r)
    idx_g = hk.hubkv_select(z_g, seqlens, kept, ns, nr)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z_g.cpu().numpy(), z_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    # compaction of the kept set, d 64 bf16 rows
    d = 64
    K = S.round_bf16(rng.standard_normal((L, Hkv, sum(seqlens), d), dtype=np.float32))
    V = S.round_bf16(rng.standard_normal((L, Hkv, sum(seqlens), d), dtype=np.float32))
    Kd, Vd = to_dev(K, "bf16"), to_dev(V, "bf16")
    ko, vo = hk.hubkv_compact(Kd, Vd, idx_g, seqlens, kept)
    # the same through strided views of the inputs and of the outputs
    kk, kv = _view(rng, Kd)
    vk, vv = _view(rng, Vd)
    Kt = int(sum(kept))
    ok_, ko_s = _view(rng, torch.full((L, Hkv, Kt, d), float("nan"), dtype=torch.bfloat16,
                                      device="cuda"))
    ov_, vo_s = _view(rng, torch.full((L, Hkv, Kt, d), float("nan"), dtype=torch.bfloat16,
                                      device="cuda"))
    note(f"  compaction views: {kk} {vk} -> {ok_} {ov_}")
    hk.hubkv_compact(kv, vv, idx_g, seqlens, kept, k_out=ko_s, v_out=vo_s)
    torch.cuda.synchronize()
    ko_o, vo_o = oracle.compact(K, V, idx_o, seqlens, kept)
    np.testing.assert_array_equal(to_host(ko), ko_o)
    np.testing.assert_array_equal(to_host(vo), vo_o)
    assert torch.equal(ko_s, ko) and torch.equal(vo_s, vo)


@pytest.mark.parametrize("seed", range(20))
def test_select_layer(seed):
    rng = np.random.default_rng(2000 + seed)
    seqlens = _seqlens(rng)
    L, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 9))
    ns, nr = _windows(rng, seqlens)
    floor = int(rng.choice([0, 1, 16, int(rng.integers(0, 5000))]))
    lk = []
    for _ in range(L):
        row = []
        for n in seqlens:
            P = oracle.protected_count(n, ns, nr)
            f = min(floor, n - P)
            row.append(int(rng.integers(Hkv * (P + f), Hkv * n + 1)))
        lk.append(row)
    z = S.random_scores(seqlens, L, Hkv, seed=seed, kind=str(rng.choice(["attention", "uniform"])),
                        ties=bool(rng.random() < 0.3))
    note(f"  seqlens={seqlens} L={L} Hkv={Hkv} sink={ns} recent={nr} floor={floor}")
    idx_g, hk_g = hk.hubkv_select_layer(to_dev(z, "f32"), seqlens, lk, ns, nr, floor)
    torch.cuda.synchronize()
    idx_o, hk_o = oracle.select_layer(z, seqlens, lk, ns, nr, floor)
    np.testing.assert_array_equal(hk_g.cpu().numpy(), hk_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)


@pytest.mark.parametrize("seed", range(24))
def test_score(seed):
    rng = np.random.default_rng(3000 + seed)
    dtype = str(rng.choice(["bf16", "bf16", "f32"]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4]))
    W = int(rng.choice([8, 16, 32, 48, 64, 100, 128]))
    while G * W > 512:
        W //= 2
    seqlens = _seqlens(rng, lo=W)
    seqlens = [min(n, 12000) for n in seqlens]
    L = int(rng.integers(1, 3))
    causal = bool(rng.random() < 0.8)
    Hq = G * Hkv
    T = sum(seqlens)
    Q = rng.standard_normal((L, Hq, len(seqlens) * W, d), dtype=np.float32)
    K = rng.standard_normal((L, Hkv, T, d), dtype=np.float32) * np.float32(rng.uniform(0.5, 2.0))
    if dtype == "bf16":
        Q, K = S.round_bf16(Q), S.round_bf16(K)
    scale = 1 / math.sqrt(d)
    note(f"  {dtype} d={d} Hq={Hq} Hkv={Hkv} W={W} seqlens={seqlens} L={L} causal={causal}")
    s_o, st_o = oracle.score(Q, K, seqlens, W, scale, causal)
    Qd, Kd = to_dev(Q, dtype), to_dev(K, dtype)
    s_g, st_g = hk.hubkv_score(Qd, Kd, seqlens, W, scale, causal)
    # the same through strided views: identical bits
    qk, qv = _view(rng, Qd)
    kk, kv = _view(rng, Kd)
    note(f"  views: q {qk}, k {kk}")
    s_v, st_v = hk.hubkv_score(qv, kv, seqlens, W, scale, causal)
    torch.cuda.synchronize()
    tol = 5e-5 if dtype == "bf16" else 1e-5
    assert rel_err(s_g.cpu().numpy(), s_o, 1e-30).max() < tol
    np.testing.assert_allclose(st_g.cpu().numpy()[..., 0], st_o[..., 0], rtol=1e-5)
    assert torch.equal(s_v, s_g) and torch.equal(st_v, st_g)


@pytest.mark.parametrize("seed", range(12))
def test_nestedkv(seed):
    rng = np.random.default_rng(4000 + seed)
    seqlens = [min(n, 9000) for n in _seqlens(rng)]
    L, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    nblocks = int(rng.choice([1, 7, 32, 100]))
    k = rng.standard_normal((L, Hkv, sum(seqlens), d), dtype=np.float32)
    if dtype == "bf16":
        k = S.round_bf16(k)
    note(f"  {dtype} d={d} seqlens={seqlens} L={L} Hkv={Hkv} nblocks={nblocks}")
    _, an_g, wt_g = hk.hubkv_nestedkv(to_dev(k, dtype), seqlens, nblocks=nblocks, want_parts=True)
    torch.cuda.synchronize()
    _, an_o, wt_o = oracle.nestedkv(k, seqlens, nblocks, 64, (0.0, 0.0, 0.0), 0.1, want_parts=True)
    np.testing.assert_allclose(an_g.cpu().numpy(), an_o, rtol=0, atol=5e-5)
    np.testing.assert_allclose(wt_g.cpu().numpy(), wt_o, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("seed", range(16))
def test_h2o_step(seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = str(rng.choice(["bf16", "f32"]))
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 5))
    B = int(rng.integers(1, 5))
    recent = int(rng.integers(1, 200))
    heavy = int(rng.integers(1, 300))
    C = heavy + recent
    fill = int(rng.choice([C, C, int(rng.integers(0, C + 1))]))
    t = fill + int(rng.integers(0, 1000))
    n_sink = min(int(rng.choice([0, 2, 10])), heavy)  # the windows fit the cache
    inc = int(rng.integers(0, 2))
    w = S.workload(4).with_(B=B, Hkv=Hkv, Hq=G * Hkv, d=d, heavy=heavy, recent=recent,
                            dtype=dtype, n_sink=n_sink)
    st = S.decode_random_state(w, t=t, seed=seed, fill=fill)
    note(f"  {dtype} d={d} B={B} Hkv={Hkv} G={G} C={C} fill={fill} t={t} sink={n_sink} "
         f"recent={recent} self={inc}")
    ds = {"K": to_dev(st["K"], dtype), "V": to_dev(st["V"], dtype),
          "acc": torch.from_numpy(st["acc"].copy()).cuda(),
          "pos": torch.from_numpy(st["pos"].copy()).cuda()}
    probs = torch.full((B, G * Hkv, C + 1), float("nan"), device="cuda")
    out = torch.full((B, G * Hkv, d), float("nan"), dtype=torch.float32, device="cuda")
    ev_g = hk.h2o_step(to_dev(st["q"], dtype), to_dev(st["k_new"], dtype),
                       to_dev(st["v_new"], dtype), ds["K"], ds["V"], ds["acc"], ds["pos"], t,
                       w.scale, n_sink, recent, inc, probs=probs, out=out)
    torch.cuda.synchronize()
    st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
    ev_o, pr_o, mg, o_o = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale,
                                          n_sink, recent, inc, want_probs=True, want_margin=True,
                                          want_out=True)
    tol = 1e-5 if dtype == "f32" else 2e-2
    np.testing.assert_allclose(probs.cpu().numpy(), pr_o, rtol=tol, atol=1e-7)
    ev_g = ev_g.cpu().numpy()
    same = ev_g == ev_o
    assert np.all(same | (mg <= 1e-4)), f"{int((~same).sum())} evictions differ without a near-tie"
    acc_g, pos_g = ds["acc"].cpu().numpy(), ds["pos"].cpu().numpy()
    K_g, V_g = to_host(ds["K"]), to_host(ds["V"])
    for b in range(B):
        for h in range(Hkv):
            if not same[b, h]:
                continue
            np.testing.assert_array_equal(pos_g[b, h], st_o["pos"][b, h])
            np.testing.assert_array_equal(K_g[b, h], st_o["K"][b, h])
            np.testing.assert_array_equal(V_g[b, h], st_o["V"][b, h])
            assert rel_err(acc_g[b, h], st_o["acc"][b, h], 1e-30).max() < tol
    # output error against the scale of its terms, sum_slot p |v|
    o_g = out.cpu().numpy()
    assert np.isfinite(o_g).all()
    Va = np.where((st["pos"] >= 0)[..., None], np.abs(st["V"].astype(np.float64)), 0.0)
    for b in range(B):
        for hq in range(G * Hkv):
            g = hq // G
            scale = pr_o[b, hq, :-1].astype(np.float64) @ Va[b, g] + \
                pr_o[b, hq, -1] * np.abs(st["v_new"][b, g].astype(np.float64))
            err = np.abs(o_g[b, hq] - o_o[b, hq]) / np.maximum(scale, 1e-30)
            assert err.max() < (1e-5 if dtype == "f32" else 1e-4), err.max()


@pytest.mark.parametrize("seed", range(10))
def test_h2o_ring_stream(seed):
    """h2o_step_ring from an empty cache for C + 10..80 steps beside the
    oracle's fixed slots: the same evictions (near-ties aside), and at the end
    the same retained positions, scores and K/V rows."""
    rng = np.random.default_rng(6000 + seed)
    dtype = str(rng.choice(["bf16", "f32"]))
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4]))
    Hkv, B = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    heavy, recent = int(rng.integers(1, 61)), int(rng.integers(1, 41))
    C = heavy + recent
    n_sink = int(rng.integers(0, min(heavy, 5) + 1))
    inc = int(rng.integers(0, 2))
    steps = C + int(rng.integers(10, 81))
    w = S.workload(4).with_(B=B, Hkv=Hkv, Hq=G * Hkv, d=d, heavy=heavy, recent=recent,
                            dtype=dtype, n_sink=n_sink)
    note(f"  {dtype} d={d} B={B} Hkv={Hkv} G={G} heavy={heavy} recent={recent} "
         f"sink={n_sink} self={inc} steps={steps}")
    q = rng.standard_normal((steps, B, G * Hkv, d), dtype=np.float32)
    k = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = S.round_bf16(q), S.round_bf16(k), S.round_bf16(v)
    st_o = oracle.empty_state(B, Hkv, C, d)
    ds = {"K": to_dev(st_o["K"], dtype), "V": to_dev(st_o["V"], dtype),
          "acc": torch.from_numpy(st_o["acc"].copy()).cuda(),
          "pos": torch.from_numpy(st_o["pos"].copy()).cuda()}
    diverged = np.zeros((B, Hkv), bool)
    for t in range(steps):
        ev_g = hk.h2o_step(to_dev(q[t], dtype), to_dev(k[t], dtype), to_dev(v[t], dtype),
                           ds["K"], ds["V"], ds["acc"], ds["pos"], t, w.scale, n_sink, recent,
                           inc, ring=True)
        ev_o, mg = oracle.h2o_step(st_o, q[t], k[t], v[t], t, w.scale, n_sink, recent, inc,
                                   want_margin=True)
        newly = (ev_g.cpu().numpy() != ev_o) & ~diverged
        assert np.all(mg[newly] <= 1e-4), f"step {t}: divergence without a near-tie"
        diverged |= newly
    pos_g, acc_g = ds["pos"].cpu().numpy(), ds["acc"].cpu().numpy()
    K_g, V_g = to_host(ds["K"]), to_host(ds["V"])
    tol = 1e-4 if dtype == "f32" else 2e-2
    for b in range(B):
        for g in range(Hkv):
            if diverged[b, g]:
                continue
            og = np.argsort(np.where(pos_g[b, g] >= 0, pos_g[b, g], np.iinfo(np.int32).max))
            oo = np.argsort(np.where(st_o["pos"][b, g] >= 0, st_o["pos"][b, g],
                                     np.iinfo(np.int32).max))
            np.testing.assert_array_equal(pos_g[b, g][og], st_o["pos"][b, g][oo])
            live = st_o["pos"][b, g][oo] >= 0
            assert rel_err(acc_g[b, g][og][live], st_o["acc"][b, g][oo][live], 1e-30).max() < tol
            np.testing.assert_array_equal(K_g[b, g][og][live], st_o["K"][b, g][oo][live])
            np.testing.assert_array_equal(V_g[b, g][og][live], st_o["V"][b, g][oo][live])
