"""GPU parity of the streaming H2O step (h2o_step) against the CPU oracle.

* Single steps from the same drawn mid-stream state (the decode workload's full
  shape: 16 sequences x 32 heads x 4096 slots x d 128, bf16): probabilities and
  accumulated scores within tolerance, identical evictions except where the
  oracle's two lowest candidate scores are a near-tie, identical slot writes.
* Free-running streams on small shapes: the evicted positions agree step by
  step; where they first diverge the oracle must report a near-tie.
* The literal budget-3 run of the greedy algorithm keeps the first 3 tokens.
* The optional attention output (decode attention over the retained tokens):
  on the full decode shape, on partly empty caches whose empty rows hold NaN,
  for every group size class (G = 1, 2, 3, 8, 16, the last with the largest
  LDS footprint) and along free-running streams.  Error bar: |out - oracle| <=
  tol * sum_slot p(slot) |v_slot| (the size of the convex combination), tol
  1e-5 for fp32 inputs and 2e-2 for bf16 inputs (with a 1e-4 diagnostic: the
  arithmetic is fp32 on exact bf16 values).
"""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic as S
from gpu_helpers import note, rel_err, threads, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import token_scoring_top_amd as hk  # noqa: E402

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, scope="module")
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hk.lib()
    oracle.set_threads(threads())


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _dev_state(st, dtype):
    return dict(K=to_dev(st["K"], dtype), V=to_dev(st["V"], dtype),
                acc=torch.from_numpy(np.ascontiguousarray(st["acc"])).cuda(),
                pos=torch.from_numpy(np.ascontiguousarray(st["pos"])).cuda())


def _gpu_step(ds, q, kn, vn, t, w, n_sink, n_recent, include_self, dtype, want_probs=True):
    B, Hq = q.shape[0], q.shape[1]
    probs = torch.full((B, Hq, w.C + 1), float("nan"), device="cuda") if want_probs else None
    ev = hk.h2o_step(to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), ds["K"], ds["V"],
                     ds["acc"], ds["pos"], t, w.scale, n_sink, n_recent, include_self, probs=probs)
    torch.cuda.synchronize()
    return ev.cpu().numpy(), (probs.cpu().numpy() if want_probs else None)


def _gpu_step_out(ds, q, kn, vn, t, w, n_sink, n_recent, include_self, dtype):
    B, Hq, d = q.shape
    probs = torch.full((B, Hq, w.C + 1), float("nan"), device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ev = hk.h2o_step(to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), ds["K"], ds["V"],
                     ds["acc"], ds["pos"], t, w.scale, n_sink, n_recent, include_self,
                     probs=probs, out=out)
    torch.cuda.synchronize()
    return ev.cpu().numpy(), probs.cpu().numpy(), out.cpu().numpy()


def _out_err(o_g, o_o, pr_o, V, vn, pos):
    """max over (b, h, e) of |o_g - o_o| / sum_slot p |v_slot| (the oracle's p;
    empty slots carry p = 0 and are masked out of V)."""
    B, Hq, d = o_o.shape
    Hkv = V.shape[1]
    G = Hq // Hkv
    Va = np.where((pos >= 0)[..., None], np.abs(V.astype(np.float64)), 0.0)
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            g = h // G
            scale = pr_o[b, h, :-1].astype(np.float64) @ Va[b, g] + \
                pr_o[b, h, -1] * np.abs(vn[b, g].astype(np.float64))
            e = np.abs(o_g[b, h].astype(np.float64) - o_o[b, h]) / np.maximum(scale, 1e-30)
            worst = max(worst, float(e.max()))
    assert np.isfinite(o_g).all()
    return worst


def _compare_step(ds, st_o, ev_g, ev_o, pr_g, pr_o, margin, tol, dtype):
    np.testing.assert_allclose(pr_g, pr_o, rtol=tol, atol=1e-7)
    acc_g = ds["acc"].cpu().numpy()
    pos_g = ds["pos"].cpu().numpy()
    K_g, V_g = to_host(ds["K"]), to_host(ds["V"])
    same = ev_g == ev_o
    # any different choice must come from a near-tie in the oracle's scores
    assert np.all(same | (margin <= 1e-4)), \
        f"{int((~same).sum())} evictions differ without a near-tie"
    for b in range(ev_g.shape[0]):
        for h in range(ev_g.shape[1]):
            if not same[b, h]:
                continue
            np.testing.assert_array_equal(pos_g[b, h], st_o["pos"][b, h])
            np.testing.assert_array_equal(K_g[b, h], st_o["K"][b, h])
            np.testing.assert_array_equal(V_g[b, h], st_o["V"][b, h])
            assert rel_err(acc_g[b, h], st_o["acc"][b, h], 1e-30).max() < tol
    return int((~same).sum())


@pytest.mark.parametrize("include_self", [0, 1])
def test_single_step_full_decode_shape(include_self):
    w = S.workload(4)
    t = w.prompt + 5
    note("  drawing a 16 x 32 x 4096-slot state")
    st = S.decode_random_state(w, t=t, seed=11 + include_self)
    ds = _dev_state(st, w.dtype)
    ev_g, pr_g = _gpu_step(ds, st["q"], st["k_new"], st["v_new"], t, w, w.n_sink, w.recent,
                           include_self, w.dtype)
    st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
    note("  oracle step")
    ev_o, pr_o, mg = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale,
                                     w.n_sink, w.recent, include_self, want_probs=True,
                                     want_margin=True)
    nd = _compare_step(ds, st_o, ev_g, ev_o, pr_g, pr_o, mg, 2e-2, w.dtype)
    assert nd <= 2
    # fp32 accumulation over exact bf16 products: far inside the bf16 bar
    assert rel_err(pr_g, pr_o, 1e-12).max() < 1e-4


@pytest.mark.parametrize("dtype,d,G", [("f32", 64, 1), ("bf16", 128, 2), ("f32", 128, 4),
                                       ("bf16", 64, 1)])
def test_single_step_partial_cache(dtype, d, G):
    # some slots still empty: the new token takes the lowest empty slot
    w = S.workload(4).with_(B=3, Hkv=2, Hq=2 * G, d=d, heavy=40, recent=24, dtype=dtype, n_sink=2)
    t = 50
    st = S.decode_random_state(w, t=t, seed=5, fill=50)
    ds = _dev_state(st, dtype)
    ev_g, pr_g = _gpu_step(ds, st["q"], st["k_new"], st["v_new"], t, w, 2, w.recent, 0, dtype)
    st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
    ev_o, pr_o, mg = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale, 2,
                                     w.recent, 0, want_probs=True, want_margin=True)
    assert (ev_o == -1).all()
    _compare_step(ds, st_o, ev_g, ev_o, pr_g, pr_o, mg, 1e-5 if dtype == "f32" else 2e-2, dtype)


def _stream_case(w, steps, n_sink, n_recent, include_self, tol):
    B, Hkv, Hq, d, Cs = w.B, w.Hkv, w.Hq, w.d, w.C
    rng = np.random.default_rng(steps + Cs)
    q = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = S.round_bf16(q), S.round_bf16(k), S.round_bf16(v)
    st_o = oracle.empty_state(B, Hkv, Cs, d)
    ds = _dev_state(st_o, w.dtype)
    diverged = np.zeros((B, Hkv), bool)
    for t in range(steps):
        ev_g, _ = _gpu_step(ds, q[t], k[t], v[t], t, w, n_sink, n_recent, include_self, w.dtype,
                            want_probs=False)
        ev_o, mg = oracle.h2o_step(st_o, q[t], k[t], v[t], t, w.scale, n_sink, n_recent,
                                   include_self, want_margin=True)
        newly = (ev_g != ev_o) & ~diverged
        # a first divergence must be a near-tie of the oracle's candidates
        assert np.all(mg[newly] <= 1e-4), f"step {t}: divergence without a near-tie"
        diverged |= newly
    pos_g = ds["pos"].cpu().numpy()
    acc_g = ds["acc"].cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            if diverged[b, h]:
                continue
            np.testing.assert_array_equal(np.sort(pos_g[b, h]), np.sort(st_o["pos"][b, h]))
            np.testing.assert_array_equal(pos_g[b, h], st_o["pos"][b, h])
            assert rel_err(acc_g[b, h], st_o["acc"][b, h], 1e-30).max() < tol
    return diverged.mean()


@pytest.mark.parametrize("dtype,include_self", [("f32", 0), ("f32", 1), ("bf16", 0)])
def test_free_running_stream(dtype, include_self):
    w = S.workload(4).with_(B=2, Hq=4, Hkv=2, d=64, heavy=24, recent=16, dtype=dtype)
    frac = _stream_case(w, 200, 2, 16, include_self, 1e-4)
    assert frac <= 0.5


@pytest.mark.parametrize("heavy,recent,n_sink", [(1, 0, 0), (0, 1, 0), (1, 0, 1), (1, 1, 0),
                                                  (1, 1, 1), (2, 0, 0), (0, 2, 0), (1, 2, 1),
                                                  (2, 0, 2), (3, 2, 0)])
@pytest.mark.parametrize("include_self", [0, 1])
def test_degenerate_caches(heavy, recent, n_sink, include_self):
    # caches of 1 to 5 slots from an empty state, windows of size 0 up to the
    # whole cache (every retained token protected: the token leaving the
    # recent window, or the new token itself, is then the only candidate)
    w = S.workload(4).with_(B=2, Hq=4, Hkv=2, d=64, heavy=heavy, recent=recent, dtype="f32")
    _stream_case(w, 40, n_sink, recent, include_self, 1e-4)


def test_literal_budget3_algorithm1_on_gpu():
    gold = json.load(open(os.path.join(GOLD, "h2o_alg1_budget3_literal.json")))
    w = S.H2O_TINY
    for seed in range(3):
        rng = np.random.default_rng(seed)
        N = gold["N"]
        q = rng.standard_normal((N, 1, w.Hq, w.d), dtype=np.float32)
        k = rng.standard_normal((N, 1, w.Hkv, w.d), dtype=np.float32)
        st_o = oracle.empty_state(1, w.Hkv, gold["budget"], w.d)
        ds = _dev_state(st_o, "f32")
        ww = w.with_(heavy=gold["budget"], recent=0)
        for t in range(N):
            ev_g, pr_g = _gpu_step(ds, q[t], k[t], k[t], t, ww, 0, 0, 0, "f32")
            ev_o, pr_o = oracle.h2o_step(st_o, q[t], k[t], k[t], t, w.scale, 0, 0, 0,
                                         want_probs=True)
            np.testing.assert_array_equal(ev_g, ev_o)
            np.testing.assert_allclose(pr_g, pr_o, rtol=1e-5, atol=1e-7)
        pos_g = ds["pos"].cpu().numpy()
        for h in range(w.Hkv):
            assert sorted(pos_g[0, h].tolist()) == gold["final_set"]


@pytest.mark.parametrize("include_self", [0, 1])
def test_attention_output_full_decode_shape(include_self):
    w = S.workload(4)
    t = w.prompt + 9
    note("  drawing a 16 x 32 x 4096-slot state")
    st = S.decode_random_state(w, t=t, seed=21 + include_self)
    ds = _dev_state(st, w.dtype)
    ev_g, pr_g, o_g = _gpu_step_out(ds, st["q"], st["k_new"], st["v_new"], t, w, w.n_sink,
                                    w.recent, include_self, w.dtype)
    st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
    note("  oracle step")
    ev_o, pr_o, mg, o_o = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale,
                                          w.n_sink, w.recent, include_self, want_probs=True,
                                          want_margin=True, want_out=True)
    err = _out_err(o_g, o_o, pr_o, st["V"], st["v_new"], st["pos"])
    assert err < 2e-2
    assert err < 1e-4, err
    # the output does not disturb the step itself
    _compare_step(ds, st_o, ev_g, ev_o, pr_g, pr_o, mg, 2e-2, w.dtype)


@pytest.mark.parametrize("dtype,d,G,C", [("f32", 64, 1, 64), ("bf16", 128, 2, 64),
                                         ("bf16", 128, 3, 96), ("f32", 128, 8, 200),
                                         ("bf16", 64, 8, 130), ("bf16", 128, 16, 960),
                                         ("f32", 64, 16, 300)])
def test_attention_output_group_sizes_with_empty_slots(dtype, d, G, C):
    # a quarter of the slots are empty and their K/V rows hold NaN: they must
    # stay out of the logits, the normaliser and the output
    rec = min(24, C // 4)
    w = S.workload(4).with_(B=3, Hkv=2, Hq=2 * G, d=d, heavy=C - rec, recent=rec, dtype=dtype,
                            n_sink=2)
    t = 3 * C
    fill = C - C // 4
    st = S.decode_random_state(w, t=t, seed=G * 7 + d, fill=fill)
    empty = st["pos"] < 0
    st["K"][empty] = np.nan
    st["V"][empty] = np.nan
    ds = _dev_state(st, dtype)
    tol = 1e-5 if dtype == "f32" else 2e-2
    for inc in (0, 1):
        ds2 = {k: v.clone() for k, v in ds.items()}
        ev_g, pr_g, o_g = _gpu_step_out(ds2, st["q"], st["k_new"], st["v_new"], t, w, 2, rec,
                                        inc, dtype)
        st_o = {k: st[k].copy() for k in ("K", "V", "acc", "pos")}
        ev_o, pr_o, o_o = oracle.h2o_step(st_o, st["q"], st["k_new"], st["v_new"], t, w.scale,
                                          2, rec, inc, want_probs=True, want_out=True)
        assert (ev_o == -1).all() and (ev_g == -1).all()
        err = _out_err(o_g, o_o, pr_o, np.nan_to_num(st["V"]), st["v_new"], st["pos"])
        assert err < tol, err
        if dtype == "bf16":
            assert err < 1e-4, err


def test_attention_output_empty_cache():
    # nothing cached: the output is v_new when the token attends to itself,
    # zeros otherwise
    w = S.workload(4).with_(B=2, Hkv=2, Hq=4, d=128, heavy=16, recent=16, dtype="f32", n_sink=0)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 128), dtype=np.float32)
    kn = rng.standard_normal((2, 2, 128), dtype=np.float32)
    vn = rng.standard_normal((2, 2, 128), dtype=np.float32)
    for inc in (0, 1):
        ds = _dev_state(oracle.empty_state(2, 2, w.C, 128), "f32")
        _, _, o_g = _gpu_step_out(ds, q, kn, vn, 0, w, 0, 16, inc, "f32")
        want = np.repeat(vn, 2, axis=1) if inc else np.zeros_like(o_g)
        np.testing.assert_array_equal(o_g, want)


@pytest.mark.parametrize("dtype,include_self", [("f32", 1), ("bf16", 0)])
def test_attention_output_free_running_stream(dtype, include_self):
    w = S.workload(4).with_(B=2, Hq=8, Hkv=2, d=64, heavy=24, recent=16, dtype=dtype)
    B, Hkv, Hq, d, Cs = w.B, w.Hkv, w.Hq, w.d, w.C
    steps = 120
    rng = np.random.default_rng(77)
    q = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = S.round_bf16(q), S.round_bf16(k), S.round_bf16(v)
    st_o = oracle.empty_state(B, Hkv, Cs, d)
    ds = _dev_state(st_o, dtype)
    diverged = np.zeros((B, Hkv), bool)
    tol = 1e-5 if dtype == "f32" else 1e-4
    G = Hq // Hkv
    for t in range(steps):
        V_before, pos_before = st_o["V"].copy(), st_o["pos"].copy()
        ev_g, _, o_g = _gpu_step_out(ds, q[t], k[t], v[t], t, w, 2, 16, include_self, dtype)
        ev_o, pr_o, mg, o_o = oracle.h2o_step(st_o, q[t], k[t], v[t], t, w.scale, 2, 16,
                                              include_self, want_probs=True, want_margin=True,
                                              want_out=True)
        if t == 0 and not include_self:
            assert (o_g == 0).all()
        else:
            # units whose caches already differ are skipped
            keep = np.repeat(~diverged, G, axis=1)
            o_gm = np.where(keep[..., None], o_g, o_o)
            assert _out_err(o_gm, o_o, pr_o, V_before, v[t], pos_before) < tol
        newly = (ev_g != ev_o) & ~diverged
        assert np.all(mg[newly] <= 1e-4), f"step {t}: divergence without a near-tie"
        diverged |= newly
    assert diverged.mean() <= 0.5


@pytest.mark.parametrize("ring", [False, True], ids=["fixed", "ring"])
def test_free_running_decode_workload(ring):
    """The decode workload at full size (16 sequences x 32 KV heads, 2048 heavy
    + 2048 recent slots, d 128, bf16) streamed through h2o_step (or
    h2o_step_ring) from an empty cache: the 16384-token prompt, then the 512
    decode steps.  The oracle follows 16 sampled (sequence, KV head) units
    beside the GPU, each side on its own state, fed the same per-step inputs.
    Every first divergence of a unit must be a near-tie of the oracle's
    eviction candidates (their two smallest accumulated scores within the
    bf16 bar); a unit that never diverges must end with the same tokens (in
    the same slots with fixed slots; matched by position with the ring, whose
    slots differ) and the same accumulated scores within that bar."""
    import bench
    w = S.workload(4)
    total = w.prompt + w.decode
    note(f"  streaming {total} steps ({'ring' if ring else 'fixed'} slots) on the GPU, the "
         f"oracle beside it on {len(bench.DECODE_SAMPLE_UNITS)} units")
    ds = bench.DecodeStream(w, total, ring=ring)
    ds.run_gpu(total, oracle_beside=True)
    ds.run_oracle(total)
    st = ds.stats()
    note(f"  identical evictions {st['identical_eviction_frac']:.5f} "
         f"(decode steps {st['identical_eviction_frac_decode']:.5f}), "
         f"{st['units_diverged']} unit(s) diverged at steps {st['first_divergence_steps']} "
         f"with oracle margins {st['first_divergence_oracle_margins']}, "
         f"final-set overlap mean {st['final_set_overlap_mean']:.5f} "
         f"min {st['final_set_overlap_min']:.5f}")
    assert st["steps"] == total
    assert st["evictions_compared"] >= len(ds.units) * (total - w.C)
    assert all(m <= 2e-2 for m in st["first_divergence_oracle_margins"]), st
    diverged = set()
    for u in range(len(ds.units)):
        if np.any(ds.ev_gpu[:, u] != ds.ev_orc[:, u]):
            diverged.add(u)
    pos_g = ds.pos[ds.ub, ds.ug].cpu().numpy()
    acc_g = ds.acc[ds.ub, ds.ug].cpu().numpy()
    for u in range(len(ds.units)):
        if u in diverged:
            continue
        po, ao = ds.ost["pos"][u, 0], ds.ost["acc"][u, 0]
        if ring:
            og, oo = np.argsort(pos_g[u]), np.argsort(po)
            np.testing.assert_array_equal(pos_g[u][og], po[oo])
            assert rel_err(acc_g[u][og], ao[oo], 1e-30).max() < 2e-2
        else:
            np.testing.assert_array_equal(pos_g[u], po)
            assert rel_err(acc_g[u], ao, 1e-30).max() < 2e-2
    if not diverged:
        assert st["final_set_overlap_min"] == 1.0
