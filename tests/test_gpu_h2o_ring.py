"""GPU checks of the ring slot layout of the streaming H2O step
(h2o_step_ring) against the CPU oracle, which keeps fixed slots.

The two layouts place tokens in different slots but must retain the same
tokens with the same scores.  Along free-running streams from an empty cache:
* the evicted positions agree step by step (a first divergence must be a
  near-tie of the oracle's candidates, as for the fixed layout);
* each step's probabilities, matched by position, agree within the dtype's
  bar, and so does the attention output (bar as in the fixed-layout tests);
* after every step the ring holds exactly the last n_recent positions, each
  in slot C - n_recent + p mod n_recent;
* at the end, per (sequence, head), the retained positions, their scores and
  their K/V rows (by position) equal the oracle's.
"""
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


def _by_pos(pos, vals):
    """{position: value} of the occupied slots of one (sequence, head)."""
    return {int(p): v for p, v in zip(pos, vals) if p >= 0}


def _check_ring(pos, t, C, R):
    """Ring slots hold the last min(R, t + 1) positions, position p in slot
    C - R + p mod R; the heavy slots hold none of them."""
    H = C - R
    want = set(range(max(0, t - R + 1), t + 1))
    ring = pos[..., H:]
    for b in range(pos.shape[0]):
        for h in range(pos.shape[1]):
            got = {int(p) for p in ring[b, h] if p >= 0}
            assert got == want, (b, h, t)
            for j, p in enumerate(ring[b, h]):
                if p >= 0:
                    assert j == p % R
            assert not (set(pos[b, h, :H].tolist()) & want)


CASES = [
    # dtype, G, d, heavy, recent, n_sink, include_self, with the output
    ("f32", 2, 64, 24, 16, 2, 0, True),
    ("f32", 1, 128, 20, 12, 0, 1, False),
    ("bf16", 4, 64, 24, 16, 2, 0, True),
    ("bf16", 2, 128, 30, 1, 3, 0, False),   # a ring of one slot
    ("f32", 8, 64, 1, 24, 0, 1, True),      # one heavy slot
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-G{c[1]}-d{c[2]}-H{c[3]}-R{c[4]}-s{c[5]}-i{c[6]}-o{int(c[7])}")
def test_ring_stream_matches_oracle(case):
    dtype, G, d, heavy, recent, n_sink, inc, want_out = case
    w = S.workload(4).with_(B=2, Hkv=2, Hq=2 * G, d=d, heavy=heavy, recent=recent, dtype=dtype,
                            n_sink=n_sink)
    B, Hkv, Hq, Cs = w.B, w.Hkv, w.Hq, w.C
    steps = 150
    rng = np.random.default_rng(heavy * 31 + recent + G)
    q = rng.standard_normal((steps, B, Hq, d), dtype=np.float32)
    k = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((steps, B, Hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = S.round_bf16(q), S.round_bf16(k), S.round_bf16(v)
    st_o = oracle.empty_state(B, Hkv, Cs, d)
    ds = dict(K=to_dev(st_o["K"], dtype), V=to_dev(st_o["V"], dtype),
              acc=torch.from_numpy(st_o["acc"].copy()).cuda(),
              pos=torch.from_numpy(st_o["pos"].copy()).cuda())
    tol = 1e-5 if dtype == "f32" else 2e-2
    diverged = np.zeros((B, Hkv), bool)
    for t in range(steps):
        pos_g0 = ds["pos"].cpu().numpy()
        pos_o0, V_o0 = st_o["pos"].copy(), st_o["V"].copy()
        probs = torch.full((B, Hq, Cs + 1), float("nan"), device="cuda")
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda") \
            if want_out else None
        ev_g = hk.h2o_step(to_dev(q[t], dtype), to_dev(k[t], dtype), to_dev(v[t], dtype),
                           ds["K"], ds["V"], ds["acc"], ds["pos"], t, w.scale, n_sink, recent,
                           inc, probs=probs, out=out, ring=True)
        torch.cuda.synchronize()
        ev_g = ev_g.cpu().numpy()
        pr_g = probs.cpu().numpy()
        res = oracle.h2o_step(st_o, q[t], k[t], v[t], t, w.scale, n_sink, recent, inc,
                              want_probs=True, want_margin=True, want_out=want_out)
        ev_o, pr_o, mg = res[:3]
        newly = (ev_g != ev_o) & ~diverged
        assert np.all(mg[newly] <= 1e-4), f"step {t}: divergence without a near-tie"
        diverged |= newly
        _check_ring(ds["pos"].cpu().numpy(), t, Cs, recent)
        for b in range(B):
            for hq in range(Hq):
                g = hq // G
                if diverged[b, g]:
                    continue
                pg = _by_pos(pos_g0[b, g], pr_g[b, hq, :-1])
                po = _by_pos(pos_o0[b, g], pr_o[b, hq, :-1])
                assert pg.keys() == po.keys()
                for p in po:
                    assert abs(pg[p] - po[p]) <= tol * abs(po[p]) + 1e-7
                assert abs(pr_g[b, hq, -1] - pr_o[b, hq, -1]) <= tol * abs(pr_o[b, hq, -1]) + 1e-7
        if want_out:
            o_g, o_o = out.cpu().numpy(), res[3]
            keep = np.repeat(~diverged, G, axis=1)
            o_g = np.where(keep[..., None], o_g, o_o)
            Va = np.where((pos_o0 >= 0)[..., None], np.abs(V_o0.astype(np.float64)), 0.0)
            for b in range(B):
                for hq in range(Hq):
                    g = hq // G
                    size = pr_o[b, hq, :-1].astype(np.float64) @ Va[b, g] + \
                        pr_o[b, hq, -1] * np.abs(v[t][b, g].astype(np.float64))
                    err = np.abs(o_g[b, hq].astype(np.float64) - o_o[b, hq])
                    assert np.all(err <= tol * np.maximum(size, 1e-30)), (t, b, hq)
    assert diverged.mean() <= 0.5
    pos_g, acc_g = ds["pos"].cpu().numpy(), ds["acc"].cpu().numpy()
    K_g, V_g = to_host(ds["K"]), to_host(ds["V"])
    for b in range(B):
        for g in range(Hkv):
            if diverged[b, g]:
                continue
            ag = _by_pos(pos_g[b, g], acc_g[b, g])
            ao = _by_pos(st_o["pos"][b, g], st_o["acc"][b, g])
            assert ag.keys() == ao.keys()
            assert rel_err([ag[p] for p in ao], list(ao.values()), 1e-30).max() < 1e-4
            kg = _by_pos(pos_g[b, g], K_g[b, g])
            ko = _by_pos(st_o["pos"][b, g], st_o["K"][b, g])
            vg = _by_pos(pos_g[b, g], V_g[b, g])
            vo = _by_pos(st_o["pos"][b, g], st_o["V"][b, g])
            for p in ko:
                np.testing.assert_array_equal(kg[p], ko[p])
                np.testing.assert_array_equal(vg[p], vo[p])


def test_ring_and_fixed_layouts_on_the_decode_shape():
    """The decode workload's cache shape (2048 heavy + 2048 recent slots,
    d 128, bf16; 4 sequences x 8 heads) for the first 4200 positions, both
    layouts on the GPU from empty.  The softmax sums round differently with
    the slot order, so a near-tie may flip an eviction; at least 3/4 of the
    (sequence, head) units must evict the same positions at every step, and
    those units must end with the same positions and scores."""
    w = S.workload(4).with_(B=4, Hkv=8, Hq=8)
    B, Hkv, Hq, d, Cs = w.B, w.Hkv, w.Hq, w.d, w.C
    steps = Cs + 104
    note(f"  {steps} steps of both layouts")
    gen = torch.Generator(device="cuda").manual_seed(3)
    st = {}
    for name in ("fixed", "ring"):
        st[name] = dict(K=torch.zeros((B, Hkv, Cs, d), dtype=torch.bfloat16, device="cuda"),
                        V=torch.zeros((B, Hkv, Cs, d), dtype=torch.bfloat16, device="cuda"),
                        acc=torch.zeros((B, Hkv, Cs), dtype=torch.float32, device="cuda"),
                        pos=torch.full((B, Hkv, Cs), -1, dtype=torch.int32, device="cuda"))
    same = torch.ones((B, Hkv), dtype=torch.bool, device="cuda")
    for t in range(steps):
        q = torch.randn((B, Hq, d), generator=gen, device="cuda").to(torch.bfloat16)
        kn = torch.randn((B, Hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
        vn = torch.randn((B, Hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
        evs = []
        for name in ("fixed", "ring"):
            s = st[name]
            evs.append(hk.h2o_step(q, kn, vn, s["K"], s["V"], s["acc"], s["pos"], t, w.scale,
                                   w.n_sink, w.recent, 0, ring=name == "ring"))
        same &= evs[0] == evs[1]
    torch.cuda.synchronize()
    # rounding of the softmax sums differs with the slot order, so a near-tie
    # may flip; it must stay rare
    assert same.float().mean().item() >= 0.75
    pf, pr = st["fixed"]["pos"].cpu().numpy(), st["ring"]["pos"].cpu().numpy()
    af, ar = st["fixed"]["acc"].cpu().numpy(), st["ring"]["acc"].cpu().numpy()
    ok = same.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            if not ok[b, g]:
                continue
            fa, ra = _by_pos(pf[b, g], af[b, g]), _by_pos(pr[b, g], ar[b, g])
            assert fa.keys() == ra.keys()
            assert rel_err([ra[p] for p in fa], list(fa.values()), 1e-30).max() < 1e-4
    _check_ring(pr, steps - 1, Cs, w.recent)
