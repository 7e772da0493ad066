"""Every entry point launched on a side stream with the binding allocating
the outputs and workspaces, while the current stream keeps allocating,
filling and freeing memory.  The binding allocates on the launch stream, so
no block a pending call still uses can be handed to other work; the results
must meet the same bars against the oracle as the main parity tests (score
within tolerance, refine / select / compaction of the GPU's own scores bit
for bit, decode steps identical up to oracle near-ties)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic as S
from gpu_helpers import note, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import token_scoring_top_amd as hk  # noqa: E402


def _churn(n=6):
    # blocks allocated, written and freed on the current stream while the
    # side stream's kernels are still in flight
    xs = [torch.full((1 << 20,), float(i), device="cuda") for i in range(n)]
    for x in xs:
        x.mul_(3.0)
    del xs


def test_prefill_entry_points_on_a_side_stream():
    w = S.workload(2).with_(seqlens=(9000,), Hq=8, Hkv=4, L=2, clusters=(24,))
    Q, K, V = S.prefill_inputs(w)
    Qd, Kd, Vd = to_dev(Q, w.dtype), to_dev(K, w.dtype), to_dev(V, w.dtype)
    kept = w.kept()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    note("  score / refine+select / refine / select / compact on a side stream")
    s, st = hk.hubkv_score(Qd, Kd, w.seqlens, w.W, w.scale, w.causal, stream=side)
    _churn()
    z, beta, idx = hk.hubkv_refine_select(s, w.seqlens, kept, w.n_sink, w.n_recent,
                                          head_stats=st, pool=w.pool, gamma=w.gamma, r=w.r,
                                          stream=side)
    _churn()
    z2, beta2 = hk.hubkv_refine(s, w.seqlens, head_stats=st, pool=w.pool, gamma=w.gamma, r=w.r,
                                stream=side)
    _churn()
    idx2 = hk.hubkv_select(z2, w.seqlens, kept, w.n_sink, w.n_recent, stream=side)
    _churn()
    ko, vo = hk.hubkv_compact(Kd, Vd, idx, w.seqlens, kept, stream=side)
    _churn()
    side.synchronize()
    s_o, _ = oracle.score(Q, K, w.seqlens, w.W, w.scale, w.causal)
    s_g = s.cpu().numpy()
    assert rel_err(s_g, s_o).max() < 5e-5
    b_g = beta.cpu().numpy()
    z_o = oracle.refine(s_g, w.seqlens, b_g, w.pool, w.gamma, w.r)
    np.testing.assert_array_equal(z.cpu().numpy(), z_o)
    np.testing.assert_array_equal(z2.cpu().numpy(), z_o)
    assert torch.equal(beta, beta2)
    idx_o = oracle.select(z_o, w.seqlens, kept, w.n_sink, w.n_recent)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    np.testing.assert_array_equal(idx2.cpu().numpy(), idx_o)
    k_o, v_o = oracle.compact(K, V, idx_o, w.seqlens, kept)
    np.testing.assert_array_equal(to_host(ko), k_o)
    np.testing.assert_array_equal(to_host(vo), v_o)


def test_layer_budget_and_nestedkv_on_a_side_stream():
    w = S.workload(2).with_(seqlens=(5000, 3000), Hq=4, Hkv=4, L=1, clusters=(12, 8))
    Q, K, V = S.prefill_inputs(w)
    Kd, Vd = to_dev(K, w.dtype), to_dev(V, w.dtype)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    note("  nestedkv / select_layer / compact_layer on a side stream")
    s = hk.hubkv_nestedkv(Kd, w.seqlens, stream=side)
    _churn()
    lk = [[w.Hkv * int(x) for x in w.kept()]]
    floor = int(min(w.kept())) // 4
    idx, hkept = hk.hubkv_select_layer(s, w.seqlens, lk, w.n_sink, w.n_recent, floor,
                                       stream=side)
    _churn()
    ko, vo = hk.hubkv_compact_layer(Kd, Vd, idx, hkept, w.seqlens, lk, stream=side)
    _churn()
    side.synchronize()
    s_g = s.cpu().numpy()
    s_o = oracle.nestedkv(K, w.seqlens)
    assert np.abs(s_g.astype(np.float64) - s_o).max() < 5e-5 or \
        np.mean(np.abs(s_g.astype(np.float64) - s_o) > 5e-5) < 0.01
    i_o, h_o = oracle.select_layer(s_g, w.seqlens, lk, w.n_sink, w.n_recent, floor)
    np.testing.assert_array_equal(idx.cpu().numpy(), i_o)
    np.testing.assert_array_equal(hkept.cpu().numpy(), h_o)
    k_o, v_o = oracle.compact_layer(K, V, i_o, h_o, w.seqlens)
    np.testing.assert_array_equal(to_host(ko), k_o)
    np.testing.assert_array_equal(to_host(vo), v_o)


def test_decode_steps_on_a_side_stream():
    wd = S.workload(4).with_(B=3, Hq=8, Hkv=4, heavy=48, recent=32)
    stt = S.decode_random_state(wd, t=400, seed=7)
    side = torch.cuda.Stream()
    ds = dict(K=to_dev(stt["K"], wd.dtype), V=to_dev(stt["V"], wd.dtype),
              acc=torch.from_numpy(stt["acc"]).cuda(), pos=torch.from_numpy(stt["pos"]).cuda())
    so = {k: stt[k].copy() for k in ("K", "V", "acc", "pos")}
    side.wait_stream(torch.cuda.current_stream())
    rng = np.random.default_rng(11)
    note("  20 decode steps on a side stream")
    for step in range(20):
        t = 400 + step
        q = S.round_bf16(rng.standard_normal((wd.B, wd.Hq, wd.d)).astype(np.float32))
        kn = S.round_bf16(rng.standard_normal((wd.B, wd.Hkv, wd.d)).astype(np.float32))
        vn = S.round_bf16(rng.standard_normal((wd.B, wd.Hkv, wd.d)).astype(np.float32))
        qd, knd, vnd = to_dev(q, wd.dtype), to_dev(kn, wd.dtype), to_dev(vn, wd.dtype)
        side.wait_stream(torch.cuda.current_stream())
        ev = hk.h2o_step(qd, knd, vnd, ds["K"], ds["V"], ds["acc"], ds["pos"], t, wd.scale, 4,
                         wd.recent, False, stream=side)
        _churn(3)
        side.synchronize()
        ev_o, mg = oracle.h2o_step(so, q, kn, vn, t, wd.scale, 4, wd.recent, 0, want_margin=True)
        ev_g = ev.cpu().numpy()
        assert np.all((ev_g == ev_o) | (mg <= 1e-4)), f"step {step}: eviction mismatch"
        if not np.all(ev_g == ev_o):
            return  # states diverged at an oracle near-tie: nothing more to compare
    np.testing.assert_array_equal(ds["pos"].cpu().numpy(), so["pos"])
    assert rel_err(ds["acc"].cpu().numpy(), so["acc"], 1e-6).max() < 2e-2
