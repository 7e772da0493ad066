"""The prefill chain (score -> refine -> select -> compact) captured into a
HIP graph: every replay must give the eager chain's results bit for bit.

Each replay runs on new inputs copied into the captured buffers, with other
eager library calls and synchronisations between the replays; the same
inputs then go through the eager chain and the outputs are compared.  The
library allocates nothing and issues no memset, so the capture holds only
its kernels.
"""
import math

import numpy as np
import pytest

import synthetic as S
from gpu_helpers import note, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import token_scoring_top_amd as hk  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hk.lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


@pytest.mark.parametrize("G,W", [(1, 64), (4, 32)])
def test_prefill_chain_graph_replays_match_eager(G, W):
    seqlens, L, Hkv, d = [3000, 1500], 2, 2, 128
    Hq, T = G * Hkv, sum(seqlens)
    kept = S.budgets(seqlens, 0.15)
    Ksum = int(kept.sum())
    scale = 1 / math.sqrt(d)
    dev = dict(device="cuda")
    Qd = torch.empty((L, Hq, len(seqlens) * W, d), dtype=torch.bfloat16, **dev)
    Kd = torch.empty((L, Hkv, T, d), dtype=torch.bfloat16, **dev)
    Vd = torch.empty_like(Kd)

    def poison(o):
        # every element a replay or an eager chain leaves unwritten stays a
        # sentinel (NaN or -2^31) and fails the comparisons below
        for v in o.values():
            v.fill_(float("nan") if v.is_floating_point() else -(1 << 31))
        return o

    def outputs():
        return poison(dict(s=torch.empty((L, Hkv, T), dtype=torch.float32, **dev),
                    st=torch.empty((L, len(seqlens), Hkv, 2), dtype=torch.float64, **dev),
                    z=torch.empty((L, Hkv, T), dtype=torch.float32, **dev),
                    beta=torch.empty((L, len(seqlens), Hkv), dtype=torch.float32, **dev),
                    idx=torch.empty((L, Hkv, Ksum), dtype=torch.int32, **dev),
                    ko=torch.empty((L, Hkv, Ksum, d), dtype=torch.bfloat16, **dev),
                    vo=torch.empty((L, Hkv, Ksum, d), dtype=torch.bfloat16, **dev)))

    sl = hk._arr64(seqlens)
    ws_s = torch.empty(hk.lib().hubkv_score_workspace(len(seqlens), sl, L, Hq, Hkv, W, d, 1),
                       dtype=torch.uint8, **dev)
    ws_r = torch.empty(max(256, hk.lib().hubkv_refine_workspace(len(seqlens), sl, L, Hkv)),
                       dtype=torch.uint8, **dev)
    ws_q = torch.empty(hk.lib().hubkv_select_workspace(len(seqlens), sl, L, Hkv),
                       dtype=torch.uint8, **dev)
    ws_s.fill_(255)
    ws_r.fill_(255)
    ws_q.fill_(255)

    def chain(o, strm):
        hk.hubkv_score(Qd, Kd, seqlens, W, scale, True, s=o["s"], head_stats=o["st"],
                       workspace=ws_s, stream=strm)
        hk.hubkv_refine(o["s"], seqlens, head_stats=o["st"], r=0.15, z=o["z"],
                        beta_out=o["beta"], workspace=ws_r, stream=strm)
        hk.hubkv_select(o["z"], seqlens, kept, 4, 32, idx=o["idx"], workspace=ws_q, stream=strm)
        hk.hubkv_compact(Kd, Vd, o["idx"], seqlens, kept, k_out=o["ko"], v_out=o["vo"],
                         stream=strm)

    def draw(seed):
        rng = np.random.default_rng(seed)
        for t in (Qd, Kd, Vd):
            t.copy_(to_dev(S.round_bf16(rng.standard_normal(tuple(t.shape), dtype=np.float32)),
                           "bf16"))
        torch.cuda.synchronize()

    og = outputs()
    draw(0)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        chain(og, cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    oe = outputs()
    other = outputs()
    for rep in range(4):
        draw(100 + rep)
        poison(og)
        poison(oe)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in og.items()}
        # eager work of the program between replays, on other output buffers
        chain(other, torch.cuda.current_stream())
        torch.cuda.synchronize()
        chain(oe, torch.cuda.current_stream())
        torch.cuda.synchronize()
        for k in og:
            assert torch.equal(got[k], oe[k]), (rep, k)
        assert torch.equal(other["idx"], oe["idx"])
