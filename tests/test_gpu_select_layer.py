"""GPU parity of the layer-wide budget (hubkv_select_layer, hubkv_compact_layer)
against the CPU oracle.

Given identical fp32 scores the kept positions and the per-head counts are
integer results: they must be bit-exact.  Cases cover single and ragged
batches, several layers, 1 to 32 KV heads, floors from none to the even
share, budgets at both bounds, lengths below, at and across the 4096-position
chunks, ties everywhere, NaN / +-0 / +-inf scores, the Llama-2-7B-shaped layer
and the ragged 64K-512K batch at their full sizes, repeated calls on one
workspace, and the compaction of the result.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from gpu_helpers import note, threads, to_dev, to_host

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


def _bounds(seqlens, Hkv, ns, nr, fl):
    lo, hi = [], []
    for n in seqlens:
        P = oracle.protected_count(n, ns, nr)
        f = min(fl, n - P)
        lo.append(Hkv * (P + f))
        hi.append(Hkv * n)
    return lo, hi


def _run_both(z, seqlens, lk, ns, nr, fl, ws=None):
    zd = to_dev(z, "f32")
    idx_g, hk_g = hk.hubkv_select_layer(zd, seqlens, lk, ns, nr, fl, workspace=ws)
    torch.cuda.synchronize()
    idx_o, hk_o = oracle.select_layer(z, seqlens, lk, ns, nr, fl)
    np.testing.assert_array_equal(hk_g.cpu().numpy(), hk_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
    return idx_o, hk_o


CASES = [
    # seqlens, L, Hkv, n_sink, n_recent, floor, budget fraction (between the bounds), kind
    ([5000], 1, 4, 4, 64, 16, 0.3, "attention"),
    ([4096], 1, 1, 0, 0, 0, 0.5, "uniform"),
    ([300], 2, 8, 2, 8, 5, 0.0, "attention"),
    ([300], 2, 8, 2, 8, 5, 1.0, "attention"),
    ([9000, 130, 4097], 2, 3, 4, 16, 7, 0.2, "attention"),
    ([12000], 1, 6, 4, 32, 0, 0.1, "attention"),
    ([12000], 1, 6, 4, 32, 10000, 0.5, "attention"),
    ([8192, 8191], 3, 2, 1, 1, 100, 0.4, "ties"),
    ([20000], 1, 32, 4, 64, 64, 0.05, "attention"),
    ([300, 5000], 1, 4, 2, 8, 1000, 0.0, "attention"),   # floors take every candidate
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_bitexact_given_scores(case):
    seqlens, L, Hkv, ns, nr, fl, frac, kind = case
    if kind == "ties":
        z = S.random_scores(seqlens, L, Hkv, seed=len(seqlens), ties=True)
    else:
        z = S.random_scores(seqlens, L, Hkv, seed=sum(seqlens) % 97, kind=kind)
    lo, hi = _bounds(seqlens, Hkv, ns, nr, fl)
    lk = [[int(a + frac * (b - a)) for a, b in zip(lo, hi)] for _ in range(L)]
    if L > 1:
        lk[1] = [int(a + (1 - frac) * (b - a)) for a, b in zip(lo, hi)]  # budgets differ per layer
    _run_both(z, seqlens, lk, ns, nr, fl)


def test_specials_and_constant_scores():
    rng = np.random.default_rng(4)
    seqlens = [6000]
    Hkv = 4
    z = rng.random((1, Hkv, 6000), dtype=np.float32)
    pick = rng.random(z.shape)
    z[pick < 0.05] = np.nan
    z[(pick >= 0.05) & (pick < 0.1)] = -0.0
    z[(pick >= 0.1) & (pick < 0.15)] = 0.0
    z[(pick >= 0.15) & (pick < 0.17)] = np.inf
    z[(pick >= 0.17) & (pick < 0.19)] = -np.inf
    z[(pick >= 0.19) & (pick < 0.3)] = -rng.random(int(((pick >= 0.19) & (pick < 0.3)).sum()))
    for lk in (400, 12000, 22000, 23990):
        _run_both(z, seqlens, [[lk]], 4, 8, 3)
    # every score equal: the layer's ties go to the lower heads first
    zc = np.full((1, Hkv, 6000), 0.25, np.float32)
    for lk in (200, 9001, 23999):
        _run_both(zc, seqlens, [[lk]], 4, 8, 20)


def test_repeated_calls_on_one_workspace():
    seqlens = [7000, 3000]
    L, Hkv = 2, 5
    z = S.random_scores(seqlens, L, Hkv, seed=9)
    nb = hk.lib().hubkv_select_layer_workspace(2, hk._arr64(seqlens), L, Hkv)
    ws = torch.full((nb,), 255, dtype=torch.uint8, device="cuda")
    lo, hi = _bounds(seqlens, Hkv, 4, 16, 8)
    for frac in (0.1, 0.7, 0.1, 0.3):
        lk = [[int(a + frac * (b - a)) for a, b in zip(lo, hi)]] * L
        _run_both(z, seqlens, lk, 4, 16, 8, ws=ws)


def test_llama2_7b_layer_full_size():
    # the Llama-2-7B-shaped layer: 32 KV heads x 32768 positions, the layer's
    # budget = 10% of every head's tokens, per-head floor 1% of a head
    w = S.workload(2)
    z = S.random_scores(list(w.seqlens), 1, w.Hkv, seed=21)
    lk = [[int(0.1 * w.T) * w.Hkv]]
    note("  layer-wide selection over 32 x 32768 scores")
    _run_both(z, list(w.seqlens), lk, w.n_sink, w.n_recent, 327)


def test_ragged_batch_full_size():
    # the ragged 64K-512K batch (8 KV heads), 10% per sequence, floor 256
    w = S.workload(5)
    z = S.random_scores(list(w.seqlens), 1, w.Hkv, seed=22)
    lk = [[int(0.1 * n) * w.Hkv for n in w.seqlens]]
    note("  layer-wide selection over 8 heads x 983040 scores")
    _run_both(z, list(w.seqlens), lk, w.n_sink, w.n_recent, 256)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_compact_layer_bitexact(dtype, d):
    seqlens = [5000, 777]
    L, Hkv = 2, 3
    rng = np.random.default_rng(d)
    T = sum(seqlens)
    K = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    V = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    if dtype == "bf16":
        K, V = S.round_bf16(K), S.round_bf16(V)
    z = S.random_scores(seqlens, L, Hkv, seed=3)
    lo, hi = _bounds(seqlens, Hkv, 4, 32, 6)
    lk = [[int(a + 0.2 * (b - a)) for a, b in zip(lo, hi)], [int(a + 0.6 * (b - a)) for a, b in zip(lo, hi)]]
    idx_o, hk_o = _run_both(z, seqlens, lk, 4, 32, 6)
    idx_d = torch.from_numpy(idx_o).cuda()
    hk_d = torch.from_numpy(hk_o).cuda()
    ko, vo = hk.hubkv_compact_layer(to_dev(K, dtype), to_dev(V, dtype), idx_d, hk_d, seqlens, lk)
    torch.cuda.synchronize()
    ko_o, vo_o = oracle.compact_layer(K, V, idx_o, hk_o, seqlens)
    np.testing.assert_array_equal(to_host(ko), ko_o)
    np.testing.assert_array_equal(to_host(vo), vo_o)
