"""GPU parity of the NestedKV key-only score (hubkv_nestedkv) against the CPU
oracle, and its use as the base score of a layer-wide selection.

Bar (derived from the arithmetic: cosines of unit vectors formed in fp32 from
exact fp32 / bf16 inputs, against the oracle's float64): anomalies within
5e-5 absolute (they lie in [-1, 1]); blend weights within 1e-5 relative;
scores within 5e-5 absolute wherever both sides route a token the same way --
a token may route differently only when the oracle's surprise lies within
1e-4 of the threshold.  Cases: fp32 and bf16, d 64 and 128, ragged batches,
several layers, sequences shorter than the window and than the block count,
a one-token sequence, long sequences with several tiles per block, bursts of
near-identical keys, and the Llama-2-7B-shaped layer at full size.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from gpu_helpers import note, threads, to_dev

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


def _keys(seqlens, L, Hkv, d, dtype, seed, bursts=True):
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    k = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    if bursts and T > 40:
        for st in rng.integers(0, T - 30, size=max(1, T // 300)):
            ln = int(rng.integers(4, 30))
            k[:, :, st:st + ln] = k[:, :, st:st + 1] + 0.2 * rng.standard_normal((L, Hkv, ln, d),
                                                                                 dtype=np.float32)
    return S.round_bf16(k) if dtype == "bf16" else k


def _check(k, seqlens, dtype, nblocks=32, prior=(0.0, 0.0, 0.0), theta=0.1):
    s_g, an_g, wt_g = hk.hubkv_nestedkv(to_dev(k, dtype), seqlens, nblocks=nblocks,
                                        log_prior=prior, theta=theta, want_parts=True)
    torch.cuda.synchronize()
    s_o, an_o, wt_o = oracle.nestedkv(k, seqlens, nblocks, 64, prior, theta, want_parts=True)
    an_g, wt_g, s_g = an_g.cpu().numpy(), wt_g.cpu().numpy(), s_g.cpu().numpy()
    np.testing.assert_allclose(an_g, an_o, rtol=0, atol=5e-5)
    np.testing.assert_allclose(wt_g, wt_o, rtol=1e-5, atol=1e-7)
    sg_o = an_o.astype(np.float64).std(axis=-1)
    near = np.abs(sg_o - theta) < 1e-4
    err = np.abs(s_g.astype(np.float64) - s_o)
    assert np.all((err <= 5e-5) | near), f"max score error {err[~near].max()}"
    assert near.mean() < 0.01
    return s_g


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_ragged_layers(dtype, d):
    seqlens = [5000, 1500, 300]
    k = _keys(seqlens, 2, 2, d, dtype, seed=d)
    _check(k, seqlens, dtype, prior=(0.2, -0.1, 0.0))


def test_short_sequences_and_block_counts():
    # shorter than the window, fewer keys than blocks, a single key
    seqlens = [40, 7, 1, 64, 65, 200]
    k = _keys(seqlens, 1, 3, 64, "f32", seed=3)
    _check(k, seqlens, "f32", nblocks=32)
    _check(k, seqlens, "f32", nblocks=1)
    _check(k, seqlens, "f32", nblocks=200)


def test_long_blocks_several_tiles():
    # blocks of 2048 keys: two tiles per block, waves running past tile edges
    seqlens = [65536]
    k = _keys(seqlens, 1, 2, 128, "bf16", seed=5)
    _check(k, seqlens, "bf16", nblocks=32, theta=0.15)


def test_routing_extremes_and_zero_keys():
    seqlens = [3000]
    k = _keys(seqlens, 1, 2, 128, "f32", seed=6)
    k[0, 0, 100:110] = 0.0                      # zero keys: every anomaly 0
    _check(k, seqlens, "f32", theta=10.0)       # always the blend
    _check(k, seqlens, "f32", theta=-1.0)       # always the largest anomaly


def test_llama2_7b_layer_full_size():
    w = S.workload(2)
    note("  drawing the 32 x 32768 x 128 keys")
    _, K, _ = S.prefill_layer_inputs(w, 0, with_v=False, threads=threads())
    _check(K[None], list(w.seqlens), "bf16")


def test_nestedkv_then_layer_budget():
    # the key-only score feeding the layer-wide allocation (the NestedKV
    # page's head-wise memory allocation): kept sets bit-exact given the GPU's
    # scores
    seqlens = [6000, 2500]
    L, Hkv = 1, 4
    k = _keys(seqlens, L, Hkv, 128, "bf16", seed=8)
    s = hk.hubkv_nestedkv(to_dev(k, "bf16"), seqlens)
    lk = [[int(0.2 * n) * Hkv for n in seqlens]]
    idx_g, hk_g = hk.hubkv_select_layer(s, seqlens, lk, 4, 64, 32)
    torch.cuda.synchronize()
    idx_o, hk_o = oracle.select_layer(s.cpu().numpy(), seqlens, lk, 4, 64, 32)
    np.testing.assert_array_equal(hk_g.cpu().numpy(), hk_o)
    np.testing.assert_array_equal(idx_g.cpu().numpy(), idx_o)
