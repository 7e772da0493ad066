"""GPU checks of the strided entry points (hubkv_score_strided,
hubkv_compact_strided) through the C ABI.

A strided call runs the same kernels with the same arithmetic order as the
packed call, only the addresses differ, so its results must equal the packed
call's bit for bit on token-major, padded, broadcast and shared-buffer views;
the packed results are themselves checked against the oracle (once more here
at the score tolerance).  Compaction into the front of a larger cache must
leave every row beyond the kept rows untouched.
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


def _token_major(x):
    """[L][H][R][d] contiguous copy laid out [L][R][H][d], returned as a
    [L][H][R][d] view."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def _padded(x, extra_rows, extra_cols):
    """Copy of x inside a larger zero buffer (more rows per head, longer
    rows), returned as a view of x's shape."""
    L, H, R, d = x.shape
    buf = torch.zeros((L, H, R + extra_rows, d + extra_cols), dtype=x.dtype, device=x.device)
    v = buf[:, :, :R, :d]
    v.copy_(x)
    return v


SCORE_CASES = [
    # dtype, seqlens, L, Hq, Hkv, W, d, causal
    ("bf16", [3000, 700, 1200], 1, 32, 8, 64, 128, True),  # 256 rows per KV head
    ("bf16", [1500, 2100], 2, 4, 2, 24, 64, True),         # GQA, two layers, d = 64
    ("bf16", [4100], 1, 4, 1, 128, 128, True),             # 512 rows, the widest group
    ("f32", [700, 260], 2, 6, 2, 20, 128, True),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: f"{c[0]}-N{c[1][0]}-L{c[2]}-G{c[3]//c[4]}-W{c[5]}-d{c[6]}")
def test_score_views_bitexact(case):
    dtype, seqlens, L, Hq, Hkv, W, d, causal = case
    rng = np.random.default_rng(11 + W)
    T = sum(seqlens)
    Q = rng.standard_normal((L, Hq, len(seqlens) * W, d), dtype=np.float32)
    K = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    if dtype == "bf16":
        Q, K = S.round_bf16(Q), S.round_bf16(K)
    scale = 1 / math.sqrt(d)
    Qd, Kd = to_dev(Q, dtype), to_dev(K, dtype)
    s0, st0 = hk.hubkv_score(Qd, Kd, seqlens, W, scale, causal)
    pad_cols = 8 if dtype == "bf16" else 4  # keeps rows 16-byte aligned
    views = {
        "token-major": (_token_major(Qd), _token_major(Kd)),
        "padded": (_padded(Qd, 5, pad_cols), _padded(Kd, 37, 2 * pad_cols)),
        "mixed": (_token_major(Qd), _padded(Kd, 0, pad_cols)),
    }
    for name, (qv, kv) in views.items():
        assert not (qv.is_contiguous() and kv.is_contiguous())
        s1, st1 = hk.hubkv_score(qv, kv, seqlens, W, scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(s1, s0), name
        assert torch.equal(st1, st0), name
    s_o, _ = oracle.score(Q, K, seqlens, W, scale, causal)
    assert rel_err(s0.cpu().numpy(), s_o).max() < (5e-5 if dtype == "bf16" else 1e-5)


def test_score_broadcast_queries_over_layers():
    """A layer stride of 0 reads the same queries in every layer."""
    seqlens, L, Hq, Hkv, W, d = [2000, 900], 3, 8, 2, 32, 128
    rng = np.random.default_rng(5)
    Q1 = S.round_bf16(rng.standard_normal((1, Hq, len(seqlens) * W, d), dtype=np.float32))
    K = S.round_bf16(rng.standard_normal((L, Hkv, sum(seqlens), d), dtype=np.float32))
    Kd = to_dev(K, "bf16")
    qv = to_dev(Q1, "bf16").expand(L, -1, -1, -1)
    assert qv.stride(0) == 0
    s1, _ = hk.hubkv_score(qv, Kd, seqlens, W, 0.088, True)
    s0, _ = hk.hubkv_score(qv.contiguous(), Kd, seqlens, W, 0.088, True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s0)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_compact_views_bitexact(dtype, d):
    seqlens = [3000, 517, 1200]
    L, Hkv = 2, 3
    T = sum(seqlens)
    rng = np.random.default_rng(40 + d)
    K = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    V = rng.standard_normal((L, Hkv, T, d), dtype=np.float32)
    if dtype == "bf16":
        K, V = S.round_bf16(K), S.round_bf16(V)
    z = S.random_scores(seqlens, L, Hkv, seed=6)
    kept = S.budgets(seqlens, 0.2)
    Kt = int(sum(kept))
    idx = torch.from_numpy(oracle.select(z, seqlens, kept, 4, 32)).cuda()
    Kd, Vd = to_dev(K, dtype), to_dev(V, dtype)
    k0, v0 = hk.hubkv_compact(Kd, Vd, idx, seqlens, kept)

    # inputs: token-major K, and V sharing one buffer with K ([L][2][Hkv][T][d])
    kv = torch.stack([Kd, Vd], dim=1)
    # outputs: the first Kt rows of caches with room for 2 * Kt rows per head,
    # and a token-major output
    cap = 2 * Kt
    kc = torch.full((L, Hkv, cap, d), 7.0, dtype=Kd.dtype, device=Kd.device)
    vc = torch.full((L, Hkv, cap, d), -3.0, dtype=Kd.dtype, device=Kd.device)
    k1, v1 = hk.hubkv_compact(_token_major(Kd), kv[:, 1], idx, seqlens, kept,
                              k_out=kc[:, :, :Kt], v_out=vc[:, :, :Kt])
    k2 = torch.full((L, Kt, Hkv, d), float("nan"), dtype=Kd.dtype,
                    device=Kd.device).permute(0, 2, 1, 3)
    v2 = torch.full((L, Kt, Hkv, d), float("nan"), dtype=Kd.dtype,
                    device=Kd.device).permute(0, 2, 1, 3)
    hk.hubkv_compact(kv[:, 0], _padded(Vd, 11, 8), idx, seqlens, kept, k_out=k2, v_out=v2)
    torch.cuda.synchronize()
    assert torch.equal(k1, k0) and torch.equal(v1, v0)
    assert torch.equal(k2, k0) and torch.equal(v2, v0)
    assert bool((kc[:, :, Kt:] == 7.0).all()) and bool((vc[:, :, Kt:] == -3.0).all())
    ko, vo = oracle.compact(K, V, idx.cpu().numpy(), seqlens, kept)
    np.testing.assert_array_equal(to_host(k0), ko)
    np.testing.assert_array_equal(to_host(v0), vo)


def test_strided_rejects_bad_views():
    """Host validation: a view whose last axis is not contiguous is refused by
    the binding; overlapping output rows by the library."""
    seqlens, L, Hkv, d = [600], 1, 2, 64
    K = torch.zeros((L, Hkv, 600, d), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((L, Hkv, 100), dtype=torch.int32, device="cuda")
    col_major = K.transpose(2, 3).contiguous().transpose(2, 3)  # same shape, d axis strided
    assert col_major.stride(3) != 1
    with pytest.raises(ValueError):
        hk.hubkv_compact(col_major, K, idx, seqlens, [100])
    out = torch.empty((L, Hkv, 1, d), dtype=K.dtype, device="cuda").expand(L, Hkv, 100, d)
    with pytest.raises(hk.HubkvError) as e:
        hk.hubkv_compact(K, K, idx, seqlens, [100], k_out=out, v_out=out.contiguous())
    assert e.value.status == -1
