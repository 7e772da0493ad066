"""The allocation-free score entry point (hubkv_score_noalloc) against
hubkv_score on a caller workspace, through the C ABI.

hubkv_score_noalloc runs the same kernels on a fixed scratch array the
library holds per device, so its scores and head statistics must equal
hubkv_score's bit for bit.  Two calls in a row, the second on a smaller
problem, check that nothing the first call left in the shared array leaks
into the second (the array is never cleared between calls).
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


def _inputs(seqlens, L, Hq, Hkv, W, d, dtype, seed):
    rng = np.random.default_rng(seed)
    T = sum(seqlens)
    Q = rng.standard_normal((L, Hq, len(seqlens) * W, d), dtype=np.float32)
    K = rng.standard_normal((L, Hkv, T, d), dtype=np.float32) * 1.5
    if dtype == "bf16":
        Q, K = S.round_bf16(Q), S.round_bf16(K)
    return to_dev(Q, dtype), to_dev(K, dtype)


# each row: seqlens, L, Hq, Hkv, W, d, dtype; consecutive calls share the
# library's scratch, the later ones smaller than the earlier ones
SEQUENCE = [
    ([32768], 1, 32, 32, 64, 128, "bf16"),          # Llama-2-7B-shaped layer
    ([3000, 700, 1200], 2, 16, 4, 64, 128, "bf16"),  # smaller, ragged, 256 rows
    ([5000], 1, 4, 1, 128, 64, "bf16"),             # 512 rows, d = 64
    ([700, 260], 2, 6, 2, 20, 128, "f32"),           # fp32 VALU path
    ([300], 1, 2, 2, 16, 128, "bf16"),              # smallest
]


def test_noalloc_score_equals_workspace_score():
    for i, (seqlens, L, Hq, Hkv, W, d, dtype) in enumerate(SEQUENCE):
        note(f"  noalloc call {i}: seqlens {seqlens} L {L} Hq {Hq} Hkv {Hkv} W {W} d {d} {dtype}")
        nb = hk.lib().hubkv_score_workspace(len(seqlens), hk._arr64(seqlens), L, Hq, Hkv, W, d,
                                            1 if dtype == "bf16" else 0)
        assert 0 < nb <= (16 << 20)
        Qd, Kd = _inputs(seqlens, L, Hq, Hkv, W, d, dtype, seed=100 + i)
        scale = 1 / math.sqrt(d)
        s_w, st_w = hk.hubkv_score(Qd, Kd, seqlens, W, scale, True)
        s_n, st_n = hk.hubkv_score_noalloc(Qd, Kd, seqlens, W, scale, True)
        torch.cuda.synchronize()
        assert not torch.isnan(s_n).any() and not torch.isnan(st_n).any()
        assert torch.equal(s_n, s_w), i
        assert torch.equal(st_n, st_w), i
        # a second noalloc call on the same inputs into fresh outputs is identical too
        s_n2, st_n2 = hk.hubkv_score_noalloc(Qd, Kd, seqlens, W, scale, True)
        torch.cuda.synchronize()
        assert torch.equal(s_n2, s_w) and torch.equal(st_n2, st_w), i


def test_noalloc_score_on_a_side_stream():
    seqlens, L, Hq, Hkv, W, d = [4100, 900], 1, 8, 2, 64, 128
    Qd, Kd = _inputs(seqlens, L, Hq, Hkv, W, d, "bf16", seed=7)
    s_w, st_w = hk.hubkv_score(Qd, Kd, seqlens, W, 0.088, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    s_n, st_n = hk.hubkv_score_noalloc(Qd, Kd, seqlens, W, 0.088, True, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(s_n, s_w) and torch.equal(st_n, st_w)
