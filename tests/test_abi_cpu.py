"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/hubkv.h declares, and
reject invalid arguments on the host before anything reaches the GPU.  The
calls below that pass non-null fake pointers always carry some invalid
argument, so validation returns before any HIP call is made.
"""
import ctypes as C

import numpy as np
import pytest

import oracle
import token_scoring_top_amd as hk

EINVAL, EDTYPE, EALIGN, EWS = -1, -2, -3, -4
P = 0x10000  # fake, 256-aligned "device" pointer; never dereferenced


def a64(xs):
    return (C.c_int64 * len(xs))(*xs)


def test_library_exports_every_declared_function():
    L = hk.lib()
    names = hk.header_functions()
    assert {"hubkv_score", "hubkv_refine", "hubkv_select", "hubkv_compact", "h2o_step"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.hubkv_version() >= 100


def test_library_exports_nothing_else():
    """Every global function symbol of the library is one the header declares
    (internal helpers have internal linkage)."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", hk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines()
                if len(ln.split()) == 3 and ln.split()[1] == "T"}
    ours = {n for n in exported if n.startswith(("hubkv", "h2o"))}
    assert ours == set(hk.header_functions()) & ours
    assert ours >= {n for n in hk.header_functions() if n.startswith(("hubkv", "h2o"))}
    assert not {n for n in exported if not n.startswith("_")} - ours


def test_strerror_and_last_error():
    L = hk.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.hubkv_strerror(code)
    assert L.hubkv_last_hip_error() == 0


def test_protected_count_matches_oracle():
    for N in (1, 5, 20, 100, 4096):
        for ns in (0, 1, 4, 50):
            for nr in (0, 3, 64, 200):
                assert hk.protected_count(N, ns, nr) == oracle.protected_count(N, ns, nr)


def test_workspace_queries():
    L = hk.lib()
    sl = a64([32768])
    assert L.hubkv_score_workspace(1, sl, 1, 32, 32, 64, 128, 1) > 0
    assert L.hubkv_score_workspace(1, sl, 1, 32, 32, 64, 96, 1) == 0      # bad d
    assert L.hubkv_score_workspace(1, sl, 1, 32, 8, 256, 128, 1) == 0     # G*W > 512
    assert L.hubkv_score_workspace(1, a64([10]), 1, 4, 4, 32, 64, 0) == 0  # W > N
    assert L.hubkv_refine_workspace(1, sl, 1, 32) > 0
    assert L.hubkv_refine_workspace(0, sl, 1, 32) == 0


def test_score_validation():
    L = hk.lib()
    sl = a64([512])
    big = 1 << 30
    ok = dict(q=P, k=P, dt=0, B=1, sl=sl, L=1, Hq=4, Hkv=4, W=32, d=64, scale=0.125, causal=1,
              s=P, st=P, ws=P, wsb=big, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return L.hubkv_score(a["q"], a["k"], a["dt"], a["B"], a["sl"], a["L"], a["Hq"], a["Hkv"],
                             a["W"], a["d"], a["scale"], a["causal"], a["s"], a["st"], a["ws"],
                             a["wsb"], a["stream"])

    assert call(dt=7) == EDTYPE
    assert call(d=96) == EDTYPE
    assert call(Hq=6) == EINVAL                      # Hq % Hkv
    assert call(W=600) == EINVAL                     # W > N
    assert call(B=0) == EINVAL
    assert call(B=65, sl=a64([512] * 65)) == EINVAL  # more than 64 sequences
    assert call(sl=a64([0])) == EINVAL
    assert call(scale=float("nan")) == EINVAL
    assert call(Hq=32, Hkv=2, W=128, sl=a64([4096])) == EINVAL  # G*W = 2048 > 512
    assert call(q=None) == EALIGN
    assert call(k=P + 8) == EALIGN
    assert call(s=P + 2) == EALIGN
    assert call(ws=None) == EWS
    assert call(wsb=16) == EWS


def test_refine_validation():
    L = hk.lib()
    sl = a64([1000])
    ok = dict(s=P, B=1, sl=sl, L=1, Hkv=2, st=None, bi=None, pool=5, gamma=0.5, lo=0.8, hi=1.2,
              r=0.1, z=P + (1 << 20), bo=None, ws=P + (1 << 24), wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.hubkv_refine(a["s"], a["B"], a["sl"], a["L"], a["Hkv"], a["st"], a["bi"],
                              a["pool"], a["gamma"], a["lo"], a["hi"], a["r"], a["z"], a["bo"],
                              a["ws"], a["wsb"], None)

    assert call(pool=4) == EINVAL
    assert call(pool=0) == EINVAL
    assert call(pool=65) == EINVAL
    assert call(gamma=0.0) == EINVAL
    assert call(gamma=1.5) == EINVAL
    assert call(lo=1.3) == EINVAL
    assert call(r=-0.1) == EINVAL
    assert call(r=1.5) == EINVAL
    assert call(z=P) == EINVAL           # z aliases s
    assert call(z=P + 400) == EINVAL     # overlapping ranges
    assert call(s=None) == EALIGN
    assert call(z=P + (1 << 20) + 2) == EALIGN
    assert call(wsb=8) == EWS


def test_select_validation():
    L = hk.lib()
    sl = a64([100, 50])

    def call(kept, ns=4, nr=16, z=P, idx=P + 4096, B=2, s=sl, ws=P, wsb=1 << 30):
        return L.hubkv_select(z, B, s, 1, 2, a64(kept), ns, nr, idx, ws, wsb, None)

    assert call([10, 30]) == EINVAL    # fewer than the 20 protected tokens
    assert call([30, 51]) == EINVAL    # more than the sequence
    assert call([30, 30], ns=-1) == EINVAL
    assert call([30, 30], z=None) == EALIGN
    assert call([30, 30], idx=P + 2) == EALIGN
    assert call([30, 30], ws=None) == EWS
    assert call([30, 30], wsb=16) == EWS
    assert call([30, 30], ws=P + 8) == EALIGN
    nb = L.hubkv_select_workspace(2, sl, 1, 2)
    assert nb > 0 and call([30, 30], wsb=nb - 1) == EWS
    # per slice: a 256-byte head record, 4096 16-bit bin starts, 4096 sorted keys
    per_slice = 256 + 4096 * 2 + 4096 * 4
    four = a64([3000, 5000, 131, 20000])   # 1 + 2 + 1 + 5 slices
    assert L.hubkv_select_workspace(4, four, 7, 9) == 7 * 9 * 9 * per_slice
    # 256 (layer, head, sequence) units fill the chip: one work-group per
    # unit, no slices, and the workspace shrinks to one aligned block
    assert L.hubkv_select_workspace(4, four, 8, 8) == 256


def test_refine_select_validation():
    L = hk.lib()
    sl = a64([100, 50])

    def call(kept=(30, 30), pool=5, gamma=0.5, r=0.1, s=P, z=P + (1 << 20), idx=P + (1 << 21),
             ws=P + (1 << 22), wsb=1 << 30, lo=0.8, hi=1.2):
        return L.hubkv_refine_select(s, 2, sl, 1, 2, None, None, pool, gamma, lo, hi, r, z, None,
                                     a64(list(kept)), 4, 16, idx, ws, wsb, None)

    assert call(kept=(10, 30)) == EINVAL
    assert call(pool=4) == EINVAL
    assert call(gamma=0.0) == EINVAL
    assert call(r=1.5) == EINVAL
    assert call(lo=1.3) == EINVAL
    assert call(z=P + 400) == EINVAL     # z overlaps s
    assert call(z=None) == EALIGN
    assert call(idx=P + (1 << 21) + 2) == EALIGN
    assert call(wsb=8) == EWS
    nb = L.hubkv_refine_select_workspace(2, sl, 1, 2)
    assert nb >= L.hubkv_select_workspace(2, sl, 1, 2)
    assert call(wsb=nb - 1) == EWS


def test_nothing_kept_writes_nothing():
    # kept = 0 everywhere (no protected tokens): the calls validate their
    # arguments, accept empty (null) row outputs, and return before any
    # launch, so they run here without a GPU
    L = hk.lib()
    sl = a64([1, 700])
    zero = a64([0, 0])
    nb = L.hubkv_select_workspace(2, sl, 2, 3)
    assert L.hubkv_select(P, 2, sl, 2, 3, zero, 0, 0, None, P, nb, None) == 0
    assert L.hubkv_select(None, 2, sl, 2, 3, zero, 0, 0, None, P, nb, None) == EALIGN
    assert L.hubkv_select(P, 2, sl, 2, 3, zero, 1, 0, None, P, nb, None) == EINVAL  # a sink must be kept
    assert L.hubkv_compact(P, P, 1, None, 2, sl, zero, 2, 3, 128, None, None, None) == 0
    assert L.hubkv_compact(P, P, 1, None, 2, sl, a64([0, 1]), 2, 3, 128, None, None, None) == EALIGN
    lk = a64([0, 0])  # L = 1, B = 2
    assert L.hubkv_compact_layer(P, P, 1, None, None, 2, sl, 1, 3, lk, 128, None, None, None) == 0


def test_compact_validation():
    L = hk.lib()
    sl = a64([100])

    def call(dt=1, d=128, kept=(10,), ki=P, ko=P + 65536):
        return L.hubkv_compact(ki, P, dt, P, 1, sl, a64(list(kept)), 1, 2, d, ko, P + 131072, None)

    assert call(dt=3) == EDTYPE
    assert call(d=32) == EDTYPE
    assert call(kept=(101,)) == EINVAL
    assert call(kept=(-1,)) == EINVAL
    assert call(ki=P + 8) == EALIGN
    assert call(ko=None) == EALIGN


def test_select_layer_validation():
    L = hk.lib()
    sl = a64([1000])
    ws = L.hubkv_select_layer_workspace(1, sl, 2, 4)
    assert ws > 0
    assert L.hubkv_select_layer_workspace(1, sl, 300, 4) == 0            # L * B > 256

    def call(lk=(500, 500), Lr=2, Hkv=4, ns=4, nr=16, fl=10, idx=P, wsb=ws, seq=(1000,)):
        return L.hubkv_select_layer(P, len(seq), a64(list(seq)), Lr, Hkv, a64(list(lk)), ns, nr,
                                    fl, idx, P, P, wsb, None)

    # per-head floor: 4 heads x (20 protected + 10) = 120 at least, 4000 at most
    assert call(lk=(119, 500)) == EINVAL
    assert call(lk=(500, 4001)) == EINVAL
    assert call(fl=-1) == EINVAL
    assert call(Lr=300, lk=(500,) * 300) == EINVAL
    assert call(idx=P + 2, lk=(120, 4000)) == EALIGN
    assert call(wsb=ws - 1, lk=(120, 4000)) == EWS
    assert call(idx=None, lk=(120, 4000)) == EALIGN


def test_compact_layer_validation():
    L = hk.lib()

    def call(dt=1, d=128, lk=(300,), Hkv=4, ko=P):
        return L.hubkv_compact_layer(P, P, dt, P, P, 1, a64([100]), 1, Hkv, a64(list(lk)), d, ko,
                                     P, None)

    assert call(d=96) == EDTYPE
    assert call(dt=7) == EDTYPE
    assert call(lk=(401,)) == EINVAL                                      # above Hkv * N
    assert call(ko=P + 8) == EALIGN


def test_h2o_step_validation():
    L = hk.lib()

    def call(C_=64, ns=0, nr=8, Hq=4, Hkv=4, t=(100,), d=128, dt=1, acc=P, scale=0.1):
        return L.h2o_step(P, P, P, dt, P, P, acc, P, a64(list(t)), len(t), Hq, Hkv, d, C_, ns, nr,
                          scale, 0, None, None, None, None)

    assert call(ns=60, nr=8) == EINVAL       # protected windows exceed the capacity
    assert call(Hq=6) == EINVAL
    assert call(Hq=64, Hkv=2) == EINVAL      # group of 32 query heads
    assert call(C_=20000) == EINVAL          # logits do not fit the work-group
    assert call(t=(-1,)) == EINVAL
    assert call(d=80) == EDTYPE
    assert call(dt=5) == EDTYPE
    assert call(acc=P + 2) == EALIGN
    assert call(scale=float("inf")) == EINVAL


def test_python_binding_raises_on_missing_library(monkeypatch, tmp_path):
    import importlib
    monkeypatch.setattr(hk, "_lib", None)
    monkeypatch.setattr(hk, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        hk.lib()


def test_score_strided_validation():
    L = hk.lib()
    sl = a64([512])
    d, Hq, Hkv, W = 64, 4, 2, 32
    qs_ok = [Hq * W * d, W * d, d]
    ks_ok = [Hkv * 512 * d, 512 * d, d]

    def call(qs=qs_ok, ks=ks_ok, dt=1, ws=None):
        q = None if qs is None else a64(qs)
        k = None if ks is None else a64(ks)
        return L.hubkv_score_strided(P, q, P, k, dt, 1, sl, 1, Hq, Hkv, W, d, 0.125, 1, P, P,
                                     ws, 1 << 30, None)

    # valid strides reach the workspace check (the last one before any launch)
    assert call() == EWS
    assert call(ks=[0, d, Hkv * d]) == EWS              # token-major K
    assert call(qs=[0, W * d, d]) == EWS                # queries broadcast over layers
    assert call(qs=None) == EINVAL
    assert call(ks=[0, -d, d]) == EINVAL
    assert call(ks=[0, 512 * d, 1 << 51]) == EINVAL     # stride out of range
    assert call(ks=[0, 1 << 50, 1 << 50]) == EINVAL     # offsets beyond 2^60 bytes
    assert call(ks=[0, 512 * d, d + 4]) == EALIGN       # bf16 row of 136 bytes
    assert call(ks=[0, 512 * d, d + 8]) == EWS          # 144 bytes: a 16-byte multiple
    assert call(dt=0, ks=[0, 512 * d, d + 2]) == EALIGN  # fp32 row of 264 bytes
    assert call(dt=0, ks=[0, 512 * d, d + 4]) == EWS


def test_compact_strided_validation():
    L = hk.lib()
    sl = a64([100])
    d, Hkv = 128, 2
    ins = [Hkv * 100 * d, 100 * d, d]
    outs = [Hkv * 10 * d, 10 * d, d]

    def call(ki=P, ks=ins, os_=outs, vos=outs, kept=(10,), dt=1):
        return L.hubkv_compact_strided(ki, a64(ks), P, a64(ins), dt, P, 1, sl,
                                       a64(list(kept)), 1, Hkv, d, P + (1 << 20), a64(os_),
                                       P + (1 << 21), a64(vos), None)

    # every stride valid: the misaligned K input is the first error left
    assert call(ki=P + 8) == EALIGN
    assert call(ki=P + 8, os_=[0, d, Hkv * d]) == EALIGN    # token-major output
    assert call(ki=P + 8, os_=[0, 64 * d, d]) == EALIGN     # rows of a 64-row cache
    assert call(os_=[0, 10 * d, d - 8]) == EINVAL            # rows overlap
    assert call(os_=[0, 5 * d, d]) == EINVAL                 # heads overlap
    assert call(os_=[0, 10 * d, 0]) == EINVAL                # every row on one
    assert call(vos=[0, d, d]) == EINVAL                     # token and head strides equal
    assert call(ks=[0, 100 * d, d + 4]) == EALIGN            # 264-byte bf16 rows
    assert call(ki=P + 8, ks=[0, 0, d]) == EALIGN            # inputs may overlap (reads only)
    # nothing is kept: no output row is addressed and nothing is launched
    assert call(kept=(0,), os_=[0, 0, 0], vos=[0, 0, 0]) == 0


def test_h2o_step_ring_validation():
    L = hk.lib()

    def call(C_=64, ns=0, nr=8, acc=P):
        return L.h2o_step_ring(P, P, P, 1, P, P, acc, P, a64([100]), 1, 4, 4, 128, C_, ns, nr,
                               0.1, 0, None, None, None, None)

    # valid layouts reach the alignment check (the last one before a launch)
    assert call(acc=P + 2) == EALIGN
    assert call(C_=64, nr=63, acc=P + 2) == EALIGN   # one heavy slot
    assert call(nr=0) == EINVAL                      # no ring
    assert call(C_=8, nr=8) == EINVAL                # no heavy slot
    assert call(ns=60, nr=8) == EINVAL               # protected windows exceed the capacity
    # the fixed-slot call keeps accepting n_recent = 0 and n_recent = C
    assert L.h2o_step(P, P, P, 1, P, P, P + 2, P, a64([100]), 1, 4, 4, 128, 8, 0, 8, 0.1, 0,
                      None, None, None, None) == EALIGN


def test_sequence_length_limit():
    """Every entry point rejects a sequence of 2^30 tokens or more on the host:
    the kernels round positions up to whole tiles and select rounds in int32."""
    L = hk.lib()
    for n in ((1 << 30), (1 << 31) - 10, (1 << 31) - 1):
        sl = a64([n])
        kept = a64([n // 2])
        assert L.hubkv_select(P, 1, sl, 1, 1, kept, 0, 0, P, P, 1 << 40, None) == EINVAL
        assert L.hubkv_refine(P, 1, sl, 1, 1, None, None, 5, 0.5, 0.8, 1.2, 0.1, P + (1 << 40),
                              None, P, 1 << 40, None) == EINVAL
        assert L.hubkv_compact(P, P, 1, P, 1, sl, kept, 1, 1, 128, P, P, None) == EINVAL
        assert L.hubkv_score(P, P, 1, 1, sl, 1, 1, 1, 16, 128, 0.1, 1, P, None, P, 1 << 40,
                             None) == EINVAL
        assert L.hubkv_score_workspace(1, sl, 1, 1, 1, 16, 128, 1) == 0
        assert L.hubkv_refine_workspace(1, sl, 1, 1) == 0
        assert L.hubkv_select_layer_workspace(1, sl, 1, 1) == 0
        assert L.hubkv_nestedkv_workspace(1, sl, 1, 1, 128, 32) == 0
    # one below the limit passes the length check
    sl = a64([(1 << 30) - 1])
    assert L.hubkv_refine_workspace(1, sl, 1, 1) > 0


def test_score_noalloc_rejects_problems_beyond_its_scratch():
    """hubkv_score_noalloc refuses, on the host, a problem whose workspace
    exceeds the library's fixed scratch (HUBKV_SCORE_NOALLOC_BYTES = 16 MiB)."""
    L = hk.lib()
    ESCRATCH = -6
    assert L.hubkv_strerror(ESCRATCH)
    # 64 layers x 64 KV heads x 512 query rows: the workspace holds (m, l) per
    # row for every (layer, head, chunk)
    sl = a64([2048])
    nb = L.hubkv_score_workspace(1, sl, 64, 512, 64, 64, 128, 1)
    assert nb > (16 << 20)
    assert L.hubkv_score_noalloc(P, P, 1, 1, sl, 64, 512, 64, 64, 128, 0.1, 1, P, None,
                                 None) == ESCRATCH
    # invalid arguments are still rejected first, as hubkv_score rejects them
    assert L.hubkv_score_noalloc(P, P, 1, 1, a64([512]), 1, 4, 4, 32, 96, 0.1, 1, P, None,
                                 None) == EDTYPE
    assert L.hubkv_score_noalloc(P, P, 1, 1, a64([10]), 1, 4, 4, 32, 64, 0.1, 1, P, None,
                                 None) == EINVAL
    assert L.hubkv_score_noalloc(P + 2, P, 1, 1, a64([512]), 1, 4, 4, 32, 64, 0.1, 1, P, None,
                                 None) == EALIGN
