"""Python access to the plain C CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports or calls it, and
it imports nothing from the GPU library.  Inputs are float32 host arrays (bf16
data are passed as their exact float32 widening).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at deliberately broken builds of oracle.c to
# show that the pins catch each planted mistake.
_LIB_OVERRIDE = os.environ.get("HUBKV_ORACLE_LIB")

_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-std=c99", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
_CLANG = "/opt/rocm/llvm/bin/clang"


def build_sanitized() -> str:
    """The oracle built by clang with AddressSanitizer and
    UndefinedBehaviorSanitizer (no OpenMP, so one thread; FP contraction still
    off), for the test suite's memory-safety run of the host code.  The
    sanitizer runtime must be preloaded into the process that loads it."""
    tmp = _SAN_LIB + ".tmp"
    subprocess.check_call([_CLANG, "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-ffp-contract=off", "-std=c99", "-fPIC", "-shared", _SRC, "-o", tmp,
                           "-lm"])
    os.replace(tmp, _SAN_LIB)
    return _SAN_LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build()
        L = C.CDLL(path)
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_score.argtypes = [_f32p, _f32p, C.c_int, _i64p, C.c_int, C.c_int, C.c_int, C.c_int,
                                C.c_int, C.c_double, C.c_int, _f32p, _f64p]
        L.orc_head_stats.argtypes = [_f32p, C.c_int, _i64p, C.c_int, C.c_int, _f64p]
        L.orc_beta.argtypes = [_f64p, C.c_int, _i64p, C.c_int, C.c_int, C.c_float, C.c_float, _f32p]
        L.orc_refine.argtypes = [_f32p, _f32p, C.c_int, _i64p, C.c_int, C.c_int, _f32p, C.c_int,
                                 C.c_float, C.c_float]
        L.orc_protected_count.argtypes = [C.c_int64, C.c_int, C.c_int]
        L.orc_protected_count.restype = C.c_int64
        L.orc_select.argtypes = [_f32p, C.c_int, _i64p, C.c_int, C.c_int, _i64p, C.c_int, C.c_int,
                                 _i32p]
        L.orc_select_layer.argtypes = [_f32p, C.c_int, _i64p, C.c_int, C.c_int, _i64p, C.c_int,
                                       C.c_int, C.c_int, _i32p, _i32p]
        L.orc_nestedkv.argtypes = [_f32p, C.c_int, _i64p, C.c_int, C.c_int, C.c_int, C.c_int,
                                   C.c_int, C.c_void_p, C.c_double, _f32p, C.c_void_p, C.c_void_p]
        L.orc_compact_layer.argtypes = [C.c_void_p, C.c_void_p, _i32p, _i32p, C.c_int, C.c_int,
                                        _i64p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_compact.argtypes = [C.c_void_p, C.c_void_p, _i32p, C.c_int, C.c_int, _i64p, _i64p,
                                  C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.orc_h2o_step.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _f32p, _i32p, _i64p, C.c_int,
                                   C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_double,
                                   C.c_int, _i32p, C.c_void_p, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (status {rc})")


def score(q, k, seqlens, W, scale, causal=True):
    """q [L][Hq][B*W][d], k [L][Hkv][T][d] -> s [L][Hkv][T] fp32, stats [L][B][Hkv][2]."""
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    L, Hq, BW, d = q.shape
    _, Hkv, T, _ = k.shape
    sl = _c(seqlens, np.int64)
    B = sl.size
    s = np.zeros((L, Hkv, T), np.float32)
    st = np.zeros((L, B, Hkv, 2), np.float64)
    _check(lib().orc_score(q, k, B, sl, L, Hq, Hkv, W, d, float(scale), int(bool(causal)), s, st))
    return s, st


def head_stats(s, seqlens):
    s = _c(s, np.float32)
    L, Hkv, T = s.shape
    sl = _c(seqlens, np.int64)
    st = np.zeros((L, sl.size, Hkv, 2), np.float64)
    _check(lib().orc_head_stats(s, sl.size, sl, L, Hkv, st))
    return st


def beta(stats, seqlens, beta_lo=0.8, beta_hi=1.2):
    st = _c(stats, np.float64)
    L, B, Hkv, _ = st.shape
    out = np.zeros((L, B, Hkv), np.float32)
    _check(lib().orc_beta(st, B, _c(seqlens, np.int64), L, Hkv, beta_lo, beta_hi, out))
    return out


def refine(s, seqlens, beta_arr, pool=5, gamma=0.5, r=0.1):
    s = _c(s, np.float32)
    L, Hkv, T = s.shape
    sl = _c(seqlens, np.int64)
    z = np.zeros_like(s)
    _check(lib().orc_refine(s, z, sl.size, sl, L, Hkv, _c(beta_arr, np.float32), pool,
                            float(gamma), float(r)))
    return z


def protected_count(N, n_sink, n_recent):
    return int(lib().orc_protected_count(int(N), int(n_sink), int(n_recent)))


def select(z, seqlens, kept, n_sink, n_recent):
    z = _c(z, np.float32)
    L, Hkv, T = z.shape
    sl = _c(seqlens, np.int64)
    kp = _c(kept, np.int64)
    idx = np.zeros((L, Hkv, int(kp.sum())), np.int32)
    _check(lib().orc_select(z, sl.size, sl, L, Hkv, kp, int(n_sink), int(n_recent), idx))
    return idx


def nestedkv(k, seqlens, nblocks=32, window=64, log_prior=(0.0, 0.0, 0.0), theta=0.1,
             want_parts=False):
    """NestedKV key-only score: k float32 [L][Hkv][T][d] -> s [L][Hkv][T]; with
    want_parts also the anomalies [L][Hkv][T][3] (stable, episodic, current)
    and the blend weights [L][B][Hkv][3]."""
    k = _c(k, np.float32)
    L, Hkv, T, d = k.shape
    sl = _c(seqlens, np.int64)
    s = np.zeros((L, Hkv, T), np.float32)
    lp = np.ascontiguousarray(log_prior, np.float64)
    an = np.zeros((L, Hkv, T, 3), np.float32) if want_parts else None
    wt = np.zeros((L, sl.size, Hkv, 3), np.float32) if want_parts else None
    _check(lib().orc_nestedkv(k, sl.size, sl, L, Hkv, d, int(nblocks), int(window), lp.ctypes.data,
                              float(theta), s, an.ctypes.data if an is not None else None,
                              wt.ctypes.data if wt is not None else None))
    return (s, an, wt) if want_parts else s


def select_layer(z, seqlens, layer_kept, n_sink, n_recent, floor_min):
    """Layer-wide budget: z [L][Hkv][T], layer_kept [L][B] (kept total over the
    layer's heads per sequence).  Returns (idx [sum layer_kept], head_kept
    [L][B][Hkv]); idx holds, per (layer, sequence), the heads' ascending
    positions one head after the other."""
    z = _c(z, np.float32)
    L, Hkv, T = z.shape
    sl = _c(seqlens, np.int64)
    lk = _c(np.asarray(layer_kept, np.int64).reshape(L, sl.size), np.int64)
    idx = np.zeros(int(lk.sum()), np.int32)
    hk = np.zeros((L, sl.size, Hkv), np.int32)
    _check(lib().orc_select_layer(z, sl.size, sl, L, Hkv, lk, int(n_sink), int(n_recent),
                                  int(floor_min), idx, hk))
    return idx, hk


def compact_layer(k_in, v_in, idx, head_kept, seqlens):
    """Rows of a layer-wide selection: k_in/v_in [L][Hkv][T][d] (bit copy) ->
    [sum of kept][d]."""
    k_in = np.ascontiguousarray(k_in)
    v_in = np.ascontiguousarray(v_in)
    L, Hkv, T, d = k_in.shape
    hk = _c(head_kept, np.int32)
    K = int(hk.sum())
    ko = np.empty((K, d), k_in.dtype)
    vo = np.empty((K, d), v_in.dtype)
    sl = _c(seqlens, np.int64)
    _check(lib().orc_compact_layer(k_in.ctypes.data, v_in.ctypes.data, _c(idx, np.int32), hk,
                                   k_in.dtype.itemsize, sl.size, sl, L, Hkv, d, ko.ctypes.data,
                                   vo.ctypes.data))
    return ko, vo


def compact(k_in, v_in, idx, seqlens, kept):
    """k_in/v_in [L][Hkv][T][d] of any 2- or 4-byte dtype (bit copy)."""
    k_in = np.ascontiguousarray(k_in)
    v_in = np.ascontiguousarray(v_in)
    L, Hkv, T, d = k_in.shape
    kp = _c(kept, np.int64)
    K = int(kp.sum())
    ko = np.empty((L, Hkv, K, d), k_in.dtype)
    vo = np.empty((L, Hkv, K, d), v_in.dtype)
    sl = _c(seqlens, np.int64)
    _check(lib().orc_compact(k_in.ctypes.data, v_in.ctypes.data, _c(idx, np.int32),
                             k_in.dtype.itemsize, sl.size, sl, kp, L, Hkv, d,
                             ko.ctypes.data, vo.ctypes.data))
    return ko, vo


def h2o_step(state: dict, q, k_new, v_new, t, scale, n_sink=0, n_recent=0, include_self=0,
             want_probs=False, want_margin=False, want_out=False):
    """One streaming step in place on state = {K, V [B][Hkv][C][d], acc, pos}.
    Returns evicted [B][Hkv] (and probs [B][Hq][C+1], margin [B][Hkv], the
    attention output [B][Hq][d] on request, in that order)."""
    K, V, acc, pos = state["K"], state["V"], state["acc"], state["pos"]
    for a, dt in ((K, np.float32), (V, np.float32), (acc, np.float32), (pos, np.int32)):
        assert a.dtype == dt and a.flags.c_contiguous
    B, Hkv, Cs, d = K.shape
    q = _c(q, np.float32)
    Hq = q.shape[1]
    tt = np.broadcast_to(np.asarray(t, np.int64), (B,)).copy()
    ev = np.zeros((B, Hkv), np.int32)
    probs = np.zeros((B, Hq, Cs + 1), np.float32) if want_probs else None
    margin = np.zeros((B, Hkv), np.float32) if want_margin else None
    att = np.zeros((B, Hq, d), np.float32) if want_out else None
    _check(lib().orc_h2o_step(q, _c(k_new, np.float32), _c(v_new, np.float32), K, V, acc, pos, tt,
                              B, Hq, Hkv, d, Cs, int(n_sink), int(n_recent), float(scale),
                              int(include_self), ev,
                              probs.ctypes.data if probs is not None else None,
                              margin.ctypes.data if margin is not None else None,
                              att.ctypes.data if att is not None else None))
    out = [ev]
    if want_probs:
        out.append(probs)
    if want_margin:
        out.append(margin)
    if want_out:
        out.append(att)
    return out[0] if len(out) == 1 else tuple(out)


def empty_state(B, Hkv, C, d):
    return dict(K=np.zeros((B, Hkv, C, d), np.float32), V=np.zeros((B, Hkv, C, d), np.float32),
                acc=np.zeros((B, Hkv, C), np.float32), pos=np.full((B, Hkv, C), -1, np.int32))


def prefill_chain(Q, K, V, w, budget: Optional[float] = None, r: Optional[float] = None,
                  beta_in=None):
    """The whole prefill path on the oracle: score -> beta -> refine -> select
    -> compact.  Q/K/V float32 [L][...]; returns a dict of every intermediate."""
    s, st = score(Q, K, w.seqlens, w.W, w.scale, w.causal)
    bt = beta(st, w.seqlens, w.beta_lo, w.beta_hi) if beta_in is None else beta_in
    z = refine(s, w.seqlens, bt, w.pool, w.gamma, w.r if r is None else r)
    kept = w.kept(budget)
    idx = select(z, w.seqlens, kept, w.n_sink, w.n_recent)
    ko, vo = compact(K, V, idx, w.seqlens, kept)
    return dict(s=s, stats=st, beta=bt, z=z, kept=kept, idx=idx, k_out=ko, v_out=vo)
