"""token_scoring_top_amd -- MI355X (gfx950) KV-cache retention scoring and Top-K.

Thin Python binding of libhubkv.so (include/hubkv.h).  It only marshals
arguments: torch tensors become device pointers, the given torch stream (the
current one by default) becomes the HIP stream, and outputs/workspaces the
caller does not pass are allocated with torch on that same stream, so the
caching allocator never hands their blocks to other work while the kernels
still use them.  Every step of the path runs in the library's HIP kernels;
there is no fallback, and importing the binding without the built library
raises.

Functions (names follow the C ABI):
    hubkv_score(q, k, seqlens, W, scale, causal=True) -> (s, head_stats)
    hubkv_score_noalloc(q, k, seqlens, W, scale, ...)  -> (s, head_stats), no workspace
    hubkv_refine(s, seqlens, ...)                      -> (z, beta)
    hubkv_select(z, seqlens, kept, n_sink, n_recent)   -> idx
    hubkv_refine_select(s, seqlens, kept, n_sink, n_recent, ...) -> (z, beta, idx)
    hubkv_compact(k, v, idx, seqlens, kept)            -> (k_out, v_out)
    (q, k, v and the compaction outputs may be strided views whose last
     axis is contiguous: those calls go to hubkv_score_strided and
     hubkv_compact_strided)
    hubkv_nestedkv(k, seqlens, ...)                    -> (s, anomalies, weights)
    hubkv_select_layer(z, seqlens, layer_kept, ...)    -> (idx, head_kept)
    hubkv_compact_layer(k, v, idx, head_kept, seqlens, layer_kept) -> (k_out, v_out)
    h2o_step(q, k_new, v_new, k_cache, v_cache, acc, pos, t, ...) -> evicted
    (ring=True: h2o_step_ring, the recent window in a ring of slots)
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import re
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# HUBKV_LIB names another build of the library (the test suite's sanitized
# host build); by default the in-tree libhubkv.so
LIB_PATH = os.environ.get("HUBKV_LIB") or os.path.join(HERE, "libhubkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hubkv.h")

HUBKV_F32, HUBKV_BF16 = 0, 1
STATUS = {0: "HUBKV_OK", -1: "HUBKV_EINVAL", -2: "HUBKV_EDTYPE", -3: "HUBKV_EALIGN",
          -4: "HUBKV_EWORKSPACE", -5: "HUBKV_EHIP", -6: "HUBKV_ESCRATCH"}


class HubkvError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        if status == -5:
            msg += f" (hipError {hip})"
        super().__init__(msg)


_lib = None
_vp, _i, _i64, _f, _sz = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_size_t
_i64p = C.POINTER(C.c_int64)

_SIGS = {
    "hubkv_score_workspace": (_sz, [_i, _i64p, _i, _i, _i, _i, _i, _i]),
    "hubkv_score": (_i, [_vp, _vp, _i, _i, _i64p, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _sz,
                         _vp]),
    "hubkv_refine_workspace": (_sz, [_i, _i64p, _i, _i]),
    "hubkv_refine": (_i, [_vp, _i, _i64p, _i, _i, _vp, _vp, _i, _f, _f, _f, _f, _vp, _vp, _vp, _sz,
                          _vp]),
    "hubkv_select_workspace": (_sz, [_i, _i64p, _i, _i]),
    "hubkv_select": (_i, [_vp, _i, _i64p, _i, _i, _i64p, _i, _i, _vp, _vp, _sz, _vp]),
    "hubkv_refine_select_workspace": (_sz, [_i, _i64p, _i, _i]),
    "hubkv_refine_select": (_i, [_vp, _i, _i64p, _i, _i, _vp, _vp, _i, _f, _f, _f, _f, _vp, _vp,
                                 _i64p, _i, _i, _vp, _vp, _sz, _vp]),
    "hubkv_compact": (_i, [_vp, _vp, _i, _vp, _i, _i64p, _i64p, _i, _i, _i, _vp, _vp, _vp]),
    "hubkv_score_noalloc": (_i, [_vp, _vp, _i, _i, _i64p, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                 _vp]),
    "hubkv_score_strided": (_i, [_vp, _i64p, _vp, _i64p, _i, _i, _i64p, _i, _i, _i, _i, _i, _f,
                                 _i, _vp, _vp, _vp, _sz, _vp]),
    "hubkv_compact_strided": (_i, [_vp, _i64p, _vp, _i64p, _i, _vp, _i, _i64p, _i64p, _i, _i,
                                   _i, _vp, _i64p, _vp, _i64p, _vp]),
    "hubkv_select_layer_workspace": (_sz, [_i, _i64p, _i, _i]),
    "hubkv_select_layer": (_i, [_vp, _i, _i64p, _i, _i, _i64p, _i, _i, _i, _vp, _vp, _vp, _sz,
                                _vp]),
    "hubkv_compact_layer": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i64p, _i, _i, _i64p, _i, _vp, _vp,
                                 _vp]),
    "hubkv_nestedkv_workspace": (_sz, [_i, _i64p, _i, _i, _i, _i]),
    "hubkv_nestedkv": (_i, [_vp, _i, _i, _i64p, _i, _i, _i, _i, _i, _vp, _f, _vp, _vp, _vp, _vp,
                            _sz, _vp]),
    "h2o_step": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i64p, _i, _i, _i, _i, _i, _i, _i, _f,
                      _i, _vp, _vp, _vp, _vp]),
    "h2o_step_ring": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i64p, _i, _i, _i, _i, _i, _i, _i,
                           _f, _i, _vp, _vp, _vp, _vp]),
    "hubkv_protected_count": (_i64, [_i64, _i, _i]),
    "hubkv_strerror": (C.c_char_p, [_i]),
    "hubkv_last_hip_error": (_i, []),
    "hubkv_version": (_i, []),
}


def lib():
    """The loaded libhubkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m token_scoring_top_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/hubkv.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", src)) - {"if", "sizeof"})


def _arr64(xs) -> C.Array:
    xs = [int(x) for x in xs]
    return (C.c_int64 * len(xs))(*xs)


def _check(fn: str, rc: int):
    if rc != 0:
        raise HubkvError(fn, rc, lib().hubkv_last_hip_error() if rc == -5 else 0)


# -------------------------------------------------------------------------
# torch helpers (torch is only used for device memory and streams)
# -------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return HUBKV_F32
    if t.dtype == torch.bfloat16:
        return HUBKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, view: bool = False) -> Optional[int]:
    """Device address of `t`; with view=True any layout whose last axis is
    contiguous is accepted (its strides go to a *_strided call)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if view:
        if t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1):
            raise ValueError("views must be 4-D with a contiguous last axis")
    elif not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _strides3(t) -> C.Array:
    """(layer, head, row) element strides of a 4-D view."""
    return _arr64(t.stride()[:3])


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on(stream):
    """Allocation context of a call: the launch stream when one is given (the
    caching allocator then orders reuse of the blocks after that stream's
    work), else the current stream."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


_POISON = False


def set_output_poison(on: bool) -> None:
    """When on, every output and workspace the binding allocates is filled
    before the call (NaN for floating point, -2^31 for integers, which no
    integer output of the library can hold, 0xff bytes for workspaces), so an
    element a kernel never writes cannot pass for a result.  Off by default; the GPU tests turn it on."""
    global _POISON
    _POISON = bool(on)


def _new(shape, dtype, device):
    """An output tensor on the current stream (poisoned when asked)."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if _POISON:
        t.fill_(float("nan") if t.is_floating_point() else -(1 << 31))
    return t


def _workspace(nbytes: int, device):
    torch = _torch()
    t = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if _POISON:
        t.fill_(255)
    return t


# -------------------------------------------------------------------------
# Entry points
# -------------------------------------------------------------------------
def hubkv_score(q, k, seqlens: Sequence[int], W: int, scale: float, causal: bool = True,
                s=None, head_stats=None, workspace=None, stream=None):
    """q [L][Hq][B*W][d], k [L][Hkv][T][d] (fp32 or bf16) -> s fp32 [L][Hkv][T],
    head_stats fp64 [L][B][Hkv][2]."""
    torch = _torch()
    L, Hq, BW, d = q.shape
    L2, Hkv, T, d2 = k.shape
    B = len(seqlens)
    if L2 != L or d2 != d or BW != B * W or T != sum(seqlens) or q.dtype != k.dtype:
        raise ValueError("inconsistent q/k shapes")
    sl = _arr64(seqlens)
    dt = _dtype_code(q)
    with _on(stream):
        if s is None:
            s = _new((L, Hkv, T), torch.float32, q.device)
        if head_stats is None:
            head_stats = _new((L, B, Hkv, 2), torch.float64, q.device)
        nb = lib().hubkv_score_workspace(B, sl, L, Hq, Hkv, W, d, dt)
        if workspace is None:
            workspace = _workspace(nb, q.device)
        if q.is_contiguous() and k.is_contiguous():
            _check("hubkv_score", lib().hubkv_score(_ptr(q), _ptr(k), dt, B, sl, L, Hq, Hkv, W, d,
                                                    float(scale), int(bool(causal)), _ptr(s),
                                                    _ptr(head_stats), _ptr(workspace),
                                                    workspace.numel(), _stream(stream)))
        else:
            _check("hubkv_score_strided",
                   lib().hubkv_score_strided(_ptr(q, True), _strides3(q), _ptr(k, True),
                                             _strides3(k), dt, B, sl, L, Hq, Hkv, W, d,
                                             float(scale), int(bool(causal)), _ptr(s),
                                             _ptr(head_stats), _ptr(workspace), workspace.numel(),
                                             _stream(stream)))
    return s, head_stats


def hubkv_score_noalloc(q, k, seqlens: Sequence[int], W: int, scale: float, causal: bool = True,
                        s=None, head_stats=None, stream=None):
    """hubkv_score on the library's fixed per-device scratch (no workspace,
    no allocation inside the library); q and k packed.  Outputs the caller
    does not pass are allocated here, by torch."""
    torch = _torch()
    L, Hq, BW, d = q.shape
    L2, Hkv, T, d2 = k.shape
    B = len(seqlens)
    if L2 != L or d2 != d or BW != B * W or T != sum(seqlens) or q.dtype != k.dtype:
        raise ValueError("inconsistent q/k shapes")
    with _on(stream):
        if s is None:
            s = _new((L, Hkv, T), torch.float32, q.device)
        if head_stats is None:
            head_stats = _new((L, B, Hkv, 2), torch.float64, q.device)
        _check("hubkv_score_noalloc",
               lib().hubkv_score_noalloc(_ptr(q), _ptr(k), _dtype_code(q), B, _arr64(seqlens), L,
                                         Hq, Hkv, W, d, float(scale), int(bool(causal)), _ptr(s),
                                         _ptr(head_stats), _stream(stream)))
    return s, head_stats


def hubkv_refine(s, seqlens: Sequence[int], head_stats=None, beta_in=None, pool: int = 5,
                 gamma: float = 0.5, beta_lo: float = 0.8, beta_hi: float = 1.2, r: float = 0.1,
                 z=None, beta_out=None, workspace=None, stream=None):
    """s fp32 [L][Hkv][T] -> z fp32 [L][Hkv][T], beta fp32 [L][B][Hkv]."""
    torch = _torch()
    L, Hkv, T = s.shape
    B = len(seqlens)
    sl = _arr64(seqlens)
    with _on(stream):
        if z is None:
            z = _new((L, Hkv, T), torch.float32, s.device)
        if beta_out is None:
            beta_out = _new((L, B, Hkv), torch.float32, s.device)
        nb = lib().hubkv_refine_workspace(B, sl, L, Hkv)
        if workspace is None:
            workspace = _workspace(nb, s.device)
        _check("hubkv_refine", lib().hubkv_refine(_ptr(s), B, sl, L, Hkv, _ptr(head_stats),
                                                  _ptr(beta_in), int(pool), float(gamma),
                                                  float(beta_lo), float(beta_hi), float(r),
                                                  _ptr(z), _ptr(beta_out), _ptr(workspace),
                                                  workspace.numel(), _stream(stream)))
    return z, beta_out


def hubkv_select(z, seqlens: Sequence[int], kept: Sequence[int], n_sink: int, n_recent: int,
                 idx=None, workspace=None, stream=None):
    """z fp32 [L][Hkv][T] -> idx int32 [L][Hkv][sum kept] (ascending per sequence)."""
    torch = _torch()
    L, Hkv, T = z.shape
    B = len(seqlens)
    sl = _arr64(seqlens)
    with _on(stream):
        if idx is None:
            idx = _new((L, Hkv, int(sum(kept))), torch.int32, z.device)
        if workspace is None:
            workspace = _workspace(lib().hubkv_select_workspace(B, sl, L, Hkv), z.device)
        _check("hubkv_select", lib().hubkv_select(_ptr(z), B, sl, L, Hkv, _arr64(kept),
                                                  int(n_sink), int(n_recent), _ptr(idx),
                                                  _ptr(workspace), workspace.numel(),
                                                  _stream(stream)))
    return idx


def hubkv_refine_select(s, seqlens: Sequence[int], kept: Sequence[int], n_sink: int,
                        n_recent: int, head_stats=None, beta_in=None, pool: int = 5,
                        gamma: float = 0.5, beta_lo: float = 0.8, beta_hi: float = 1.2,
                        r: float = 0.1, z=None, beta_out=None, idx=None, workspace=None,
                        stream=None):
    """hubkv_refine then hubkv_select in one call: s fp32 [L][Hkv][T] ->
    (z fp32 [L][Hkv][T], beta fp32 [L][B][Hkv], idx int32 [L][Hkv][sum kept])."""
    torch = _torch()
    L, Hkv, T = s.shape
    B = len(seqlens)
    sl = _arr64(seqlens)
    with _on(stream):
        if z is None:
            z = _new((L, Hkv, T), torch.float32, s.device)
        if beta_out is None:
            beta_out = _new((L, B, Hkv), torch.float32, s.device)
        if idx is None:
            idx = _new((L, Hkv, int(sum(kept))), torch.int32, s.device)
        if workspace is None:
            workspace = _workspace(lib().hubkv_refine_select_workspace(B, sl, L, Hkv), s.device)
        _check("hubkv_refine_select", lib().hubkv_refine_select(
            _ptr(s), B, sl, L, Hkv, _ptr(head_stats), _ptr(beta_in), int(pool), float(gamma),
            float(beta_lo), float(beta_hi), float(r), _ptr(z), _ptr(beta_out), _arr64(kept),
            int(n_sink), int(n_recent), _ptr(idx), _ptr(workspace), workspace.numel(),
            _stream(stream)))
    return z, beta_out, idx


def hubkv_compact(k_in, v_in, idx, seqlens: Sequence[int], kept: Sequence[int], k_out=None,
                  v_out=None, stream=None):
    """k_in/v_in [L][Hkv][T][d] -> k_out/v_out [L][Hkv][sum kept][d] (any of
    the four may be a view with a contiguous last axis)."""
    L, Hkv, T, d = k_in.shape
    K = int(sum(kept))
    with _on(stream):
        if k_out is None:
            k_out = _new((L, Hkv, K, d), k_in.dtype, k_in.device)
        if v_out is None:
            v_out = _new((L, Hkv, K, d), v_in.dtype, v_in.device)
        for t, shape in ((v_in, (L, Hkv, T, d)), (k_out, (L, Hkv, K, d)),
                         (v_out, (L, Hkv, K, d))):
            if tuple(t.shape) != shape or t.dtype != k_in.dtype:
                raise ValueError("inconsistent k/v shapes or dtypes")
        dt = _dtype_code(k_in)
        if all(t.is_contiguous() for t in (k_in, v_in, k_out, v_out)):
            _check("hubkv_compact", lib().hubkv_compact(_ptr(k_in), _ptr(v_in), dt, _ptr(idx),
                                                        len(seqlens), _arr64(seqlens),
                                                        _arr64(kept), L, Hkv, d, _ptr(k_out),
                                                        _ptr(v_out), _stream(stream)))
        else:
            _check("hubkv_compact_strided",
                   lib().hubkv_compact_strided(_ptr(k_in, True), _strides3(k_in),
                                               _ptr(v_in, True), _strides3(v_in), dt, _ptr(idx),
                                               len(seqlens), _arr64(seqlens), _arr64(kept), L,
                                               Hkv, d, _ptr(k_out, True), _strides3(k_out),
                                               _ptr(v_out, True), _strides3(v_out),
                                               _stream(stream)))
    return k_out, v_out


def hubkv_nestedkv(k, seqlens: Sequence[int], nblocks: int = 32, window: int = 64,
                   log_prior=(0.0, 0.0, 0.0), theta: float = 0.1, s=None, anomalies=None,
                   weights=None, want_parts: bool = False, workspace=None, stream=None):
    """k [L][Hkv][T][d] -> s fp32 [L][Hkv][T] (and, with want_parts, the
    anomalies [L][Hkv][T][3] and blend weights [L][B][Hkv][3])."""
    torch = _torch()
    L, Hkv, T, d = k.shape
    B = len(seqlens)
    sl = _arr64(seqlens)
    with _on(stream):
        if s is None:
            s = _new((L, Hkv, T), torch.float32, k.device)
        if want_parts and anomalies is None:
            anomalies = _new((L, Hkv, T, 3), torch.float32, k.device)
        if want_parts and weights is None:
            weights = _new((L, B, Hkv, 3), torch.float32, k.device)
        nb = lib().hubkv_nestedkv_workspace(B, sl, L, Hkv, d, int(nblocks))
        if workspace is None:
            workspace = _workspace(nb, k.device)
        lp = (C.c_float * 3)(*[float(x) for x in log_prior])
        _check("hubkv_nestedkv", lib().hubkv_nestedkv(
            _ptr(k), _dtype_code(k), B, sl, L, Hkv, d, int(nblocks), int(window),
            C.cast(lp, C.c_void_p), float(theta), _ptr(s), _ptr(anomalies), _ptr(weights),
            _ptr(workspace), workspace.numel(), _stream(stream)))
    return (s, anomalies, weights) if want_parts else s


def hubkv_select_layer(z, seqlens: Sequence[int], layer_kept, n_sink: int, n_recent: int,
                       floor_min: int = 0, idx=None, head_kept=None, workspace=None, stream=None):
    """z fp32 [L][Hkv][T]; layer_kept [L][B] kept totals over each layer's heads ->
    idx int32 [sum layer_kept] (per (layer, sequence), head after head, each
    ascending), head_kept int32 [L][B][Hkv]."""
    torch = _torch()
    L, Hkv, T = z.shape
    B = len(seqlens)
    sl = _arr64(seqlens)
    lk = [int(x) for row in layer_kept for x in (row if hasattr(row, "__len__") else [row])]
    if len(lk) != L * B:
        raise ValueError(f"layer_kept must hold L * B = {L * B} totals")
    with _on(stream):
        if idx is None:
            idx = _new(sum(lk), torch.int32, z.device)
        if head_kept is None:
            head_kept = _new((L, B, Hkv), torch.int32, z.device)
        nb = lib().hubkv_select_layer_workspace(B, sl, L, Hkv)
        if workspace is None:
            workspace = _workspace(nb, z.device)
        _check("hubkv_select_layer", lib().hubkv_select_layer(
            _ptr(z), B, sl, L, Hkv, _arr64(lk), int(n_sink), int(n_recent), int(floor_min),
            _ptr(idx), _ptr(head_kept), _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx, head_kept


def hubkv_compact_layer(k_in, v_in, idx, head_kept, seqlens: Sequence[int], layer_kept,
                        k_out=None, v_out=None, stream=None):
    """k_in/v_in [L][Hkv][T][d] -> k_out/v_out [sum layer_kept][d] in idx's order."""
    L, Hkv, T, d = k_in.shape
    B = len(seqlens)
    lk = [int(x) for row in layer_kept for x in (row if hasattr(row, "__len__") else [row])]
    K = sum(lk)
    with _on(stream):
        if k_out is None:
            k_out = _new((K, d), k_in.dtype, k_in.device)
        if v_out is None:
            v_out = _new((K, d), v_in.dtype, v_in.device)
        _check("hubkv_compact_layer", lib().hubkv_compact_layer(
            _ptr(k_in), _ptr(v_in), _dtype_code(k_in), _ptr(idx), _ptr(head_kept), B,
            _arr64(seqlens), L, Hkv, _arr64(lk), d, _ptr(k_out), _ptr(v_out), _stream(stream)))
    return k_out, v_out


def h2o_step(q, k_new, v_new, k_cache, v_cache, acc, pos, t, scale: float, n_sink: int = 0,
             n_recent: int = 0, include_self: bool = False, evicted=None, probs=None,
             out=None, stream=None, ring: bool = False):
    """One H2O decode step, in place on (k_cache, v_cache, acc, pos).
    q [B][Hq][d], k_new/v_new [B][Hkv][d], caches [B][Hkv][C][d], acc/pos
    [B][Hkv][C]; t: int or per-sequence list.  probs (fp32 [B][Hq][C+1]) and
    out (fp32 [B][Hq][d], the attention output) are filled when given.
    ring=True keeps the recent window in a ring of the last n_recent slots
    (h2o_step_ring).  Returns evicted int32 [B][Hkv]."""
    torch = _torch()
    B, Hq, d = q.shape
    _, Hkv, Cs, _ = k_cache.shape
    tt = [int(t)] * B if isinstance(t, int) else [int(x) for x in t]
    for name, x, shape in (("probs", probs, (B, Hq, Cs + 1)), ("out", out, (B, Hq, d))):
        if x is not None and (x.dtype != torch.float32 or tuple(x.shape) != shape):
            raise ValueError(f"{name} must be float32 of shape {shape}")
    name = "h2o_step_ring" if ring else "h2o_step"
    with _on(stream):
        if evicted is None:
            evicted = _new((B, Hkv), torch.int32, q.device)
        _check(name, getattr(lib(), name)(_ptr(q), _ptr(k_new), _ptr(v_new), _dtype_code(q),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(acc), _ptr(pos),
                                          _arr64(tt), B, Hq, Hkv, d, Cs, int(n_sink),
                                          int(n_recent), float(scale), int(bool(include_self)),
                                          _ptr(evicted), _ptr(probs), _ptr(out),
                                          _stream(stream)))
    return evicted


def protected_count(N: int, n_sink: int, n_recent: int) -> int:
    return int(lib().hubkv_protected_count(int(N), int(n_sink), int(n_recent)))
