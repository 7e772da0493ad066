"""Seeded synthetic inputs shared by the CPU oracle, the GPU tests and the benchmark.

This module only draws random numbers and arranges them into the shapes of the
workloads; it holds none of the scoring, refinement, selection or eviction
arithmetic.  Every array is reproducible from (workload id, layer, unit).

Workload shapes follow the prefill-compression and streaming-decode settings
the pages discuss:

* H2O breakdown page, "Observation 2" (accumulated attention over query
  positions) and the heavy + recent budget section;
* HubKV walkthrough, "Observation" (high scores come in local clusters), which
  is why prefill workloads plant bursts of keys aligned with the window queries;
* KV-cache survey page, section 3.3 (GQA: query heads share a KV head per group)
  and section 4.1 (sink tokens at the start of the sequence are kept).

Layouts (d contiguous):
    Q  [L][Hq][B*W][d]      observation-window queries (the last W positions)
    K  [L][Hkv][T][d]       T = sum of the sequence lengths, packed
    V  [L][Hkv][T][d]
bf16 tensors are produced as float32 values that are exactly representable in
bf16 (round-to-nearest-even of an fp32 draw) together with their uint16 bits.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "PrefillWorkload", "DecodeWorkload", "WORKLOADS", "workload",
    "to_bf16_bits", "bf16_bits_to_f32", "round_bf16",
    "prefill_inputs", "prefill_layer_inputs", "random_scores",
    "decode_unit_stream", "decode_random_state", "budgets", "cluster_spans",
]


# --------------------------------------------------------------------------
# bf16 helpers (bit manipulation only)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(to_bf16_bits(x))


# --------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    wid: int
    name: str
    seqlens: tuple
    L: int
    Hq: int
    Hkv: int
    d: int
    W: int
    dtype: str                      # "f32" or "bf16"
    clusters: Optional[tuple]       # per sequence: number of planted key bursts
    cluster_len: tuple = (16, 16)   # inclusive range of burst lengths
    cluster_gain: tuple = (3.0, 3.0)  # range of a burst's key gain along the window-query mean
    zipf_alpha: Optional[float] = None
    budget: float = 0.1
    r: float = 0.1
    n_sink: int = 4
    n_recent: int = 64
    causal: bool = True
    pool: int = 5
    gamma: float = 0.5
    beta_lo: float = 0.8
    beta_hi: float = 1.2

    @property
    def B(self) -> int:
        return len(self.seqlens)

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def kept(self, budget: Optional[float] = None) -> np.ndarray:
        b = self.budget if budget is None else budget
        return budgets(self.seqlens, b)

    def with_(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    heavy: int
    recent: int
    prompt: int
    decode: int
    dtype: str
    n_sink: int = 0
    include_self: int = 0

    @property
    def C(self) -> int:
        return self.heavy + self.recent

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


def budgets(seqlens: Sequence[int], budget: float) -> np.ndarray:
    """Kept tokens per sequence: floor(budget * N_b), sinks and recents included."""
    return np.array([int(math.floor(budget * n + 1e-9)) for n in seqlens], dtype=np.int64)


WORKLOADS = {
    # tiny fp32 prefill compression: 4 heads, N=512, window 32, 20% kept
    1: PrefillWorkload(1, "tiny-prefill-n512-h4-d64-f32", (512,), 1, 4, 4, 64, 32, "f32",
                       clusters=(8,), cluster_len=(16, 16), budget=0.2, r=0.2,
                       n_sink=0, n_recent=16),
    # Llama-2-7B-shaped layer: 32 MHA heads, d=128, N=32768, window 64, 10% kept
    2: PrefillWorkload(2, "llama2-7b-layer-n32768-h32-d128-bf16", (32768,), 1, 32, 32, 128, 64,
                       "bf16", clusters=(256,), cluster_len=(8, 64), budget=0.1, r=0.1,
                       n_sink=4, n_recent=64),
    # GQA long context: 32 query / 8 KV heads, N=131072, 32 layers, Zipf mass
    3: PrefillWorkload(3, "gqa-n131072-hq32-hkv8-d128-bf16-l32", (131072,), 32, 32, 8, 128, 64,
                       "bf16", clusters=None, zipf_alpha=1.1, budget=0.1, r=0.1,
                       n_sink=4, n_recent=64),
    # H2O streaming decode
    4: DecodeWorkload(4, "h2o-decode-b16-h32-d128-bf16-c4096", 16, 32, 32, 128,
                      heavy=2048, recent=2048, prompt=16384, decode=512, dtype="bf16"),
    # coverage diagnostic: bursts of graded strength (key gain 4..24 along the
    # window-query mean), so a plain Top-K can spend its budget inside the
    # strongest bursts
    6: PrefillWorkload(6, "coverage-graded-n32768-h8-d128-bf16", (32768,), 1, 8, 8, 128, 64,
                       "bf16", clusters=(256,), cluster_len=(8, 64), cluster_gain=(4.0, 24.0),
                       budget=0.02, r=0.02, n_sink=4, n_recent=64),
    # ragged batch at scale: 4 sequences 64K..512K, 8 KV heads x 4, window 128
    5: PrefillWorkload(5, "ragged-b4-64k-512k-hkv8-g4-d128-bf16", (65536, 131072, 262144, 524288),
                       1, 32, 8, 128, 128, "bf16",
                       clusters=(32, 64, 128, 256), cluster_len=(8, 128), budget=0.1, r=0.1,
                       n_sink=4, n_recent=128),
}

# H2O Algorithm-1 tiny case: budget 3 on N=12 (fp32, 4 heads, d=64)
H2O_TINY = DecodeWorkload(1, "h2o-alg1-budget3-n12-h4-d64-f32", 1, 4, 4, 64,
                          heavy=3, recent=0, prompt=12, decode=0, dtype="f32")


def workload(wid: int):
    return WORKLOADS[wid]


# --------------------------------------------------------------------------
# Random streams
# --------------------------------------------------------------------------
def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _cluster_spans(rng, n_clusters, lens_range, lo, hi):
    """Non-overlapping [start, start+len) spans inside [lo, hi), in order."""
    if n_clusters <= 0:
        return []
    a, b = lens_range
    lens = rng.integers(a, b + 1, size=n_clusters)
    free = (hi - lo) - int(lens.sum())
    if free < 0:
        raise ValueError("clusters do not fit")
    pts = np.sort(rng.integers(0, free + 1, size=n_clusters))
    spans, off = [], lo
    for p, ln in zip(pts, lens):
        s = off + int(p)
        spans.append((s, s + int(ln)))
        off += int(ln)
    return spans


def _spans_and_gains(w: PrefillWorkload, layer: int):
    seed = 1000 * w.wid + layer
    base = np.random.default_rng(seed)
    spans, gains = [], []
    for b, n in enumerate(w.seqlens):
        if w.clusters is not None:
            sp = _cluster_spans(base, w.clusters[b], w.cluster_len, w.n_sink, n - w.n_recent)
        else:
            sp = []
        spans.append(sp)
        lo, hi = w.cluster_gain
        if lo == hi:
            gains.append(None)
        else:
            grng = np.random.default_rng([seed, 1, b])
            gains.append(grng.uniform(lo, hi, size=len(sp)).astype(np.float32))
    return spans, gains


def cluster_spans(w: PrefillWorkload, layer: int = 0):
    """The planted bursts of one layer: per sequence, a list of [start, end)
    positions local to the sequence (the same spans prefill_layer_inputs plants)."""
    return _spans_and_gains(w, layer)[0]


def prefill_layer_inputs(w: PrefillWorkload, layer: int = 0, with_v: bool = True, threads: int = 8):
    """One layer of Q [Hq][B*W][d], K [Hkv][T][d], V [Hkv][T][d] as float32
    (bf16-representable when w.dtype == 'bf16').  Seed = 1000*wid + layer; one
    child stream per KV head so units can be drawn in parallel."""
    seed = 1000 * w.wid + layer
    B, W, d, G, T = w.B, w.W, w.d, w.G, w.T
    cu = np.concatenate([[0], np.cumsum(w.seqlens)]).astype(np.int64)
    Q = np.empty((w.Hq, B * W, d), np.float32)
    K = np.empty((w.Hkv, T, d), np.float32)
    V = np.empty((w.Hkv, T, d), np.float32) if with_v else None
    # burst spans (and gains) shared by every head of a sequence
    spans, gains = _spans_and_gains(w, layer)
    unit_rngs = _streams(seed, w.Hkv)

    def unit(g):
        rng = unit_rngs[g]
        q = _normal(rng, (G, B * W, d))
        k = _normal(rng, (T, d))
        if w.zipf_alpha is not None:
            for b, n in enumerate(w.seqlens):
                u = _normal(rng, (d,))
                u /= np.float32(np.linalg.norm(u))
                mu = np.float32(8.0)
                q[:, b * W:(b + 1) * W, :] += mu * u
                rho = rng.permutation(n).astype(np.float64) + 1.0
                c = (math.sqrt(d) / 8.0) * w.zipf_alpha * np.log(n / rho)
                k[cu[b]:cu[b + 1]] += (c[:, None] * u[None, :]).astype(np.float32)
        for b, sp in enumerate(spans):
            if not sp:
                continue
            mean = q[:, b * W:(b + 1) * W, :].reshape(-1, d).mean(axis=0)
            center = np.float32(w.cluster_gain[0]) * mean if gains[b] is None else None
            for j, (s0, s1) in enumerate(sp):
                cj = center if gains[b] is None else gains[b][j] * mean
                k[cu[b] + s0:cu[b] + s1] = cj[None, :] + _normal(rng, (s1 - s0, d), 0.3)
        if w.dtype == "bf16":
            q = round_bf16(q)
            k = round_bf16(k)
        Q[g * G:(g + 1) * G] = q
        K[g] = k
        if with_v:
            v = _normal(rng, (T, d))
            V[g] = round_bf16(v) if w.dtype == "bf16" else v

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(unit, range(w.Hkv)))
    return Q, K, V


def prefill_inputs(w: PrefillWorkload, layers: Optional[Sequence[int]] = None, with_v=True,
                   threads: int = 8):
    """Stack layers -> Q [L][Hq][B*W][d], K/V [L][Hkv][T][d]."""
    layers = list(range(w.L)) if layers is None else list(layers)
    qs, ks, vs = [], [], []
    for l in layers:
        q, k, v = prefill_layer_inputs(w, l, with_v=with_v, threads=threads)
        qs.append(q); ks.append(k); vs.append(v)
    Q = np.stack(qs); K = np.stack(ks)
    V = np.stack(vs) if with_v else None
    return Q, K, V


def random_scores(seqlens, L, Hkv, seed, kind="attention", ties=False):
    """Stand-alone fp32 score arrays [L][Hkv][T] for testing refine/select with
    identical inputs on both sides.  kind='attention' draws a power-law mass
    with local bursts; 'uniform' draws U(0,1)."""
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    if kind == "uniform":
        s = rng.random((L, Hkv, T), dtype=np.float32)
    else:
        s = (rng.pareto(1.5, size=(L, Hkv, T)) + 0.01).astype(np.float32)
        # local bursts: smooth a fraction of positions upward
        nb = max(1, T // 256)
        for l in range(L):
            for h in range(Hkv):
                starts = rng.integers(0, max(1, T - 16), size=nb)
                for st in starts:
                    ln = int(rng.integers(2, 16))
                    s[l, h, st:st + ln] += np.float32(rng.random() * 4.0)
    if ties:
        s = np.round(s * 4.0).astype(np.float32) / np.float32(4.0)
    return np.ascontiguousarray(s)


# --------------------------------------------------------------------------
# Streaming decode inputs
# --------------------------------------------------------------------------
def decode_unit_stream(w: DecodeWorkload, b: int, g: int, steps: int):
    """Per (sequence b, KV head g) stream of step inputs: q [steps][G][d],
    k [steps][d], v [steps][d] (float32, bf16-representable when bf16).
    Each unit has its own seed so sampled units can be drawn alone."""
    G = w.Hq // w.Hkv
    rng = np.random.default_rng([1000 * w.wid, b, g])
    q = _normal(rng, (steps, G, w.d))
    k = _normal(rng, (steps, w.d))
    v = _normal(rng, (steps, w.d))
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def decode_random_state(w: DecodeWorkload, t: int, seed: int, fill: Optional[int] = None):
    """A mid-stream cache state drawn directly (not produced by any step):
    K/V slots [B][Hkv][C][d], acc [B][Hkv][C] >= 0, pos [B][Hkv][C] with
    distinct positions < t (-1 = empty), plus the step inputs q [B][Hq][d],
    k_new/v_new [B][Hkv][d].  Recent positions (> t - recent) are always
    present, as a running stream guarantees."""
    rng = np.random.default_rng(seed)
    B, Hkv, Hq, C, d = w.B, w.Hkv, w.Hq, w.C, w.d
    fill = C if fill is None else fill
    Kc = _normal(rng, (B, Hkv, C, d))
    Vc = _normal(rng, (B, Hkv, C, d))
    acc = np.zeros((B, Hkv, C), np.float32)
    pos = np.full((B, Hkv, C), -1, np.int32)
    nrec = min(w.recent - 1, fill, t) if w.recent > 0 else 0
    for b in range(B):
        for g in range(Hkv):
            recent = np.arange(t - nrec, t)
            older_pool = np.arange(0, t - nrec)
            n_old = fill - nrec
            older = np.sort(rng.choice(older_pool, size=n_old, replace=False))
            p = np.concatenate([older, recent]).astype(np.int32)
            slots = rng.permutation(C)[:fill]
            pos[b, g, slots] = p
            # accumulated mass grows with age; a power-law spread
            age = (t - p).astype(np.float32)
            acc[b, g, slots] = (rng.pareto(1.2, size=fill).astype(np.float32) * 0.05
                                + age * np.float32(1e-3))
    q = _normal(rng, (B, Hq, d))
    kn = _normal(rng, (B, Hkv, d))
    vn = _normal(rng, (B, Hkv, d))
    if w.dtype == "bf16":
        Kc, Vc, q, kn, vn = (round_bf16(x) for x in (Kc, Vc, q, kn, vn))
    return dict(K=Kc, V=Vc, acc=acc, pos=pos, q=q, k_new=kn, v_new=vn)
