"""Benchmark of the per-head KV retention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline]
    python bench.py --copy-calibration      # 1 GiB device copies, for counter scaling

One step = the whole prefill path over one batch of synthetic input already
resident in HBM: hubkv_score -> hubkv_refine -> hubkv_select -> hubkv_compact
(every KV head, every layer of the workload).  Prints one JSON line with
scored+selected tokens per second per head (K steps timed back to back
between two synchronisations), per-op times measured with HIP events on the
launch stream over K further steps, the roofline position of the dominant
op, and the CPU oracle timed on this host's cores on a bounded sample.

Default workload: the Llama-2-7B-shaped layer (32 MHA heads, d 128, 32768
tokens, window 64, 10% kept with 4 sink and 64 recent tokens, bf16).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
COPY_BYTES = 1 << 30         # size of one calibration copy

# HBM bytes per launch of the score op (all of its kernels) on the
# Llama-2-7B-shaped layer, from two rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE) of `bench.py --steps 5 --warmup 1 --no-cpu-baseline`, each scaled
# by the same counter over a plain 1 GiB device copy (`bench.py
# --copy-calibration`).  Valid only for the score source they were taken on.
SCORE_TRAFFIC = {"sha256": "8e4c6ddedc997dfcedafdd1267de45c1e2c7b1c853c64f8410c1731b14945500", "workload": 2,
                 "fetch_bytes": 546619531, "write_bytes": 4350961}


# The same for one full-cache h2o_step launch of the decode workload (scores
# only, fixed slots), from `bench.py --workload 4 --steps 8 --warmup 1
# --no-cpu-baseline` (the last 1000 launches).  Valid only for the decode
# source it was taken on.
DECODE_TRAFFIC = {"sha256": "73b295d5acfa5d786c8b46c62cbb7493d36e9df5701b0aac7745b0e402b0ec39", "workload": 4,
                  "fetch_bytes": 554371979, "write_bytes": 8683520}


def _source_sha(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "token_scoring_top_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _score_source_sha() -> str:
    return _source_sha(("score.hip", "internal.hpp"))


def copy_calibration(reps: int = 5) -> int:
    """Plain device-to-device copies of COPY_BYTES, for scaling HBM counters."""
    import torch
    assert torch.cuda.is_available(), "copy calibration needs a GPU"
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": reps, "GBs": 2 * COPY_BYTES / dt / 1e9}))
    return 0


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def op_bytes(w, kept_total, elem):
    """Algorithmic HBM bytes of each op for one step (every layer and head)."""
    L, Hkv, Hq, d, T, W, B = w.L, w.Hkv, w.Hq, w.d, w.T, w.W, w.B
    q = L * Hq * B * W * d * elem
    k = L * Hkv * T * d * elem
    s = L * Hkv * T * 4
    idx = L * Hkv * kept_total * 4
    rows = L * Hkv * kept_total * d * elem
    return {
        "score": q + k + s,                 # Q and K read once, s written
        "refine": 2 * s,                    # s read, z written
        "select": s + idx,                  # z read, indices written
        "compact": idx + 4 * rows,          # indices read, K and V rows read and written
    }


def score_flops(w):
    """One QK^T sweep (2 flops per multiply-add; the causal corner is ignored)."""
    return 2.0 * w.L * w.Hq * w.W * w.T * w.d


def h2o_step_bytes(w, elem, with_out=False):
    """Algorithmic HBM bytes of one h2o_step launch: every retained K row read,
    acc read and written, pos read, the query, the new K/V rows read, and one
    slot's K/V/acc/pos written per (sequence, KV head).  With the attention
    output, every retained V row is read too and the fp32 output written."""
    B, Hkv, Hq, d, C = w.B, w.Hkv, w.Hq, w.d, w.C
    n = (B * Hkv * C * (d * elem + 4 + 4 + 4) + B * Hq * d * elem
         + B * Hkv * (2 * d * elem) + B * Hkv * (2 * d * elem + 8))
    if with_out:
        n += B * Hkv * C * d * elem + B * Hq * d * 4
    return n


# (sequence, KV head) units of the decode workload that the oracle follows
# beside the GPU: one per sequence, KV heads spread over the 32
DECODE_SAMPLE_UNITS = tuple((i, (5 * i + 3) % 32) for i in range(16))


class DecodeStream:
    """The decode workload streamed through h2o_step (or h2o_step_ring) on the
    GPU for every (sequence, KV head) unit, with the oracle beside it on the
    sampled units, each side running freely on its own state.  Both sides get
    the same per-step inputs for those units: their rows of q, k and v come
    from each unit's own seeded stream (synthetic.decode_unit_stream); every
    other unit's rows are seeded normal draws made on the GPU.  The GPU records
    each sampled unit's evicted position at every step; the oracle catches up
    on demand and reports its candidates' margin, so a divergence can be
    traced to a near-tie."""

    def __init__(self, w, total, units=DECODE_SAMPLE_UNITS, ring=False, attn_out=False,
                 with_oracle=True, block=256):
        import numpy as np
        import torch

        import synthetic as S
        self.np, self.torch = np, torch
        self.w, self.total, self.ring, self.block = w, int(total), ring, block
        self.units = [(b, g) for b, g in units if b < w.B and g < w.Hkv]
        B, Hq, Hkv, d, C = w.B, w.Hq, w.Hkv, w.d, w.C
        self.G = Hq // Hkv
        dev = "cuda"
        self.dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.Kc = torch.zeros((B, Hkv, C, d), dtype=self.dt, device=dev)
        self.Vc = torch.zeros_like(self.Kc)
        self.acc = torch.zeros((B, Hkv, C), dtype=torch.float32, device=dev)
        self.pos = torch.full((B, Hkv, C), -1, dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev) if attn_out else None
        self.gen = torch.Generator(device=dev)
        self.gen.manual_seed(1000 * w.wid)
        streams = [S.decode_unit_stream(w, b, g, self.total) for b, g in self.units]
        self.uq = np.stack([x[0] for x in streams], 1)   # [total][units][G][d]
        self.uk = np.stack([x[1] for x in streams], 1)   # [total][units][d]
        self.uv = np.stack([x[2] for x in streams], 1)
        nu = len(self.units)
        self.ub = torch.tensor([b for b, _ in self.units], device=dev, dtype=torch.long)
        self.ug = torch.tensor([g for _, g in self.units], device=dev, dtype=torch.long)
        self.ev_gpu = np.full((self.total, nu), -2, np.int32)
        self.t = 0
        self.with_oracle = with_oracle
        if with_oracle:
            import oracle
            self.oracle = oracle
            self.ost = oracle.empty_state(nu, 1, C, d)
            self.ev_orc = np.full((self.total, nu), -2, np.int32)
            self.mg_orc = np.full((self.total, nu), np.inf, np.float32)
            self.to = 0

    def inputs(self, t0, n):
        """q, k, v of steps [t0, t0 + n) on the device, [n][B][...][d]."""
        torch, w = self.torch, self.w
        B, Hq, Hkv, d, G = w.B, w.Hq, w.Hkv, w.d, self.G
        q = torch.randn((n, B, Hq, d), generator=self.gen, device="cuda").to(self.dt)
        k = torch.randn((n, B, Hkv, d), generator=self.gen, device="cuda").to(self.dt)
        v = torch.randn((n, B, Hkv, d), generator=self.gen, device="cuda").to(self.dt)
        uq = torch.from_numpy(self.uq[t0:t0 + n]).cuda().to(self.dt)
        uk = torch.from_numpy(self.uk[t0:t0 + n]).cuda().to(self.dt)
        uv = torch.from_numpy(self.uv[t0:t0 + n]).cuda().to(self.dt)
        for i, (b, g) in enumerate(self.units):
            q[:, b, g * G:(g + 1) * G] = uq[:, i]
            k[:, b, g] = uk[:, i]
            v[:, b, g] = uv[:, i]
        return q, k, v

    def launch(self, q, k, v, t, evicted, stream=None):
        import token_scoring_top_amd as hk
        w = self.w
        hk.h2o_step(q, k, v, self.Kc, self.Vc, self.acc, self.pos, t, w.scale, w.n_sink,
                    w.recent, bool(w.include_self), evicted=evicted, out=self.out,
                    stream=stream, ring=self.ring)

    def run_gpu(self, n, stream=None, oracle_beside=False):
        """n more steps on the GPU (blocks of inputs drawn on the device); the
        oracle follows block by block when asked."""
        torch = self.torch
        end = self.t + n
        while self.t < end:
            m = min(self.block, end - self.t)
            q, k, v = self.inputs(self.t, m)
            evs = torch.empty((m, self.w.B, self.w.Hkv), dtype=torch.int32, device="cuda")
            for i in range(m):
                self.launch(q[i], k[i], v[i], self.t + i, evs[i], stream)
            if oracle_beside and self.with_oracle:
                self.run_oracle(self.t)   # the previous blocks, while this one runs
            self.record(self.t, evs[:, self.ub, self.ug])
            self.t += m

    def record(self, t0, ev_units):
        ev = ev_units.cpu().numpy()
        self.ev_gpu[t0:t0 + ev.shape[0]] = ev

    def run_oracle(self, until):
        w = self.w
        while self.to < min(until, self.total):
            t = self.to
            ev, mg = self.oracle.h2o_step(self.ost, self.uq[t], self.uk[t][:, None],
                                          self.uv[t][:, None], t, w.scale, w.n_sink, w.recent,
                                          w.include_self, want_margin=True)
            self.ev_orc[t] = ev[:, 0]
            self.mg_orc[t] = mg[:, 0]
            self.to += 1

    def stats(self):
        """Free-running agreement over the steps both sides have run."""
        np = self.np
        T = min(self.t, self.to)
        evg, evo, mg = self.ev_gpu[:T], self.ev_orc[:T], self.mg_orc[:T]
        evicting = (evg >= 0) | (evo >= 0)
        same = evg == evo
        prompt = self.w.prompt
        dec = np.zeros_like(same)
        dec[prompt:] = True
        first, first_margin = [], []
        for u in range(len(self.units)):
            bad = np.flatnonzero(~same[:, u])
            if bad.size:
                first.append(int(bad[0]))
                first_margin.append(float(mg[bad[0], u]))
        # retained sets after step T (the GPU cache must be at the same step)
        pos_g = self.pos[self.ub, self.ug].cpu().numpy()
        overlap = [np.intersect1d(pos_g[u][pos_g[u] >= 0], self.ost["pos"][u, 0][
            self.ost["pos"][u, 0] >= 0]).size / self.w.C for u in range(len(self.units))]
        return {
            "steps": int(T), "units": [list(x) for x in self.units],
            "evictions_compared": int(evicting.sum()),
            "identical_eviction_frac": float(same[evicting].mean()) if evicting.any() else 1.0,
            "identical_eviction_frac_decode": (float(same[evicting & dec].mean())
                                               if (evicting & dec).any() else None),
            "units_diverged": len(first),
            "first_divergence_steps": first,
            "first_divergence_oracle_margins": first_margin,
            "final_set_overlap_mean": float(np.mean(overlap)),
            "final_set_overlap_min": float(np.min(overlap)),
        }


def bench_decode(args, w):
    """Streaming H2O decode: the prompt is streamed through h2o_step to build
    the cache state (untimed), then `steps` decode steps are timed.  With the
    CPU baseline on, the oracle also follows sampled units beside the GPU
    through the whole stream (free running) and the line reports how often
    both evict the same token and how far their final caches overlap."""
    import numpy as np
    import torch

    steps = 512 if args.steps is None else args.steps
    B, Hq, Hkv, d, C = w.B, w.Hq, w.Hkv, w.d, w.C
    elem = 2 if w.dtype == "bf16" else 4
    follow = not args.no_cpu_baseline
    total = w.prompt + args.warmup + 2 * steps
    ds = DecodeStream(w, total, ring=args.ring, attn_out=args.attn_out, with_oracle=follow)
    stream = torch.cuda.current_stream()
    # the prompt and the warm-up steps, streamed token by token (builds the
    # retained cache); the oracle follows block by block on the host
    ds.run_gpu(w.prompt + args.warmup, stream, oracle_beside=follow)
    t = ds.t
    # timed decode steps; inputs are drawn before the timed region
    q, k, v = ds.inputs(t, steps)
    evs = torch.empty((steps, B, Hkv), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ds.launch(q[i], k[i], v[i], t + i, evs[i], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ds.record(t, evs[:, ds.ub, ds.ug])
    ds.t = t = t + steps
    ms_step = (t1 - t0) * 1e3 / steps
    # per-launch kernel time from HIP events on the launch stream
    ev_t = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)]
    q, k, v = ds.inputs(t, steps)
    for i in range(steps):
        ev_t[i][0].record(stream)
        ds.launch(q[i], k[i], v[i], t + i, evs[i], stream)
        ev_t[i][1].record(stream)
    torch.cuda.synchronize()
    ds.record(t, evs[:, ds.ub, ds.ug])
    ds.t = t = t + steps
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_t]))
    nbytes = h2o_step_bytes(w, elem, args.attn_out)
    ach = nbytes / (k_ms / 1e3) / 1e9
    dec_traffic = None
    if (not args.attn_out and not args.ring and DECODE_TRAFFIC["workload"] == w.wid
            and DECODE_TRAFFIC["sha256"] == _source_sha(("h2o_step.hip", "internal.hpp"))):
        dec_traffic = DECODE_TRAFFIC["fetch_bytes"] + DECODE_TRAFFIC["write_bytes"]

    cpu = None
    free = None
    if follow:
        import oracle
        nthreads = min(16, _cores())
        oracle.set_threads(nthreads)
        used = oracle.get_threads()
        # the oracle's free-running units catch up with the GPU's last step
        ds.run_oracle(ds.t)
        free = ds.stats()
        # bounded sample: decode steps of the oracle from a copy of the GPU state
        def f32(x):
            return np.ascontiguousarray(x.float().cpu().numpy())
        state = {"K": f32(ds.Kc), "V": f32(ds.Vc), "acc": ds.acc.cpu().numpy().copy(),
                 "pos": ds.pos.cpu().numpy().copy()}
        qs, ks, vs = (f32(x) for x in ds.inputs(min(t, total - 64), 64))
        reps, tc0 = 0, time.perf_counter()
        while reps < 64:
            oracle.h2o_step(state, qs[reps], ks[reps], vs[reps], t + reps, w.scale, w.n_sink,
                            w.recent, w.include_self, want_out=args.attn_out)
            reps += 1
            if time.perf_counter() - tc0 >= args.cpu_budget_s:
                break
        tc = (time.perf_counter() - tc0) / reps
        cpu = {"value": C / tc, "unit": "retained-cache tokens/s/head", "cores": used,
               "cpu_model": _cpu_model(),
               "kind": "oracle",
               "sample": f"{reps} decode step(s) of the full batch ({B} x {Hkv} heads x {C} "
                         f"slots) from a copy of the GPU state, {tc:.3f} s each"}

    out = {
        "metric": "retained-cache tokens scored per second per head (H2O decode)",
        "value": C / (ms_step / 1e3),
        "unit": "tokens/s/head",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "heavy": w.heavy,
                   "recent": w.recent, "prompt_steps_untimed": w.prompt,
                   "attention_output": bool(args.attn_out),
                   "slot_layout": "ring" if args.ring else "fixed",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": dec_traffic, "op": "h2o_step",
                     "kernels": "h2o_step_kernel", "algorithmic_bytes": nbytes},
        "kernel_ms": k_ms,
        "free_running": free,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


def bench_coverage(args):
    """Cluster-coverage diagnostic: on workloads with planted key bursts, the
    number of bursts that keep at least one token, for a plain Top-K (r = 0,
    so z = s) and for the hub-corrected score under two readings of r (r =
    kept fraction, and r = 1 - kept fraction), across budgets.  One JSON line
    per workload; the path (score, refine, select) runs on the GPU."""
    import numpy as np
    import torch

    import synthetic as S
    import token_scoring_top_amd as hk
    from token_scoring_top_amd.diagnostics import cluster_coverage, tokens_in_clusters

    budgets = [0.01, 0.02, 0.05, 0.1, 0.2]
    for wid in (2, 6):
        w = S.workload(wid)
        q, k, _ = S.prefill_layer_inputs(w, 0, with_v=False, threads=min(16, _cores()))

        def dev(x):
            bits = S.to_bf16_bits(x).view(np.int16)
            return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)

        Qd, Kd = dev(q[None]), dev(k[None])
        del q, k
        spans = S.cluster_spans(w, 0)
        ncl = sum(len(sp) for sp in spans)
        ntok = sum(e - s for sp in spans for s, e in sp)
        s, st = hk.hubkv_score(Qd, Kd, w.seqlens, w.W, w.scale, w.causal)
        rows = []
        for bud in budgets:
            kept = S.budgets(w.seqlens, bud)
            row = {"budget": bud, "kept_per_head": int(kept.sum())}
            for name, r in (("plain_topk", 0.0), ("r=budget", bud), ("r=1-budget", 1.0 - bud)):
                z, _ = hk.hubkv_refine(s, w.seqlens, head_stats=st, pool=w.pool, gamma=w.gamma,
                                       beta_lo=w.beta_lo, beta_hi=w.beta_hi, r=r)
                idx = hk.hubkv_select(z, w.seqlens, kept, w.n_sink, w.n_recent)
                ih = idx.cpu().numpy()
                cov = cluster_coverage(ih, kept, spans).sum(axis=2)      # [L][Hkv]
                tin = tokens_in_clusters(ih, kept, spans).sum(axis=2)
                row[name] = {"covered_mean": float(cov.mean()), "covered_min": int(cov.min()),
                             "covered_max": int(cov.max()),
                             "tokens_in_bursts_mean": float(tin.mean())}
            rows.append(row)
        print(json.dumps({"diagnostic": "planted-burst coverage", "workload": w.name,
                          "bursts": ncl, "burst_tokens": ntok, "heads": w.Hkv,
                          "r_readings": {"plain_topk": 0.0, "r=budget": "budget",
                                         "r=1-budget": "1 - budget"},
                          "rows": rows}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 512 decode steps for the decode workload)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--layer-budget", action="store_true",
                    help="prefill: one budget per layer shared by its KV heads (hubkv_select_layer)")
    ap.add_argument("--nestedkv", action="store_true",
                    help="prefill with the NestedKV key-only score and the layer-wide budget")
    ap.add_argument("--coverage", action="store_true",
                    help="planted-burst coverage diagnostic instead of the benchmark")
    ap.add_argument("--attn-out", action="store_true",
                    help="decode workload: h2o_step also writes the attention output")
    ap.add_argument("--graph", action="store_true",
                    help="prefill: time replays of one step captured into a HIP graph")
    ap.add_argument("--ring", action="store_true",
                    help="decode workload: the recent window in a ring of slots (h2o_step_ring)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode: every (layer, sequence, KV head) unit is independent, so N GPUs "
              "would each run this same kernel chain on their own share of heads.",
              file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()

    import numpy as np
    import torch

    import synthetic as S
    import token_scoring_top_amd as hk

    hk.lib()  # fails loudly when the native library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.coverage:
        return bench_coverage(args)
    w = S.workload(args.workload)
    if isinstance(w, S.DecodeWorkload):
        return bench_decode(args, w)
    if args.steps is None:
        args.steps = 20
    nthreads = min(16, _cores())
    elem = 2 if w.dtype == "bf16" else 4
    tdt = torch.bfloat16 if elem == 2 else torch.float32

    def dev(x, out):
        if w.dtype == "bf16":
            bits = S.to_bf16_bits(x).view(np.int16)
            out.copy_(torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16))
        else:
            out.copy_(torch.from_numpy(np.ascontiguousarray(x)))

    # inputs drawn layer by layer on the host and copied into device tensors
    # (the 32-layer GQA workload does not fit host memory all at once)
    Qd = torch.empty((w.L, w.Hq, w.B * w.W, w.d), dtype=tdt, device="cuda")
    Kd = torch.empty((w.L, w.Hkv, w.T, w.d), dtype=tdt, device="cuda")
    Vd = torch.empty_like(Kd)
    layer0 = None
    for l in range(w.L):
        q, k, v = S.prefill_layer_inputs(w, l, threads=nthreads)
        dev(q, Qd[l]); dev(k, Kd[l]); dev(v, Vd[l])
        if l == 0:
            layer0 = (q, k, v)
        del q, k, v
        if w.L > 1:
            print(f"inputs: layer {l + 1}/{w.L} on the device", file=sys.stderr, flush=True)
    kept = w.kept()
    Ksum = int(kept.sum())
    L, Hkv, T = w.L, w.Hkv, w.T
    f32 = dict(dtype=torch.float32, device="cuda")
    s = torch.empty((L, Hkv, T), **f32)
    z = torch.empty((L, Hkv, T), **f32)
    st = torch.empty((L, w.B, Hkv, 2), dtype=torch.float64, device="cuda")
    beta = torch.empty((L, w.B, Hkv), **f32)
    idx = torch.empty((L, Hkv, Ksum), dtype=torch.int32, device="cuda")
    ko = torch.empty((L, Hkv, Ksum, w.d), dtype=Kd.dtype, device="cuda")
    vo = torch.empty_like(ko)
    # layer-wide budget: each (layer, sequence) keeps Hkv x kept_b over its
    # heads, every head at least its protected tokens plus a quarter of its
    # even share
    lk = [[w.Hkv * int(kb) for kb in kept] for _ in range(L)]
    floor = int(min(kept)) // 4
    if args.nestedkv:
        args.layer_budget = True  # the NestedKV path allocates the layer's budget across heads
        ws_n = torch.empty(hk.lib().hubkv_nestedkv_workspace(w.B, hk._arr64(w.seqlens), L, Hkv,
                                                             w.d, 32),
                           dtype=torch.uint8, device="cuda")
    if args.layer_budget:
        idx_l = torch.empty(L * Hkv * Ksum, dtype=torch.int32, device="cuda")
        hkept = torch.empty((L, w.B, Hkv), dtype=torch.int32, device="cuda")
        ws_l = torch.empty(hk.lib().hubkv_select_layer_workspace(w.B, hk._arr64(w.seqlens), L, Hkv),
                           dtype=torch.uint8, device="cuda")
        ko = ko.view(L * Hkv * Ksum, w.d)
        vo = vo.view(L * Hkv * Ksum, w.d)
    sl = hk._arr64(w.seqlens)
    ws_s = torch.empty(hk.lib().hubkv_score_workspace(w.B, sl, L, w.Hq, Hkv, w.W, w.d,
                                                      1 if elem == 2 else 0),
                       dtype=torch.uint8, device="cuda")
    ws_r = torch.empty(max(256, hk.lib().hubkv_refine_workspace(w.B, sl, L, Hkv)),
                       dtype=torch.uint8, device="cuda")
    ws_rs = torch.empty(hk.lib().hubkv_refine_select_workspace(w.B, sl, L, Hkv),
                        dtype=torch.uint8, device="cuda")
    fused = not args.layer_budget  # refine and select in one call (hubkv_refine_select)
    launch_stream = torch.cuda.current_stream()

    def step(ev=None, strm=None):
        stream = strm if strm is not None else launch_stream
        if ev: ev[0].record(stream)
        if args.nestedkv:
            # key-only score: no queries, no refinement (the scores are not
            # attention mass); they go straight to the layer-wide selection
            hk.hubkv_nestedkv(Kd, w.seqlens, s=z, workspace=ws_n, stream=stream)
            if ev: ev[1].record(stream)
            if ev: ev[2].record(stream)
        else:
            hk.hubkv_score(Qd, Kd, w.seqlens, w.W, w.scale, w.causal, s=s, head_stats=st,
                           workspace=ws_s, stream=stream)
            if ev: ev[1].record(stream)
            if fused:
                hk.hubkv_refine_select(s, w.seqlens, kept, w.n_sink, w.n_recent, head_stats=st,
                                       pool=w.pool, gamma=w.gamma, beta_lo=w.beta_lo,
                                       beta_hi=w.beta_hi, r=w.r, z=z, beta_out=beta, idx=idx,
                                       workspace=ws_rs, stream=stream)
            else:
                hk.hubkv_refine(s, w.seqlens, head_stats=st, pool=w.pool, gamma=w.gamma,
                                beta_lo=w.beta_lo, beta_hi=w.beta_hi, r=w.r, z=z, beta_out=beta,
                                workspace=ws_r, stream=stream)
            if ev: ev[2].record(stream)
        if args.layer_budget:
            hk.hubkv_select_layer(z, w.seqlens, lk, w.n_sink, w.n_recent, floor, idx=idx_l,
                                  head_kept=hkept, workspace=ws_l, stream=stream)
        elif not fused:
            hk.hubkv_select(z, w.seqlens, kept, w.n_sink, w.n_recent, idx=idx, workspace=ws_rs,
                            stream=stream)
        if ev: ev[3].record(stream)
        if args.layer_budget:
            hk.hubkv_compact_layer(Kd, Vd, idx_l, hkept, w.seqlens, lk, k_out=ko, v_out=vo,
                                   stream=stream)
        else:
            hk.hubkv_compact(Kd, Vd, idx, w.seqlens, kept, k_out=ko, v_out=vo, stream=stream)
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    graph = None
    if args.graph:
        # one step captured into a HIP graph (every buffer is preallocated and
        # the library allocates nothing, so the capture holds only kernels)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(launch_stream)
        with torch.cuda.graph(graph, stream=cap):
            step(strm=cap)
        launch_stream.wait_stream(cap)
        for _ in range(args.warmup):
            graph.replay()
    # timed region: whole steps back to back, no markers between the ops
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # per-op times: the same number of steps again, with HIP events recorded
    # on the launch stream between the ops (the markers cost a little time,
    # so these steps are not the ones `value` comes from)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ["score", "refine", "select", "compact"]
    op_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
             for j, n in enumerate(names)}
    if fused:  # one call covers refinement and selection: one time for both
        op_ms["refine_select"] = op_ms.pop("refine") + op_ms.pop("select")
    tokens = float(w.T * w.L)
    value = tokens / (ms_step / 1e3)

    # the Zipf workload's attention mass: slope of log(score) against log(rank)
    # on layer 0 (ranks 16 .. N/16, every KV head), against the planted -alpha
    zipf = None
    if w.zipf_alpha is not None and not args.nestedkv:
        s0 = s[0].cpu().numpy().astype(np.float64)
        slopes = []
        for h in range(w.Hkv):
            for b in range(w.B):
                c0 = int(sum(w.seqlens[:b]))
                v = np.sort(s0[h, c0:c0 + w.seqlens[b]])[::-1]
                rk = np.arange(1, v.size + 1)
                sel = (rk >= 16) & (rk <= v.size // 16) & (v > 0)
                slopes.append(float(np.polyfit(np.log(rk[sel]), np.log(v[sel]), 1)[0]))
        zipf = {"planted_alpha": w.zipf_alpha, "fitted_slope_mean": float(np.mean(slopes)),
                "fitted_slope_min": float(np.min(slopes)), "fitted_slope_max": float(np.max(slopes)),
                "ranks": "16 .. N/16, layer 0, every KV head"}

    nb = op_bytes(w, Ksum, elem)
    nb["refine_select"] = nb["refine"] + nb["select"]
    if args.nestedkv:
        nb["score"] = w.L * w.Hkv * w.T * (w.d * elem + 4)  # K read once, s written
    dom = max(op_ms, key=op_ms.get)
    traffic = None
    if (dom == "score" and SCORE_TRAFFIC is not None and SCORE_TRAFFIC["workload"] == w.wid
            and SCORE_TRAFFIC["sha256"] == _score_source_sha()):
        traffic = SCORE_TRAFFIC["fetch_bytes"] + SCORE_TRAFFIC["write_bytes"]
    ach = nb[dom] / (op_ms[dom] / 1e3) / 1e9
    rsc_bytes = nb["refine"] + nb["select"] + nb["compact"]
    rsc_ms = sum(op_ms[k] for k in op_ms if k != "score")
    mfma_util = score_flops(w) / (op_ms["score"] / 1e3) / (BF16_PEAK_TFLOPS * 1e12)
    # one 64-row group per KV head runs score_pass_mfma, several score_pass_shared
    sk = "score_pass_mfma" if (w.Hq // w.Hkv) * w.W <= 64 else "score_pass_shared"
    kernels = {"score": f"{sk}<1> (row partials) + {sk}<2> (fold, column sums)" if elem == 2 else
               "score_stats_f32 + score_combine + score_probs_f32 + stats_final",
               "refine": "refine_kernel",
               "refine_select": "msel_bin<refine> + msel_pick",
               "select": ("lsel_init + lsel_floor_level<0..2> + lsel_pool_level<0..2> + lsel_count"
                          " + lsel_emit_count + lsel_emit") if args.layer_budget else "select_kernel",
               "compact": "compact_layer_kernel" if args.layer_budget else "compact_kernel"}
    if args.nestedkv:
        kernels["score"] = "nkv_tile_sum + nkv_block_sum + nkv_anomaly + nkv_route"

    roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ach / HBM_PEAK_GBS, "traffic": traffic, "op": dom,
            "kernels": kernels[dom], "algorithmic_bytes": nb[dom]}
    # a bf16 score whose one-sweep flops per algorithmic byte exceed the
    # ridge (2.5 PFLOP/s over 8 TB/s) is priced against the MFMA peak instead
    if dom == "score" and not args.nestedkv and elem == 2:
        fl = score_flops(w)
        if fl / nb["score"] > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            tf = fl / (op_ms["score"] / 1e3) / 1e12
            roof = {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tf / BF16_PEAK_TFLOPS, "traffic": traffic, "op": dom,
                    "kernels": kernels[dom], "algorithmic_flops": fl,
                    "algorithmic_bytes": nb[dom]}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.set_threads(nthreads)
        used = oracle.get_threads()
        # bounded sample: whole prefill chains of layer 0 (of the first
        # sequence only when there are several), repeated for about the CPU
        # budget (at least once)
        ws = w.with_(L=1) if w.B == 1 else w.with_(L=1, seqlens=w.seqlens[:1],
                                                    clusters=(w.clusters[:1] if w.clusters else None))
        q0, k0, v0 = layer0
        if w.B > 1:
            n0 = w.seqlens[0]
            q0 = q0[:, :w.W]
            k0, v0 = k0[:, :n0], v0[:, :n0]
        q0, k0, v0 = q0[None], k0[None], v0[None]
        def chain():
            if args.nestedkv:
                z0 = oracle.nestedkv(k0, ws.seqlens)
                kb0 = ws.kept()
                i0, h0 = oracle.select_layer(z0, ws.seqlens, [[ws.Hkv * int(x) for x in kb0]],
                                             ws.n_sink, ws.n_recent, int(min(kb0)) // 4)
                oracle.compact_layer(k0, v0, i0, h0, ws.seqlens)
            elif args.layer_budget:
                s0, st0 = oracle.score(q0, k0, ws.seqlens, ws.W, ws.scale, ws.causal)
                z0 = oracle.refine(s0, ws.seqlens, oracle.beta(st0, ws.seqlens, ws.beta_lo,
                                                              ws.beta_hi), ws.pool, ws.gamma, ws.r)
                kb0 = ws.kept()
                i0, h0 = oracle.select_layer(z0, ws.seqlens, [[ws.Hkv * int(x) for x in kb0]],
                                             ws.n_sink, ws.n_recent, int(min(kb0)) // 4)
                oracle.compact_layer(k0, v0, i0, h0, ws.seqlens)
            else:
                oracle.prefill_chain(q0, k0, v0, ws)

        reps, tc0 = 0, time.perf_counter()
        while True:
            chain()
            reps += 1
            if time.perf_counter() - tc0 >= args.cpu_budget_s or reps >= 50:
                break
        tc = (time.perf_counter() - tc0) / reps
        # one chain on one thread, when that is expected to take at most 30 s
        one = None
        if tc * used <= 30.0:
            oracle.set_threads(1)
            t1c = time.perf_counter()
            chain()
            one = float(ws.T) / (time.perf_counter() - t1c)
            oracle.set_threads(nthreads)
        cpu = {"value": float(ws.T) / tc, "unit": "tokens/s/head", "cores": used, "kind": "oracle",
               "cpu_model": _cpu_model(), "value_1thread": one,
               "sample": f"{reps} prefill chain(s) of layer 0" +
                         (f", sequence 0 ({ws.T} tokens)" if w.B > 1 else f" ({ws.T} tokens)") +
                         f", {ws.Hkv} KV heads, {tc:.2f} s each" +
                         ("; one more on one thread" if one is not None else "")}

    out = {
        "metric": "scored+selected KV tokens/sec per head",
        "value": value,
        "unit": "tokens/s/head",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "seqlens": list(w.seqlens), "layers": w.L, "Hq": w.Hq,
                   "Hkv": w.Hkv, "d": w.d, "window": w.W, "budget": w.budget, "r": w.r,
                   "n_sink": w.n_sink, "n_recent": w.n_recent, "kept_per_head": int(Ksum),
                   "budget_scope": "layer" if args.layer_budget else "head",
                   "scorer": "nestedkv" if args.nestedkv else "attention-mass",
                   "head_floor": floor if args.layer_budget else None,
                   "zipf_mass": zipf,
                   "launch": "hip graph replay of one step" if args.graph else "eager",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "token_heads_per_s": value * w.Hkv,  # aggregate over the KV heads
        "ops_ms": op_ms,
        "refine_select_compact": {"ms": rsc_ms, "bytes": rsc_bytes,
                                  "GBs": rsc_bytes / (rsc_ms / 1e3) / 1e9,
                                  "frac_hbm": rsc_bytes / (rsc_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "score_mfma": None if args.nestedkv else {"flops_one_sweep": score_flops(w),
                                                  "util": mfma_util,
                                                  "util_executed": 2 * mfma_util,  # two sweeps
                                                  "peak_tflops": BF16_PEAK_TFLOPS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
