"""Benchmark of the TokenGate pruned-prefill hot path on one MI355X.

One step = gate score -> top-K select -> compaction of the kept rows (hidden,
Q, K, V, scores) -> token-gated attention over the kept rows, on one batch of
synthetic input already resident in HBM, launched as one HIP graph.  The
variant whose attention reads Q, K, V and the scores through the kept indices
(gather on load, compacting only hidden rows and scores) is timed beside it.  The headline workload is the
16K-token gated layer (16320 document + 64 question tokens, d = 2048, gate
MLP 2048 -> 256 -> 1, K = 2048, 16 query / 8 key-value heads, head_dim 128).
The 128K-token layer at K = 2048 is measured too and reported beside it, and
so is the 28-layer pruned-stack prefill over a 65536-token prompt (13 full
layers, the gate, K = 4096, 15 token-gated layers) next to the same stack
unpruned.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-long | --only-long] [--no-stack | --only-stack]

Prints one JSON line.  Per-kernel times come from HIP events recorded on the
stream the kernels run on, inside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "gated prefill tokens/s at N=16K/128K, K=2K; attention TFLOP/s as % of MFMA peak"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Pipeline:
    """Device-resident inputs, outputs and workspaces of one gated layer."""

    def __init__(self, layer, k_budget, torch, tg, gather=False, query_tau=False, prepacked=True):
        assert not (gather and query_tau)
        self.torch, self.tg, self.gather, self.query_tau = torch, tg, gather, query_tau
        self.prepacked = prepacked
        dev = torch.device("cuda")
        seg = layer.segments.with_budget(k_budget)
        self.layer, self.seg = layer, seg

        def bf(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        def f32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

        self.plan = tg.plan_from(seg, device=dev)
        m = self.plan.total_kept
        self.n, self.m = seg.n_tokens, m
        self.x, self.w1, self.w2 = bf(layer.x), bf(layer.w1), f32(layer.w2)
        # the gate's W1 in MFMA fragment order, packed once (weights are constant across steps)
        self.w1p = tg.gate_pack_w1(self.w1) if prepacked else None
        self.q, self.k, self.v = bf(layer.q), bf(layer.k), bf(layer.v)
        self.tau, self.gain = f32(layer.tau), f32(layer.gain)
        self.scores = torch.empty(self.n, dtype=torch.float32, device=dev)
        self.kept = torch.empty(m, dtype=torch.int32, device=dev)
        self.gws = torch.empty(max(tg.gate_workspace_bytes(self.plan, layer.d, layer.h), 256), dtype=torch.uint8, device=dev)
        self.sws = torch.empty(max(tg.select_workspace_bytes(self.plan), 256), dtype=torch.uint8, device=dev)
        self.hc = torch.empty((m, layer.d), dtype=torch.bfloat16, device=dev)
        self.qc = torch.empty((m, layer.hq, layer.head_dim), dtype=torch.bfloat16, device=dev)
        self.kc = torch.empty((m, layer.hkv, layer.head_dim), dtype=torch.bfloat16, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.sc = torch.empty(m, dtype=torch.float32, device=dev)
        self.out = torch.empty_like(self.qc)
        # zero-filled once; the attention leaves its merge counters at zero (size 0: no query tile is split)
        self.aws = tg.attention_prefill_workspace(self.plan, layer.hq, layer.hkv, layer.head_dim, dev)
        # gather on load: attention reads Q, K, V and the scores through the kept indices, so only the
        # rows the next layer needs (hidden state, scores) are compacted
        self.pairs = ([(self.x, self.hc), (self.scores, self.sc)] if gather else
                      [(self.x, self.hc), (self.q, self.qc), (self.k, self.kc), (self.v, self.vc),
                       (self.scores, self.sc)])
        if query_tau:
            # per-query temperature with softplus(sigma_h) = tau_h; the original positions of the kept
            # rows are compacted with the other rows
            self.sigma = f32(np.log(np.expm1(layer.tau.astype(np.float64))))
            self.pos = torch.from_numpy(np.concatenate(
                [np.arange(seg.seg_len(i), dtype=np.int32) for i in range(seg.n_seg)])).to(dev)
            self.pc = torch.empty(m, dtype=torch.int32, device=dev)
            self.pairs.append((self.pos, self.pc))

    def stages(self):
        tg = self.tg
        return [
            ("gate", (lambda: tg.gate_score_prepacked(self.x, self.w1p, self.layer.h, None, self.w2, 0.0, self.plan,
                                                      scores=self.scores, workspace=self.gws))
             if self.prepacked else
             (lambda: tg.gate_score(self.x, self.w1, None, self.w2, 0.0, self.plan, scores=self.scores,
                                    workspace=self.gws))),
            ("select", lambda: tg.select_topk(self.scores, self.plan, kept_idx=self.kept, workspace=self.sws)),
            ("compact", lambda: tg.compact_kept(self.kept, self.pairs)),
            ("attention", (lambda: tg.gated_attention_prefill_gather(
                self.q, self.k, self.v, self.scores, self.tau, self.gain, self.plan, self.kept, out=self.out,
                workspace=self.aws))
             if self.gather else
             (lambda: tg.gated_attention_prefill_query_tau(self.qc, self.kc, self.vc, self.sc, self.sigma, self.gain,
                                                           self.pc, self.plan, out=self.out, workspace=self.aws))
             if self.query_tau else
             (lambda: tg.gated_attention_prefill(self.qc, self.kc, self.vc, self.sc, self.tau, self.gain, self.plan,
                                                 out=self.out, workspace=self.aws))),
        ]

    # algorithmic work (what the method must do), per launch
    def gate_bytes(self):
        L = self.layer
        n_doc = self.seg.n_doc(0)
        return 2 * n_doc * L.d + 2 * L.d * L.h + 4 * L.h + 4 * self.n

    def gate_flops(self):
        L = self.layer
        n_doc = self.seg.n_doc(0)
        return 2 * n_doc * L.d * L.h + 2 * n_doc * L.h

    def compact_row_bytes(self):
        L = self.layer
        return (2 * L.d + 4 + (0 if self.gather else 2 * L.hq * L.head_dim + 2 * 2 * L.hkv * L.head_dim)
                + (4 if self.query_tau else 0))

    def select_compact_bytes(self):
        return 4 * self.seg.n_doc(0) + 4 * self.m + 4 * self.m + 2 * self.m * self.compact_row_bytes()

    def compact_bytes(self):
        return 4 * self.m + 2 * self.m * self.compact_row_bytes()

    def attention_flops(self):
        L = self.layer
        return 4 * L.hq * L.head_dim * self.m * (self.m + 1) // 2


def time_pipeline(pipe, steps, warmup):
    torch = pipe.torch
    stages = pipe.stages()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, (_, f) in enumerate(stages):
            f()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_stage = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)])) * 1e3
                 for j, (name, _) in enumerate(stages)}
    gpu_step = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(steps)])) * 1e3
    return wall / steps * 1e6, gpu_step, per_stage


def time_stage_kernels(pipe, reps=20):
    """Average duration of each stage's kernels (`events_us`: the stage captured
    `reps` times in a row in one HIP graph, so its launches run back to back with
    no host work between them), after one whole step so that every stage's
    inputs are valid (every stage is idempotent).  Unlike the eager per-stage
    intervals of `time_pipeline`, this leaves out the host's launch gaps."""
    torch = pipe.torch
    stages = pipe.stages()
    for _, f in stages:
        f()
    return {name: events_us(torch, f, reps) for name, f in stages}


def capture_step(pipe):
    """One step (all stages) captured as a HIP graph on a side stream; every
    buffer is preallocated, and no stage allocates, synchronises or memsets."""
    torch = pipe.torch
    stages = pipe.stages()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the stream before capture
        for _, f in stages:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, f in stages:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(pipe, steps, warmup):
    """Wall time per step of graph replays, bracketed by device synchronisation."""
    torch = pipe.torch
    g = capture_step(pipe)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e6


def time_graph_cold(pipe, steps, flush_bytes=1 << 30):
    """Per-step time of graph replays that each start with the last-level cache
    holding none of the step's data: before every replay a 1 GiB buffer (four
    times the 256 MiB cache) is overwritten, outside the events that time the
    replay."""
    torch = pipe.torch
    g = capture_step(pipe)
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    g.replay()
    times = []
    for _ in range(steps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return float(np.median(times))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layer, k_budget, budget_s=10.0, threads=None):
    """The oracle (as it stands) on the same 16K workload, timed on the host cores (all the BLAS threads the
    host offers, or `threads`): whole-layer runs repeated until `budget_s` seconds have passed (at least 3,
    at most 30 runs)."""
    import oracle
    from learned_token_pruning_amd import workloads as W
    from contextlib import nullcontext
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ctx = threadpool_limits(threads) if threads else nullcontext()
    except Exception:  # pragma: no cover
        threadpool_info, ctx = None, nullcontext()
    seg = layer.segments.with_budget(k_budget)
    x, w1 = W.bf16_bits_to_f64(layer.x), W.bf16_bits_to_f64(layer.w1)
    q, k, v = (W.bf16_bits_to_f64(a) for a in (layer.q, layer.k, layer.v))
    reps, t_total = 0, 0.0
    with ctx:
        used = (max([p.get("num_threads", 1) for p in threadpool_info()] + [1]) if threadpool_info
                else (os.cpu_count() or 1))
        while reps < 3 or (t_total < budget_s and reps < 30):
            t0 = time.perf_counter()
            s = oracle.gate_scores(x, w1, None, layer.w2.astype(np.float64), 0.0, seg.seg_start, seg.doc_begin,
                                   seg.doc_end)
            idx, offs = oracle.kept_indices(s, seg.seg_start, seg.doc_begin, seg.doc_end, seg.k_budget)
            hc, qc, kc, vc, sc = (oracle.compact_rows(a, idx) for a in (x, q, k, v, s))
            oracle.gated_attention(qc, kc, vc, sc, layer.tau.astype(np.float64), layer.gain.astype(np.float64), offs)
            t_total += time.perf_counter() - t0
            reps += 1
    t = t_total / reps
    return {"value": seg.n_tokens / t, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"full 16K-token gated layer (gate over {seg.n_doc(0)} documents, select, compaction, "
                      f"attention over {idx.size} kept rows), float64 NumPy, mean of {reps} run(s), "
                      f"{t:.2f} s each"}


def events_us(torch, f, reps, warm=3, replays=5):
    """Mean time of f(): `reps` calls captured back to back in one HIP graph (no
    host work between the launches), timed by events around a replay on the
    current stream; median of `replays` replays.  f must allocate nothing and
    may be re-run on the same buffers."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the stream before capture
        for _ in range(warm):
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            f()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / reps * 1e3)
    del g
    return float(np.median(ts))


def time_k_sweep(torch, tg, reps=50):
    """The 32K-token layer (32704 documents + 64 question tokens) at every budget K in {1024, 2048, 4096, 8192}:
    the select on the fp32 mixture scores of that workload (95 % N(0,1), 5 % N(4, 0.5), exact duplicates, ties
    planted across every K), the compaction of H, Q, K, V and the scores, and the attention over the kept rows
    (with split query tiles when the prompt is too short to fill the GPU); the gate once (it does not depend on
    K).  Rooflines: attention against the bf16 MFMA peak, select + compaction against HBM."""
    from learned_token_pruning_amd import workloads as W
    dev = torch.device("cuda")
    L = W.workload(3)
    seg0 = L.segments
    s_host = W.mixture_scores(3, seg0, k_marks=(1024, 2048, 4096, 8192))
    rec = {"workload": "gated layer N=32768 (32704 doc + 64 question), d=2048, gate 2048-256-1, 16 Q / 8 KV heads, "
                       "head_dim 128; select input: fp32 mixture scores", "by_k": {}}
    p = Pipeline(L, 1024, torch, tg)
    rec["gate_us"] = round(events_us(torch, p.stages()[0][1], reps), 2)
    gf = p.gate_flops()
    rec["gate_roofline"] = {"bound": "hbm", "achieved": p.gate_bytes() / (rec["gate_us"] * 1e-6) / 1e9,
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "mfma_tflops": gf / (rec["gate_us"] * 1e-6) / 1e12}
    rec["gate_roofline"]["frac"] = rec["gate_roofline"]["achieved"] / HBM_PEAK_GBS
    rec["gate_roofline"]["mfma_frac"] = rec["gate_roofline"]["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS
    del p
    s_dev = torch.from_numpy(s_host).to(dev)
    for kb in (1024, 2048, 4096, 8192):
        pk = Pipeline(L, kb, torch, tg)
        pk.scores.copy_(s_dev)  # the select input of this workload
        st = dict(pk.stages())
        t_sel = events_us(torch, st["select"], reps)
        t_cmp = events_us(torch, st["compact"], reps)
        t_att = events_us(torch, st["attention"], reps)
        sc_bytes = pk.select_compact_bytes()
        att = pk.attention_flops() / (t_att * 1e-6) / 1e12
        sc_gbs = sc_bytes / ((t_sel + t_cmp) * 1e-6) / 1e9
        rec["by_k"][str(kb)] = {
            "kept_rows": pk.m, "select_us": round(t_sel, 2), "compact_us": round(t_cmp, 2),
            "attention_us": round(t_att, 2),
            "attention_roofline": {"bound": "mfma", "achieved": att, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": att / MFMA_BF16_PEAK_TFLOPS},
            "select_plus_compact_roofline": {"bound": "hbm", "achieved": sc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                             "frac": sc_gbs / HBM_PEAK_GBS, "bytes": sc_bytes,
                                             "frac_of_copy_rate": sc_gbs / COPY_GBS if COPY_GBS else None}}
        log(f"K sweep K={kb}: select {t_sel:.1f} us, compact {t_cmp:.1f} us, attention {t_att:.1f} us "
            f"({att:.0f} TFLOP/s)")
        del pk
        torch.cuda.empty_cache()
    return rec


def time_bias_ratio(torch, tg, reps=50):
    """The same attention launch with the gate bias (key scores and gains) and without it (key_score = NULL):
    one prompt of M kept rows, 16 Q / 8 KV heads, head_dim 128, with the temperature in both.  The pages quote
    1.0-1.1x for the biased call of their FlashAttention-2 kernel on A100."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(79)
    hq, hkv, dh = 16, 8, 128
    rec = {"workload": "token-gated attention with vs without the key-score bias, one prompt of M kept rows, "
                       "16 Q / 8 KV heads, head_dim 128"}
    for m in (2112, 4160):
        q = torch.randn(m, hq, dh, generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn(m, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(m, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        sc = torch.randn(m, generator=gen, device=dev)
        tau = 0.8 + 0.4 * torch.rand(hq, generator=gen, device=dev)
        gain = 0.5 + torch.rand(hq, generator=gen, device=dev)
        plan = tg.plan_segments([0, m], [0], [0], [0], device=dev)
        ws = tg.attention_prefill_workspace(plan, hq, hkv, dh, dev)
        out = torch.empty_like(q)
        on, off = [], []
        for _ in range(3):  # interleaved
            on.append(events_us(torch, lambda: tg.gated_attention_prefill(q, k, v, sc, tau, gain, plan, out=out,
                                                                        workspace=ws), reps))
            off.append(events_us(torch, lambda: tg.gated_attention_prefill(q, k, v, None, tau, None, plan, out=out,
                                                                         workspace=ws), reps))
        a, b = float(np.median(on)), float(np.median(off))
        rec[f"m{m}"] = {"bias_us": round(a, 2), "no_bias_us": round(b, 2), "ratio": a / b}
        del q, k, v, ws
    return rec


def time_select_sweep(torch, tg, reps=20):
    """The select alone on batches of many prompts, where it reads enough scores to be bandwidth-bound: 64
    prompts of 16384 tokens (one workgroup per prompt) and 64 prompts of 131072 tokens (the multi-workgroup
    path), each prompt 64 question tokens after its document, K = 2048 and 4096; N(0,1) fp32 scores.  Bytes:
    4 per token read, 4 per kept row written."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(80)
    rec = {"workload": "select over 64-prompt batches, N(0,1) fp32 scores, 64 question tokens per prompt"}
    for n_tok in (16384, 131072):
        for kb in (2048, 4096):
            nseg = 64
            offs = [i * n_tok for i in range(nseg + 1)]
            plan = tg.plan_segments(offs, [0] * nseg, [n_tok - 64] * nseg, [kb] * nseg, device=dev)
            s = torch.randn(n_tok * nseg, generator=gen, device=dev)
            kept = torch.empty(plan.total_kept, dtype=torch.int32, device=dev)
            ws = torch.empty(max(tg.select_workspace_bytes(plan), 256), dtype=torch.uint8, device=dev)
            us = events_us(torch, lambda: tg.select_topk(s, plan, kept_idx=kept, workspace=ws), reps)
            nbytes = 4 * n_tok * nseg + 4 * plan.total_kept
            gbs = nbytes / (us * 1e-6) / 1e9
            rec[f"{nseg}x{n_tok}_k{kb}"] = {"us": round(us, 2), "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                                            "frac_of_copy_rate": gbs / COPY_GBS if COPY_GBS else None}
            log(f"select sweep {nseg}x{n_tok} K={kb}: {us:.1f} us, {gbs:.0f} GB/s")
            del s, kept, ws
    torch.cuda.empty_cache()
    return rec


def kernel_traffic(kernel_source):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (profiles/traffic.json), or None when the kernel source has
    changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)[os.path.basename(kernel_source)]
        with open(kernel_source, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == sha else None


def copy_rate_gbs(torch, reps=20):
    """Read + write bytes per second of a plain 1 GiB device-to-device copy on
    this GPU: the practical HBM rate that the published peak overstates."""
    x = torch.empty(2 ** 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    del x, y
    torch.cuda.empty_cache()
    return 2 * 2 ** 30 / (us * 1e-6) / 1e9


COPY_GBS = None  # set in main()


def stage_rooflines(pipe, st, csrc):
    """Roofline entry of every stage: algorithmic work / the stage's kernel time
    (`time_stage_kernels`)."""
    attn_tflops = pipe.attention_flops() / (st["attention"] * 1e-6) / 1e12
    gate_gbs = pipe.gate_bytes() / (st["gate"] * 1e-6) / 1e9
    compact_gbs = pipe.compact_bytes() / (st["compact"] * 1e-6) / 1e9
    select_gbs = (4 * pipe.seg.n_tokens + 4 * pipe.m) / (st["select"] * 1e-6) / 1e9
    roofs = {
        "attention": {"kernel": "gated_attention_dma_kernel<128,2>", "bound": "mfma", "achieved": attn_tflops,
                      "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS,
                      "traffic": kernel_traffic(os.path.join(csrc, "gated_attention.hip"))},
        "gate": {"kernel": ("" if pipe.prepacked else "pack_w1_kernel + ") + "gate_mlp_kernel<2,4> + gate_normalize_kernel",
                 "bound": "hbm",
                 "achieved": gate_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gate_gbs / HBM_PEAK_GBS,
                 "traffic": kernel_traffic(os.path.join(csrc, "gate_score.hip")),
                 "mfma_tflops": pipe.gate_flops() / (st["gate"] * 1e-6) / 1e12},
        "compact": {"kernel": "compact_kernel", "bound": "hbm", "achieved": compact_gbs, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": compact_gbs / HBM_PEAK_GBS,
                    "traffic": kernel_traffic(os.path.join(csrc, "compact.hip"))},
        "select": {"kernel": "select_topk_kernel", "bound": "hbm", "achieved": select_gbs, "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": select_gbs / HBM_PEAK_GBS,
                   "traffic": kernel_traffic(os.path.join(csrc, "select_topk.hip"))},
    }
    if COPY_GBS:
        for r in roofs.values():
            if r["bound"] == "hbm":
                r["frac_of_copy_rate"] = r["achieved"] / COPY_GBS
    return roofs


def time_decode(torch, tg, reps=200):
    """One decode step of token-gated attention for 32 sequences whose 16K-token
    prompts were pruned to K = 2048 (2112 kept rows + 1 generated row in the
    cache), against the same step over the unpruned caches (16385 rows): 16 Q /
    8 KV heads, head_dim 128, random bf16 caches, fp32 scores (0 on the
    generated row).  Kernel time from events around `reps` back-to-back steps."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(77)
    bsz, hq, hkv, dh = 32, 16, 8, 128
    tau = 0.8 + 0.4 * torch.rand(hq, generator=gen, device=dev)
    gain = 0.5 + torch.rand(hq, generator=gen, device=dev)
    rec = {"workload": "decode step, 32 sequences, 16 Q / 8 KV heads, head_dim 128: pruned caches "
                       "(16K prompt, K=2048: 2112 kept + 1 generated rows) vs unpruned caches (16385 rows)"}
    for name, cap in (("pruned", 2113), ("full", 16385)):
        q = torch.randn(bsz, hq, dh, generator=gen, device=dev).to(torch.bfloat16)
        kc = torch.randn(bsz, cap, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        vc = torch.randn(bsz, cap, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        sc = torch.randn(bsz, cap, generator=gen, device=dev)
        sc[:, -1] = 0.0
        lens = torch.full((bsz,), cap, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(tg.decode_workspace_bytes(bsz, hq, dh, cap), dtype=torch.uint8, device=dev)
        step = lambda: tg.gated_attention_decode(q, kc, vc, sc, tau, gain, lens, out=out, workspace=ws)
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        nbytes = bsz * cap * (2 * hkv * dh * 2 + 4) + 2 * bsz * hq * dh * 2  # K, V, scores once; q and out
        gbs = nbytes / (us * 1e-6) / 1e9
        rec[name] = {"cache_rows": cap, "us_per_step": round(us, 2), "kv_gib": bsz * cap * 2 * hkv * dh * 2 / 2 ** 30,
                     "roofline": {"kernel": "decode_partial_kernel<128,2> + decode_combine_kernel<128>",
                                  "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                                  "frac_of_copy_rate": gbs / COPY_GBS if COPY_GBS else None}}
        del q, kc, vc, sc, ws
        torch.cuda.empty_cache()
    rec["speedup_pruned_vs_full"] = rec["full"]["us_per_step"] / rec["pruned"]["us_per_step"]
    return rec


def time_backward(torch, tg, reps=20):
    """Forward with the saved log-sum-exp, then the backward (dq, dk, dv and
    the key-score / gain / temperature gradients) of token-gated attention over
    M kept rows of one prompt: 16 Q / 8 KV heads, head_dim 128, random bf16
    inputs.  Algorithmic work: forward 4 hq D M(M+1)/2 flop (QK and PV over
    the causal pairs), backward 2.5x that (QK recompute, dP, dV, dK, dQ)."""
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(78)
    hq, hkv, dh = 16, 8, 128
    rec = {"workload": "token-gated attention backward, one prompt of M kept rows, 16 Q / 8 KV heads, head_dim 128"}
    for m in (2112, 4160):
        q = torch.randn(m, hq, dh, generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn(m, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(m, hkv, dh, generator=gen, device=dev).to(torch.bfloat16)
        do = torch.randn(m, hq, dh, generator=gen, device=dev).to(torch.bfloat16)
        sc = torch.randn(m, generator=gen, device=dev)
        tau = 0.8 + 0.4 * torch.rand(hq, generator=gen, device=dev)
        gain = 0.5 + torch.rand(hq, generator=gen, device=dev)
        plan = tg.plan_segments([0, m], [0], [0], [0], device=dev)
        out, lse = tg.gated_attention_prefill_lse(q, k, v, sc, tau, gain, plan)
        ws = torch.empty(max(tg.attention_backward_workspace_bytes(plan, hq, hkv, dh), 256), dtype=torch.uint8, device=dev)

        def timed(f):
            for _ in range(3):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e3

        us_f = timed(lambda: tg.gated_attention_prefill_lse(q, k, v, sc, tau, gain, plan, out=out, lse=lse))
        us_b = timed(lambda: tg.gated_attention_backward(q, k, v, sc, tau, gain, plan, out, do, lse, workspace=ws))
        fwd = 4 * hq * dh * m * (m + 1) // 2
        tf_b = 2.5 * fwd / (us_b * 1e-6) / 1e12
        rec[f"m{m}"] = {"forward_lse_us": round(us_f, 2), "backward_us": round(us_b, 2),
                        "forward_tflops": fwd / (us_f * 1e-6) / 1e12,
                        "roofline": {"kernel": "bwd_rowdot + bwd_dkdv<128,2> + bwd_dq<128,2> + bwd_reduce",
                                     "bound": "mfma", "achieved": tf_b, "peak": MFMA_BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": tf_b / MFMA_BF16_PEAK_TFLOPS, "traffic": None}}
        del q, k, v, do, out, lse, ws
        torch.cuda.empty_cache()
    return rec


STACK = dict(n=65536, n_q=64, k=4096, layers=28, gate_layer=12, d=2048, hq=16, hkv=8, dh=128, f=6144, h_gate=256)


def stack_flops(rows_per_segment, c):
    """Model flops of one decoder layer over prompts of the given lengths:
    the four projections (2 flop per multiply-add) plus causal attention
    (QK and PV over the causal pairs only)."""
    d, hq, hkv, dh, f = c["d"], c["hq"], c["hkv"], c["dh"], c["f"]
    m = sum(rows_per_segment)
    proj = 2 * m * (d * (hq + 2 * hkv) * dh + hq * dh * d + d * 2 * f + f * d)
    attn = sum(4 * hq * dh * r * (r + 1) // 2 for r in rows_per_segment)
    return proj, attn


def time_stack(torch, tg, steps, warmup):
    """28-layer random-init stack over a 65536-token prompt: 13 full layers,
    the gate on layer 13's normalised residual, top-4096 select, compaction,
    15 token-gated layers over 4096 + 64 kept rows; and the same stack with no
    pruning.  Returns the record of both."""
    from learned_token_pruning_amd.stack import PrunedStack, random_layers
    c = STACK
    dev = torch.device("cuda")
    n, nq = c["n"], c["n_q"]
    layers = random_layers(5, c["layers"], c["gate_layer"] + 1, c["d"], c["hq"], c["hkv"], c["dh"], c["f"], dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(50)
    w1 = (torch.randn(c["h_gate"], c["d"], generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    w2 = torch.randn(c["h_gate"], generator=gen, device=dev) * 0.02
    x = torch.randn(n, c["d"], generator=gen, device=dev).to(torch.bfloat16)
    st = PrunedStack(layers, c["gate_layer"], w1, w2, c["d"], c["hq"], c["hkv"], c["dh"], c["f"])
    plan = st.plan([0, n], [0], [n - nq], [c["k"]], dev)
    stream = torch.cuda.current_stream()
    rec = {}
    for prune in (True, False):
        for _ in range(warmup):
            st.forward(x, plan=plan, prune=prune)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        phases = []
        t0 = time.perf_counter()
        for _ in range(steps):
            ev = {"start": torch.cuda.Event(enable_timing=True)}
            ev["start"].record(stream)

            def mark(name, ev=ev):
                ev[name] = torch.cuda.Event(enable_timing=True)
                ev[name].record(stream)

            st.forward(x, plan=plan, prune=prune, mark=mark)
            phases.append(ev)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        names = ["lower", "prune", "upper"] if prune else ["lower", "upper"]
        ph = {}
        prev = "start"
        for nm in names:
            ph[nm] = float(np.mean([e[prev].elapsed_time(e[nm]) for e in phases]))
            prev = nm
        m_up = plan.pruned.total_kept if prune else n
        lo = stack_flops([n], c)
        up = stack_flops([m_up], c)
        n_lo, n_up = c["gate_layer"] + 1, c["layers"] - c["gate_layer"] - 1
        flops = n_lo * sum(lo) + n_up * sum(up)
        attn_flops = n_lo * lo[1] + n_up * up[1]
        key = "pruned" if prune else "full"
        rec[key] = {"ms": wall * 1e3, "tokens_per_s": n / wall, "phases_ms": {k: round(v, 3) for k, v in ph.items()},
                    "model_tflops": flops / wall / 1e12, "model_frac_mfma_peak": flops / wall / 1e12 /
                    MFMA_BF16_PEAK_TFLOPS, "attention_share_of_flops": attn_flops / flops,
                    "peak_device_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30}
        log(f"stack {key}: {wall * 1e3:.1f} ms/step", ph)
    # the same pruned forward captured as one graph (all 28 layers, gate, select, compaction) and replayed
    eager = st.forward(x, plan=plan)
    graph = st.capture(x, plan)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        out = graph.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    same = bool(torch.equal(out["kept"], eager["kept"]) and
                torch.equal(out["hidden"].view(torch.int16), eager["hidden"].view(torch.int16)))
    rec["pruned_graph"] = {"ms": wall * 1e3, "tokens_per_s": n / wall, "equal_to_eager": same}
    log(f"stack pruned, graph replay: {wall * 1e3:.1f} ms/step (bitwise equal to eager: {same})")
    del eager, graph, out
    rec["prefill_speedup"] = rec["full"]["ms"] / rec["pruned"]["ms"]
    rec["workload"] = (f"pruned-stack prefill, 28 random-init layers (d 2048, 16 Q / 8 KV heads, head_dim 128, "
                       f"SwiGLU 6144), N={n} ({n - nq} doc + {nq} question), 13 full layers, gate after layer 13, "
                       f"K={c['k']} (M={plan.pruned.total_kept}), 15 token-gated layers; and the same stack unpruned")
    rec["steps"], rec["warmup"] = steps, warmup
    kv_row = 2 * c["hkv"] * c["dh"] * 2
    rec["kv_cache_gib_if_kept"] = {
        "pruned": ((c["gate_layer"] + 1) * n + (c["layers"] - c["gate_layer"] - 1) * plan.pruned.total_kept) * kv_row
        / 2 ** 30, "full": c["layers"] * n * kv_row / 2 ** 30}
    del st, layers, x
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 128K-token layer")
    ap.add_argument("--only-long", action="store_true", help="time only the 128K-token layer (profiling)")
    ap.add_argument("--no-stack", action="store_true", help="skip the 28-layer pruned-stack prefill")
    ap.add_argument("--only-stack", action="store_true", help="time only the 28-layer pruned-stack prefill")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step and backward timings")
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the decode step and the attention backward (profiling)")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the 32K K sweep, the bias on/off ratio and the batched select sweep")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (reference for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path is single-GPU here); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(os.path.join(ROOT, "learned_token_pruning_amd", "libtokengate.so")):
        from learned_token_pruning_amd import build as _b
        _b.build()
    from learned_token_pruning_amd import tokengate as tg
    from learned_token_pruning_amd import workloads as W
    csrc = os.path.join(ROOT, "learned_token_pruning_amd", "csrc")
    global COPY_GBS
    COPY_GBS = copy_rate_gbs(torch)
    log(f"device copy rate {COPY_GBS:.0f} GB/s (read + write)")

    if args.calibrate_copy:
        src = torch.empty(64 * 2 ** 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = None
    l16 = None
    if args.only_decode:
        args.only_long, args.no_long, args.no_stack, args.no_cpu_baseline = True, True, True, True
    elif args.only_stack:
        args.only_long, args.no_long = True, True
    elif args.only_long:
        args.no_stack = True
    if args.only_long and not args.only_decode:
        args.no_decode = True
    if not args.only_long:
        log("generating the 16K-token workload")
        l16 = W.workload(2)
        p16 = Pipeline(l16, 2048, torch, tg)
        log("timing 16K", args.steps, "steps")
        us_eager, us_gpu, st16 = time_pipeline(p16, args.steps, args.warmup)
        log("16K: eager", f"{us_eager:.1f} us/step, events {us_gpu:.1f} us/step", st16)
        us_wall = time_graph(p16, args.steps, args.warmup)
        log("16K: graph replay", f"{us_wall:.1f} us/step")
        us_cold = time_graph_cold(p16, max(5, args.steps // 4))
        log("16K: graph replay after a last-level-cache flush", f"{us_cold:.1f} us/step")
        p16g = Pipeline(l16, 2048, torch, tg, gather=True)
        us_gather = time_graph(p16g, args.steps, args.warmup)
        log("16K: graph replay, attention gathering Q/K/V", f"{us_gather:.1f} us/step")
        del p16g
        p16r = Pipeline(l16, 2048, torch, tg, prepacked=False)
        us_repack = time_graph(p16r, args.steps, args.warmup)
        log("16K: graph replay, W1 re-packed inside every step", f"{us_repack:.1f} us/step")
        del p16r
        p16t = Pipeline(l16, 2048, torch, tg, query_tau=True)
        us_qtau = time_graph(p16t, args.steps, args.warmup)
        _, _, st16t = time_pipeline(p16t, args.steps, args.warmup)
        log("16K: graph replay, per-query temperature", f"{us_qtau:.1f} us/step", st16t)
        del p16t
        kt16 = time_stage_kernels(p16)
        log("16K: kernel time per stage (repetitions inside one graph)", "", kt16)
        roofs = stage_rooflines(p16, kt16, csrc)
        dominant = max(kt16, key=kt16.get)
        sc_gbs = p16.select_compact_bytes() / ((kt16["select"] + kt16["compact"]) * 1e-6) / 1e9
        result = {
            "metric": METRIC,
            "value": p16.n / (us_wall * 1e-6),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": us_wall / 1e3,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "gated layer N=16384 (16320 doc + 64 question), d=2048, gate 2048-256-1, "
                                   "K=2048 (M=2112 kept), 16 Q / 8 KV heads, head_dim 128",
                       "global_batch": 1, "seq_len": p16.n, "k_budget": 2048, "kept_rows": p16.m,
                       "parallelism": "none", "launch": "one HIP graph per step (stages_us: eager launches, host gaps included; "
                                 "kernel_us and the rooflines: each stage repeated back to back inside one graph)",
                       "gate_weights": "W1 packed into MFMA fragment order once at load"},
            "roofline": dict(roofs[dominant], stage=dominant),
            "stages_us": {k: round(v, 2) for k, v in st16.items()},
            "kernel_us": {k: round(v, 2) for k, v in kt16.items()},
            "stage_rooflines": roofs,
            "gpu_us_per_step_events": round(us_gpu, 2),
            "cold_cache_us_per_step": round(us_cold, 2),
            "eager_us_per_step": round(us_eager, 2),
            "gather_on_load_us_per_step": round(us_gather, 2),
            "w1_repacked_every_step_us_per_step": round(us_repack, 2),
            "query_tau": {"us_per_step": round(us_qtau, 2), "attention_us": round(st16t["attention"], 2),
                          "note": "tau_rh = softplus(sigma_h) log(rank) / log(max(2, position)), graph replay"},
            "attention": {"tflops": roofs["attention"]["achieved"], "frac_mfma_peak": roofs["attention"]["frac"]},
            "select_plus_compact": {"gbs": sc_gbs, "frac_hbm_peak": sc_gbs / HBM_PEAK_GBS,
                                    "frac_of_copy_rate": sc_gbs / COPY_GBS},
        }
        del p16
        torch.cuda.empty_cache()

    if not args.no_long:
        log("generating the 128K-token workload")
        l128 = W.workload(4)
        torch.cuda.reset_peak_memory_stats()
        p128 = Pipeline(l128, 2048, torch, tg)
        steps = args.steps if args.only_long else max(10, args.steps // 4)
        us_eager128, us_gpu128, st128 = time_pipeline(p128, steps, max(3, args.warmup // 4))
        us_wall128 = time_graph(p128, steps, max(3, args.warmup // 4))
        kt128 = time_stage_kernels(p128, reps=10)
        log("128K: eager", f"{us_eager128:.1f} us/step, graph replay {us_wall128:.1f} us/step", st128)
        p128g = Pipeline(l128, 2048, torch, tg, gather=True)
        us_gather128 = time_graph(p128g, steps, max(3, args.warmup // 4))
        log("128K: graph replay, attention gathering Q/K/V", f"{us_gather128:.1f} us/step")
        del p128g
        long_rec = {
            "workload": "gated layer N=131072 (131008 doc + 64 question), d=2048, K=2048 (M=2112 kept)",
            "tokens_per_s": p128.n / (us_wall128 * 1e-6), "ms_per_step": us_wall128 / 1e3, "steps": steps,
            "eager_us_per_step": round(us_eager128, 2), "launch": "one HIP graph per step",
            "gather_on_load_us_per_step": round(us_gather128, 2),
            "stages_us": {k: round(v, 2) for k, v in st128.items()},
            "kernel_us": {k: round(v, 2) for k, v in kt128.items()},
            "stage_rooflines": stage_rooflines(p128, kt128, csrc),
            "peak_device_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30,
        }
        del p128
        torch.cuda.empty_cache()
        # the long-context configuration's own budget, K = 4096 (M = 4160 kept)
        torch.cuda.reset_peak_memory_stats()
        p128k = Pipeline(l128, 4096, torch, tg)
        us_eager4k, _, st4k = time_pipeline(p128k, steps, max(3, args.warmup // 4))
        us_wall4k = time_graph(p128k, steps, max(3, args.warmup // 4))
        kt4k = time_stage_kernels(p128k, reps=10)
        log("128K, K=4096: eager", f"{us_eager4k:.1f} us/step, graph replay {us_wall4k:.1f} us/step", st4k)
        long_rec4k = {
            "workload": "gated layer N=131072 (131008 doc + 64 question), d=2048, K=4096 (M=4160 kept)",
            "tokens_per_s": p128k.n / (us_wall4k * 1e-6), "ms_per_step": us_wall4k / 1e3, "steps": steps,
            "eager_us_per_step": round(us_eager4k, 2), "launch": "one HIP graph per step",
            "stages_us": {k: round(v, 2) for k, v in st4k.items()},
            "kernel_us": {k: round(v, 2) for k, v in kt4k.items()},
            "stage_rooflines": stage_rooflines(p128k, kt4k, csrc),
            "peak_device_mem_gib": torch.cuda.max_memory_allocated() / 2 ** 30,
        }
        del p128k, l128
        torch.cuda.empty_cache()
        if result is None:
            result = {"metric": METRIC, "value": long_rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                      "steps": steps, "warmup": args.warmup, "ms_per_step": long_rec["ms_per_step"],
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": long_rec["workload"]}}
        result["n131072_k2048"] = long_rec
        result["n131072_k4096"] = long_rec4k

    if not args.no_stack:
        log("timing the 28-layer pruned stack at N=65536")
        stack = time_stack(torch, tg, max(2, args.steps // 50), 1)
        if result is None:
            result = {"metric": METRIC, "value": stack["pruned"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                      "steps": stack["steps"], "warmup": 1, "ms_per_step": stack["pruned"]["ms"],
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                      "data": "synthetic", "config": {"workload": stack["workload"]}}
        result["stack_n65536_k4096"] = stack

    if args.only_decode:
        result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": 0,
                  "warmup": 0, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
                  "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                  "config": {"workload": "decode step and attention backward only (profiling mode)"}}
    if not args.only_long and not args.only_decode and result is not None and not args.no_sweeps:
        log("timing the K sweep of the 32K-token layer")
        result["n32768_k_sweep"] = time_k_sweep(torch, tg)
        log("timing attention with and without the gate bias")
        result["bias_on_off"] = time_bias_ratio(torch, tg)
        log("timing the batched select sweep")
        result["select_sweep"] = time_select_sweep(torch, tg)

    if not args.no_decode and result is not None:
        log("timing the decode step over pruned and unpruned caches")
        result["decode_b32"] = time_decode(torch, tg)
        log("decode", {k: v["us_per_step"] for k, v in result["decode_b32"].items() if isinstance(v, dict)})

    if not args.no_decode and result is not None:
        log("timing the attention backward")
        result["attention_backward"] = time_backward(torch, tg)
        log("backward", {k: v["backward_us"] for k, v in result["attention_backward"].items() if isinstance(v, dict)})

    if not args.no_cpu_baseline and l16 is not None:
        log("timing the CPU oracle on the 16K workload")
        result["cpu_baseline"] = cpu_baseline(l16, 2048)
        log("timing the CPU oracle on one core")
        result["cpu_baseline_1core"] = cpu_baseline(l16, 2048, budget_s=12.0, threads=1)
    result["hbm_copy_rate_gbs"] = COPY_GBS
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
