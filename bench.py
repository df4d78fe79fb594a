#!/usr/bin/env python3
"""Benchmark of the Q8_0 decode path on one MI355X.

Default workload: a Llama-2-110M-shaped decode step at batch 1 (12 layers of
wq/wk/wv/wo 768x768, w1/w3 2048x768, w2 768x2048, plus a 32000x768
classifier; 85 Q8_0 matvecs per step with weights N(0, 0.02) and a fresh
N(0,1) activation per matvec, quantized to Q8_0 before use), 200 sequential
steps.  The weights are repacked once, at load and outside the timed region,
into the row-interleaved R8 layout; one step is then ONE launch over all 85
products in which every workgroup quantizes the fp32 activation row of its
matrix (the native-layout forms of the same step are timed beside it).

Prints ONE JSON line: throughput (algorithmic bytes / s over the timed
steps), tokens/s, the roofline of the dominant kernel (the step launch, timed
with HIP events on the stream it runs on) and the CPU oracle timed on a
bounded sample of the same workload.  Timing protocol: the K steps are one HIP
graph; 11 rounds, the first dropped, each round the best of 3 replays of the
headline, the cold form (rotating weight copies) and the headline again as a
control series; value = the median of the rounds' bests; the control's
per-round ratios to the headline must straddle 1x; GPU clocks are recorded
(rocm-smi) before and after.  The same line carries the vocabulary projection
(262144 x 2048) and the 30-layer MoE expert FFN at 1 and 16 tokens (layer
after layer and grouped, native and R8 weights), timed in the same run.

Other workloads (one JSON line each), for the per-configuration tables:
  --workload c1      768x768 matvec
  --workload c3      GPT-2-124M-shaped batch-8 decode step (49 products)
  --workload c4b1    MoE expert FFN, 30 layers, 1 token
  --workload c4b16   MoE expert FFN, 30 layers, 16 tokens
  --workload c5a     prefill GEMM 512x4096 x 14336x4096
  --workload c5b     vocabulary projection 262144x2048
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q8_0 matvec achieved HBM GB/s (% of peak) and decode tokens/s-equivalent"
HBM_PEAK_GBS = 8000.0
BB = 34          # bytes per Q8_0 block
QK = 32


def q8_bytes(rows, k):
    return rows * (k // QK) * BB


# ---------------------------------------------------------------------------
# workload definitions (shapes only)

LLAMA_STACKS = [  # (name, n, k, batch): same-shape projections stacked
    ("wq_wk_wv_wo", 768, 768, 48),
    ("w1_w3", 2048, 768, 24),
    ("w2", 768, 2048, 12),
    ("classifier", 32000, 768, 1),
]

GPT2_STACKS = [
    ("c_attn", 2304, 768, 12),
    ("attn_c_proj", 768, 768, 12),
    ("c_fc", 3072, 768, 12),
    ("mlp_c_proj", 768, 3072, 12),
    ("lm_head", 50257, 768, 1),
]


class StepPlan:
    """Stacks of same-shape products executed by one engine launch per step."""

    def __init__(self, stacks, m, device, q, synth, tag):
        import torch
        self.stacks = stacks
        self.m = m
        self.q = q
        self.w = []
        for name, n, k, batch in stacks:
            wf = synth.normal_f32_torch((batch * n, k), 0.02, device, 0, tag, name)
            self.w.append(q.q8_0_quantize_rows(wf))
            del wf
        torch.cuda.synchronize()
        self.k_total = sum(k * batch for _, n, k, batch in stacks)   # activation floats / token
        self.nb_total = self.k_total // QK
        self.xq = torch.empty((m, self.nb_total * BB), dtype=torch.uint8, device=device)
        self.n_out = sum(n * batch for _, n, k, batch in stacks)
        self.y = torch.empty((m, self.n_out), dtype=torch.float32, device=device)
        self.descs = []
        xoff = 0
        yoff = 0
        for (name, n, k, batch), w in zip(stacks, self.w):
            nb = k // QK
            self.descs.append(q.make_desc(
                w, (self.xq, xoff), (self.y, yoff), n, k, m=m, batch=batch,
                w_batch_stride=n * nb, x_row_stride=self.nb_total, x_batch_stride=nb,
                y_row_stride=self.n_out, y_batch_stride=n))
            xoff += batch * nb
            yoff += batch * n
        self.w_bytes = sum(q8_bytes(batch * n, k) for _, n, k, batch in stacks)
        self.x_bytes = m * self.nb_total * BB
        self.y_bytes = m * self.n_out * 4
        self.engine_bytes = self.w_bytes + self.x_bytes + self.y_bytes
        self.quant_bytes = m * self.k_total * 4 + self.x_bytes
        # one fused launch per step: weights + fp32 activations read, outputs written
        self.fused_bytes = self.w_bytes + m * self.k_total * 4 + self.y_bytes
        self.products = m * sum(n * k * batch for _, n, k, batch in stacks)   # MACs
        self._f32_descs = {}

    def descs_f32(self, x_step):
        """Descriptors of the fused launch reading the fp32 rows of x_step."""
        key = x_step.data_ptr()
        if key not in self._f32_descs:
            descs, xoff, yoff = [], 0, 0
            for (name, n, k, batch), w in zip(self.stacks, self.w):
                nb = k // QK
                descs.append(self.q.make_f32_desc(
                    w, (x_step, xoff), (self.y, yoff), n, k, m=self.m, batch=batch,
                    w_batch_stride=n * nb, x_row_stride=self.k_total, x_batch_stride=k,
                    y_row_stride=self.n_out, y_batch_stride=n))
                xoff += batch * k
                yoff += batch * n
            self._f32_descs[key] = descs
        return self._f32_descs[key]

    def step(self, x_step):
        """x_step: fp32 [m][k_total] of this step: a quantize launch, then one
        launch of every product of the step."""
        self.q.q8_0_quantize_rows(x_step, y=self.xq)
        self.q.q8_0_matmul_batched(self.descs, self.y)

    def cold_descs(self, copies):
        """Descriptor sets over `copies` separate copies of the weights (for a
        cold-cache timing: consecutive steps read different copies)."""
        sets = [self.descs]
        self._cold_w = []
        for c in range(1, copies):
            ws = [w.clone() for w in self.w]
            self._cold_w.append(ws)
            descs, xoff, yoff = [], 0, 0
            for (name, n, k, batch), w in zip(self.stacks, ws):
                nb = k // QK
                descs.append(self.q.make_desc(
                    w, (self.xq, xoff), (self.y, yoff), n, k, m=self.m, batch=batch,
                    w_batch_stride=n * nb, x_row_stride=self.nb_total, x_batch_stride=nb,
                    y_row_stride=self.n_out, y_batch_stride=n))
                xoff += batch * nb
                yoff += batch * n
            sets.append(descs)
        return sets

    def step_one(self, x_step):
        """The same step as one launch in which each activation row is quantized
        once (q8_0_matmul_f32_step; m <= 2)."""
        descs = self.descs_f32(x_step)
        if getattr(self, "_step_ws", None) is None:
            self._step_ws = self.q.q8_0_matmul_f32_step_workspace(descs, self.y.device)
        self.q.q8_0_matmul_f32_step(descs, self._step_ws)

    def setup_r8(self):
        """Repack every stack into the row-interleaved (R8) layout (matrix b of
        a stack starts at b * q8_0_r8_bytes(n, k)) and build the descriptors of
        one launch: the matvec engine at m = 1, the small-batch matrix-core
        engine above."""
        q = self.q
        self.w_r8, self.descs_r8 = [], []
        xoff = yoff = 0
        for (name, n, k, batch), w in zip(self.stacks, self.w):
            nb = k // QK
            mb = q.q8_0_r8_bytes(n, k)
            wr = torch_empty_u8(batch * mb, w.device)
            for b in range(batch):
                q.q8_0_repack_r8(w[b * n:(b + 1) * n], n, k, out=wr[b * mb:(b + 1) * mb])
            self.w_r8.append(wr)
            if self.m == 1:
                self.descs_r8.append(q.make_r8_desc(wr, (self.xq, xoff), (self.y, yoff), n, k,
                                                    batch=batch, w_batch_stride=mb,
                                                    x_batch_stride=nb, y_batch_stride=n))
            else:
                self.descs_r8.append(q.make_r8_mm_desc(
                    wr, (self.xq, xoff), (self.y, yoff), n, k, m=self.m, batch=batch,
                    w_batch_stride=mb, x_row_stride=self.nb_total, x_batch_stride=nb,
                    y_row_stride=self.n_out, y_batch_stride=n))
            xoff += batch * nb
            yoff += batch * n

    def r8_engine(self):
        if self.m == 1:
            self.q.q8_0_matvec_r8_batched(self.descs_r8, self.y)
        else:
            self.q.q8_0_matmul_r8_batched(self.descs_r8, self.y)

    def descs_r8_f32(self, x_step):
        key = ("r8", x_step.data_ptr())
        if key not in self._f32_descs:
            descs, xoff, yoff = [], 0, 0
            for (name, n, k, batch), wr in zip(self.stacks, self.w_r8):
                mb = self.q.q8_0_r8_bytes(n, k)
                descs.append(self.q.make_r8_f32_desc(
                    wr, (x_step, xoff), (self.y, yoff), n, k, batch=batch, w_batch_stride=mb,
                    x_batch_stride=k, y_batch_stride=n))
                xoff += batch * k
                yoff += batch * n
            self._f32_descs[key] = descs
        return self._f32_descs[key]

    def cold_r8(self, copies):
        """Descriptor builders over `copies` separate copies of the R8 weights
        (each maps an fp32 step input to the descriptors of one launch)."""
        sets = [self.descs_r8_f32]
        self._cold_w = []
        for c in range(1, copies):
            ws = [w.clone() for w in self.w_r8]
            self._cold_w.append(ws)

            def build(x_step, ws=ws):
                descs, xoff, yoff = [], 0, 0
                for (name, n, k, batch), wr in zip(self.stacks, ws):
                    descs.append(self.q.make_r8_f32_desc(
                        wr, (x_step, xoff), (self.y, yoff), n, k, batch=batch,
                        w_batch_stride=self.q.q8_0_r8_bytes(n, k), x_batch_stride=k,
                        y_batch_stride=n))
                    xoff += batch * k
                    yoff += batch * n
                return descs
            sets.append(build)
        return sets

    def step_r8_one(self, x_step):
        """The step over the R8 weights as one launch: every workgroup
        quantizes the fp32 activation row of its matrix into LDS."""
        self.q.q8_0_matvec_r8_f32_batched(self.descs_r8_f32(x_step), self.y)

    def step_r8(self, x_step):
        """The step over the R8 weights: the quantize launch, then one launch
        of every product."""
        self.q.q8_0_quantize_rows(x_step, y=self.xq)
        self.r8_engine()

    def step_fused(self, x_step):
        """The same step as one launch with the activations quantized inside
        (every wave quantizes the rows it needs; slower here, see the JSON)."""
        self.q.q8_0_matmul_f32_batched(self.descs_f32(x_step), self.y)


def torch_empty_u8(nbytes, device):
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def capture(fn):
    """Capture fn()'s launches (on torch's current stream) in a HIP graph."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # one eager pass on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps=1):
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    g.replay()                    # untimed: first replay after instantiation
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def time_replay(g):
    """Seconds of one replay of graph g, timed with HIP events on the current
    stream (the stream the replayed launches run on)."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3


def protocol(series, rounds=11, best_of=3):
    """The timing protocol: `rounds` rounds, the first dropped; in every round
    each series (name -> captured graph, in the given order) is replayed
    `best_of` times and its best replay kept; the result per series is the
    median of the per-round bests (and their spread).  Series rotate inside a
    round, so slow drift of clocks or temperature reaches all of them alike."""
    import statistics
    per = {k: [] for k in series}
    for g in series.values():          # untimed: first replay after instantiation
        g.replay()
    import torch
    torch.cuda.synchronize()
    for r in range(rounds):
        for k, g in series.items():
            best = min(time_replay(g) for _ in range(best_of))
            if r > 0:
                per[k].append(best)
    return {k: {"median": statistics.median(v), "min": min(v), "max": max(v), "rounds": v}
            for k, v in per.items()}


def control_check(prot, base, control):
    """A control series (the headline graph replayed again inside every round)
    against the headline: the per-round ratios must straddle 1x for the
    headline median to be trusted as a stable figure."""
    ratios = [c / b for b, c in zip(prot[base]["rounds"], prot[control]["rounds"])]
    return {"control_over_headline_min": round(min(ratios), 4),
            "control_over_headline_max": round(max(ratios), 4),
            "straddles_1x": bool(min(ratios) <= 1.0 <= max(ratios))}


def gpu_clocks():
    """Current clocks as rocm-smi reports them (None where it is unavailable);
    the clocks are recorded, not set."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout)
    except Exception:
        return None
    out = {}
    for card, vals in data.items():
        if isinstance(vals, dict):
            out[card] = {k: v for k, v in vals.items() if "clock" in k.lower() or "clk" in k.lower()}
    return out or None


def time_steps(plan, xs, steps, warmup):
    """The K timed steps of each form are captured in one HIP graph and
    replayed once inside the timed region; per-kernel means come from graphs
    of K launches of that kernel alone.  Forms: native layout with 2 launches
    per step (quantize, engine), the same with quantization fused into every
    wave, one launch with each row quantized once (m <= 2); and for m = 1 the
    R8 layout with 2 launches and with 1 launch.  Returns a dict of seconds
    (totals over the K steps, per-launch means)."""
    import torch
    n_in = xs.shape[0]
    one = plan.m <= 2
    r8 = plan.m <= 16
    r8_one = plan.m == 1
    if r8:
        plan.setup_r8()
    for i in range(warmup):
        plan.step(xs[i % n_in])
        plan.step_fused(xs[i % n_in])
        if one:
            plan.step_one(xs[i % n_in])
        if r8:
            plan.step_r8(xs[i % n_in])
        if r8_one:
            plan.step_r8_one(xs[i % n_in])
    torch.cuda.synchronize()

    graphs = {}

    def graph_of(fn, key):
        def body():
            for i in range(steps):
                fn(xs[i % n_in])
        graphs[key] = capture(body)
        return time_graph(graphs[key])

    out = dict(total=graph_of(plan.step, "two"), total_fused=graph_of(plan.step_fused, "fused"),
               total_one=graph_of(plan.step_one, "one") if one else None,
               total_r8=graph_of(plan.step_r8, "r8") if r8 else None,
               total_r8_one=graph_of(plan.step_r8_one, "r8_one") if r8_one else None)
    out["graphs"] = graphs

    def eng_only():
        for _ in range(steps):
            plan.q.q8_0_matmul_batched(plan.descs, plan.y)
    out["eng"] = time_graph(capture(eng_only)) / steps

    def qnt_only():
        for i in range(steps):
            plan.q.q8_0_quantize_rows(xs[i % n_in], y=plan.xq)
    out["qnt"] = time_graph(capture(qnt_only)) / steps
    if r8:
        def eng_r8_only():
            for _ in range(steps):
                plan.r8_engine()
        out["eng_r8"] = time_graph(capture(eng_r8_only)) / steps

    # cold reference: consecutive steps read different copies of the weights,
    # together well over the 256 MB Infinity Cache
    copies = max(2, -(-3 * 256 * 2**20 // plan.w_bytes))
    out["copies"] = copies
    if r8_one:
        sets = plan.cold_r8(copies)

        def all_cold():
            for i in range(steps):
                plan.q.q8_0_matvec_r8_f32_batched(sets[i % copies](xs[i % n_in]), plan.y)
        for i in range(copies):
            plan.q.q8_0_matvec_r8_f32_batched(sets[i](xs[0]), plan.y)
    else:
        sets = plan.cold_descs(copies)

        def all_cold():
            for i in range(steps):
                plan.q.q8_0_quantize_rows(xs[i % n_in], y=plan.xq)
                plan.q.q8_0_matmul_batched(sets[i % copies], plan.y)
        for i in range(copies):
            plan.q.q8_0_matmul_batched(sets[i], plan.y)
    graphs["cold"] = capture(all_cold)
    out["total_cold"] = time_graph(graphs["cold"])
    return out


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload shapes)

def cpu_baseline_steps(stacks, m, sample_steps, threads):
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    ws = []
    for name, n, k, batch in stacks:
        ws.append([oracle.quantize_rows(synth.normal_f32((n, k), 0.02, "cpu", name, b))
                   for b in range(batch)])
    work_bytes = 0
    jobs = []
    for s in range(sample_steps):
        for (name, n, k, batch), wl in zip(stacks, ws):
            for b in range(batch):
                xq = oracle.quantize_rows(synth.normal_f32((m, k), 1.0, "cpu-x", name, b, s))
                jobs.append((wl[b], xq, n, k))
                work_bytes += q8_bytes(n, k) + xq.nbytes + m * n * 4

    def run(part):
        w, xq, n, k, lo, hi = part
        oracle.matmul(w, xq, n, k, m, lo, hi)

    # the products are independent: they go to the threads whole, the large
    # ones in slices of 4096 rows (thin row slices of small products cost more
    # in per-call overhead than they save)
    parts = [(w, xq, n, k, lo, min(n, lo + 4096)) for w, xq, n, k in jobs
             for lo in range(0, n, 4096)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, parts))
    dt = time.perf_counter() - t0
    return work_bytes / dt / 1e9, dt, work_bytes


# ---------------------------------------------------------------------------

def bench_decode(args, q, synth, stacks, m, name, wl_desc, n_steps_cfg):
    import torch
    dev = "cuda"
    plan = StepPlan(stacks, m, dev, q, synth, name)
    n_in = min(args.steps + args.warmup, n_steps_cfg)
    xs = synth.normal_f32_torch((n_in, m, plan.k_total), 1.0, dev, 0, name, "x")
    torch.cuda.synchronize()
    clocks_before = gpu_clocks()
    t = time_steps(plan, xs, args.steps, args.warmup)
    K = args.steps
    two_bytes = plan.engine_bytes + plan.quant_bytes      # quantize launch + engine launch
    # the protocol over the headline form: warm, cold (rotating weight
    # copies), and the headline again as the control series
    head = "r8_one" if m == 1 else "two"
    prot = protocol({"headline": t["graphs"][head], "cold": t["graphs"]["cold"],
                     "control": t["graphs"][head]})
    if m == 1:
        # headline: R8 weights, one launch per step (weights + fp32 rows read,
        # outputs written)
        total, step_bytes, launch_bytes = prot["headline"]["median"], plan.fused_bytes, plan.fused_bytes
        launch_s = total / K
        kernel = ("r8_matvec_kernel<true> (one launch per step over the R8 weights; every "
                  "workgroup quantizes the fp32 activation row of its matrix)")
        launches = 1
        headline_series = "warm"
    else:
        # the step's 131 MB of weights fit the 256 MB Infinity Cache: the
        # cold series (rotating weight copies) is the headline
        total, step_bytes, launch_bytes = prot["cold"]["median"], two_bytes, plan.engine_bytes
        launch_s = t["eng"]
        kernel = ("stream_flat_kernel (decode engine)" if m == 2 else
                  "stream_mfma_kernel (small-batch decode engine)")
        launches = 2
        headline_series = "cold"
    value = step_bytes * K / total / 1e9
    achieved = launch_bytes / launch_s / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot, fp32 scale (Q8_0)",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; random init, no checkpoint)",
        "config": {"workload": wl_desc.format(K=K), "batch": m, "products_per_step": sum(
            b for _, _, _, b in stacks), "launches_per_step": launches,
            "timing": ("HIP graph of the K sequential steps; 11 rounds, the first dropped, each "
                       "round the best of 3 replays (HIP events) of the headline, cold and "
                       "control series in turn; value = median of the rounds' bests "
                       f"({headline_series} series)"),
            "weight_bytes_per_step": plan.w_bytes, "algorithmic_bytes_per_step": step_bytes},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(m * K / total, 1),
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(launch_s * 1e6, 3),
                     "bytes_per_launch": launch_bytes},
    }
    if m == 1:
        out["config"]["weights"] = ("Q8_0, repacked once at load (outside the timed region) into "
                                    "the row-interleaved R8 layout: the same bytes, moved")
    out["protocol"] = {
        "rounds": 11, "dropped": 1, "best_of": 3,
        "headline_ms_per_step": {kk: round(prot["headline"][kk] / K * 1e3, 5)
                                 for kk in ("median", "min", "max")},
        "cold_ms_per_step": {kk: round(prot["cold"][kk] / K * 1e3, 5)
                             for kk in ("median", "min", "max")},
        "control": control_check(prot, "headline", "control"),
        "gpu_clocks_before": clocks_before, "gpu_clocks_after": gpu_clocks()}
    # context: a plain streaming read of the same number of bytes per launch
    # (q8_read_probe; non-temporal 16-byte loads, no arithmetic)
    probe_bytes = (launch_bytes + 65535) // 65536 * 65536
    src = torch.ones(probe_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    tp = _time_launches(lambda: q.q8_read_probe(src, sink), K, 5) / K
    del src
    out["roofline"]["read_probe_same_bytes"] = {
        "bytes": probe_bytes, "us": round(tp * 1e6, 3), "gbs": round(probe_bytes / tp / 1e9, 1),
        "kernel_over_probe": round(tp / launch_s, 4)}
    out["cold_reference"] = {
        "timing": f"the same steps reading {t['copies']} rotating copies of the weights "
                  f"({t['copies'] * plan.w_bytes / 2**20:.0f} MiB, > the 256 MB Infinity Cache); "
                  "median of the protocol's cold series",
        "ms_per_step": round(prot["cold"]["median"] / K * 1e3, 5),
        "gbs": round(step_bytes * K / prot["cold"]["median"] / 1e9, 1),
        "pct_of_hbm_peak": round(step_bytes * K / prot["cold"]["median"] / 1e9 / HBM_PEAK_GBS * 100, 2)}
    if m > 1:
        out["warm_reference"] = {
            "timing": "the same steps over one weight copy (cache-resident); median of the "
                      "protocol's headline series",
            "ms_per_step": round(prot["headline"]["median"] / K * 1e3, 5),
            "gbs": round(step_bytes * K / prot["headline"]["median"] / 1e9, 1)}
    plan._cold_w = []
    if m == 1:
        out["r8_two_launch_reference"] = {
            "timing": "R8 weights: quantize launch + one q8_0_matvec_r8_batched launch per step",
            "ms_per_step": round(t["total_r8"] / K * 1e3, 5),
            "gbs": round(two_bytes * K / t["total_r8"] / 1e9, 1),
            "engine_avg_launch_us": round(t["eng_r8"] * 1e6, 3),
            "engine_gbs": round(plan.engine_bytes / t["eng_r8"] / 1e9, 1)}
        out["native_layout_reference"] = {
            "timing": "native Q8_0 rows: quantize launch + one q8_0_matmul_batched launch per "
                      "step (stream_pair_kernel)",
            "ms_per_step": round(t["total"] / K * 1e3, 5),
            "gbs": round(two_bytes * K / t["total"] / 1e9, 1),
            "engine_avg_launch_us": round(t["eng"] * 1e6, 3),
            "engine_gbs": round(plan.engine_bytes / t["eng"] / 1e9, 1),
            "engine_frac": round(plan.engine_bytes / t["eng"] / 1e9 / HBM_PEAK_GBS, 4),
            "quantize_kernel_avg_us": round(t["qnt"] * 1e6, 3)}
        nt = os.path.join(ROOT, "profiles", "stream_pair_kernel_llama110m_decode_step.traffic.json")
        if os.path.exists(nt):
            out["native_layout_reference"]["engine_traffic"] = read_traffic(nt)
    else:
        out["quantize_kernel_avg_us"] = round(t["qnt"] * 1e6, 3)
        if t["total_r8"] is not None:
            out["r8_layout_reference"] = {
                "timing": "R8 weights: quantize launch + one q8_0_matmul_r8_batched launch per "
                          "step (r8_mm_kernel, int8 matrix cores)",
                "ms_per_step": round(t["total_r8"] / K * 1e3, 5),
                "gbs": round(two_bytes * K / t["total_r8"] / 1e9, 1),
                "engine_avg_launch_us": round(t["eng_r8"] * 1e6, 3),
                "engine_gbs": round(plan.engine_bytes / t["eng_r8"] / 1e9, 1)}
    out["fused_reference"] = {
        "timing": "native rows, one launch per step, every wave quantizing the rows it reads",
        "ms_per_step": round(t["total_fused"] / K * 1e3, 5),
        "gbs": round(plan.fused_bytes * K / t["total_fused"] / 1e9, 1)}
    if t["total_one"] is not None:
        out["one_launch_reference"] = {
            "timing": "native rows, one launch per step, every activation row quantized once "
                      "inside it by the launch's first workgroups",
            "ms_per_step": round(t["total_one"] / K * 1e3, 5),
            "gbs": round(plan.fused_bytes * K / t["total_one"] / 1e9, 1)}
    return out, plan


# ---------------------------------------------------------------------------
# the other configurations (one JSON line each; not the headline)

def _time_launches(fn, steps, warmup):
    """Seconds for `steps` calls of fn, captured in one HIP graph and replayed
    once (after `warmup` eager calls and one untimed replay)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()

    def many():
        for _ in range(steps):
            fn()
    return time_graph(capture(many))


def run_extra(args, q, synth):
    import torch
    dev = "cuda"
    wl = args.workload
    res = {"workload": wl, "steps": args.steps, "warmup": args.warmup}
    if wl == "readbw":
        # achievable read bandwidth for context: the library's plain streaming
        # read (q8_read_probe) over 2 GiB, or --read-bytes (e.g. the 116.9 MB of
        # the Llama-110M-shaped step, to see the ramp and tail of a launch that
        # size)
        nbytes = args.read_bytes if args.read_bytes else 2 << 30
        nbytes = (nbytes + 65535) // 65536 * 65536
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4096, dtype=torch.int32, device=dev)
        total = _time_launches(lambda: q.q8_read_probe(src, sink), max(10, args.steps // 10), 3)
        t = total / max(10, args.steps // 10)
        res.update(bytes_read_per_launch=nbytes, us_per_read=round(t * 1e6, 2),
                   gbs=round(nbytes / t / 1e9, 1),
                   pct_of_hbm_peak=round(nbytes / t / 1e9 / HBM_PEAK_GBS * 100, 2))
    elif wl == "copy":
        # calibration for hardware byte counters: a plain device-to-device copy of
        # a known size (256 MiB read + 256 MiB written per launch)
        nbytes = 256 << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        total = _time_launches(lambda: dst.copy_(src), args.steps, args.warmup)
        t = total / args.steps
        res.update(bytes_read_per_launch=nbytes, bytes_written_per_launch=nbytes,
                   us_per_copy=round(t * 1e6, 2), gbs=round(2 * nbytes / t / 1e9, 1))
    elif wl in ("c1", "c5b"):
        n, k = (768, 768) if wl == "c1" else (262144, 2048)
        wf = synth.normal_f32_torch((n, k), 0.02, dev, 0, wl, "w")
        w = q.q8_0_quantize_rows(wf)
        del wf
        xf = synth.normal_f32_torch((1, k), 1.0, dev, 0, wl, "x")
        x = q.q8_0_quantize_rows(xf)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        total = _time_launches(lambda: q.q8_0_matvec(w, x, n, k, y=y), args.steps, args.warmup)
        nbytes = q8_bytes(n, k) + q8_bytes(1, k) + 4 * n
        t = total / args.steps
        res.update(shape=[n, k], us_per_matvec=round(t * 1e6, 3),
                   gbs=round(nbytes / t / 1e9, 1), pct_of_hbm_peak=round(nbytes / t / 1e9 / HBM_PEAK_GBS * 100, 2),
                   tokens_per_s_equiv=round(1 / t, 1), bytes_per_launch=nbytes)
        # from fp32 activations: quantize launch + matvec, or one fused launch
        t2 = _time_launches(lambda: (q.q8_0_quantize_rows(xf, y=x), q.q8_0_matvec(w, x, n, k, y=y)),
                            args.steps, args.warmup) / args.steps
        fd = [q.make_f32_desc(w, xf, y, n, k)]
        tf = _time_launches(lambda: q.q8_0_matmul_f32_batched(fd, w), args.steps,
                            args.warmup) / args.steps
        sws = q.q8_0_matmul_f32_step_workspace(fd, dev)
        ts = _time_launches(lambda: q.q8_0_matmul_f32_step(fd, sws), args.steps,
                            args.warmup) / args.steps
        res.update(from_fp32={"us_quantize_then_matvec": round(t2 * 1e6, 3),
                              "us_fused": round(tf * 1e6, 3),
                              "us_one_launch_quantize_once": round(ts * 1e6, 3)})
    elif wl == "ffn":
        # dense FFN up_gate + SwiGLU of the Llama-2-110M layers (n_embd 768,
        # n_ff 2048, 12 layers in one launch, batch 1): fused launch against the
        # two-product form (one batched product over both halves + elementwise)
        L, n_ff, k = 12, 2048, 768
        nb = k // QK
        w = q.q8_0_quantize_rows(synth.normal_f32_torch((L * 2 * n_ff, k), 0.02, dev, 0, wl, "w"))
        x = q.q8_0_quantize_rows(synth.normal_f32_torch((1, L * k), 1.0, dev, 0, wl, "x"))
        h = torch.empty((1, L * n_ff), dtype=torch.float32, device=dev)
        d = [q.make_up_gate_desc(w, x, h, n_ff, k, batch=L, w_batch_stride=2 * n_ff * nb,
                                 x_batch_stride=nb, h_batch_stride=n_ff)]
        total = _time_launches(lambda: q.q8_0_up_gate_swiglu_batched(d, w), args.steps, args.warmup)
        t = total / args.steps
        nbytes = q8_bytes(L * 2 * n_ff, k) + q8_bytes(L, k) + 4 * L * n_ff
        y = torch.empty((1, L * 2 * n_ff), dtype=torch.float32, device=dev)
        d2 = [q.make_desc(w, x, y, 2 * n_ff, k, batch=L, w_batch_stride=2 * n_ff * nb,
                          x_batch_stride=nb, y_batch_stride=2 * n_ff)]
        yv = y.view(L, 2, n_ff)
        hv = h.view(L, n_ff)

        def two_product():
            q.q8_0_matmul_batched(d2, w)
            torch.mul(torch.nn.functional.silu(yv[:, 0]), yv[:, 1], out=hv)
        t2 = _time_launches(two_product, args.steps, args.warmup) / args.steps
        res.update(shape={"layers": L, "n_ff": n_ff, "n_embd": k, "batch": 1},
                   us_per_launch=round(t * 1e6, 3), gbs=round(nbytes / t / 1e9, 1),
                   pct_of_hbm_peak=round(nbytes / t / 1e9 / HBM_PEAK_GBS * 100, 2),
                   bytes_per_launch=nbytes,
                   two_product_reference={"us": round(t2 * 1e6, 3),
                                          "timing": "q8_0_matmul_batched over both halves, "
                                                    "then torch silu and multiply"})
        if not args.no_cpu_baseline:
            # the oracle's dense up_gate on the same 12 layers (seeded numpy
            # inputs of the same shapes), one host thread
            import oracle
            wl_h = [oracle.quantize_rows(synth.normal_f32((2 * n_ff, k), 0.02, "cpu-ffn", i))
                    for i in range(L)]
            xs_h = [oracle.quantize_rows(synth.normal_f32((1, k), 1.0, "cpu-ffn-x", i))
                    for i in range(L)]
            t0 = time.perf_counter()
            for wi, xi in zip(wl_h, xs_h):
                oracle.up_gate_swiglu(wi, xi, k, n_ff)
            dt = time.perf_counter() - t0
            res["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                   "kind": "oracle", "sample": f"the 12 layers once, {dt:.2f} s"}
    elif wl == "r8":
        # the row-interleaved weight layout (repacked once, outside the timed
        # region) against native rows: one matvec per launch, the vocabulary
        # projection and the Llama-110M matrix shapes
        shapes = [(262144, 2048), (32000, 768), (2048, 768), (768, 2048), (768, 768)]
        rows_out = []
        for n, k in shapes:
            w = q.q8_0_quantize_rows(synth.normal_f32_torch((n, k), 0.02, dev, 0, wl, "w", n, k))
            x = q.q8_0_quantize_rows(synth.normal_f32_torch((1, k), 1.0, dev, 0, wl, "x", n, k))
            y = torch.empty(n, dtype=torch.float32, device=dev)
            t_rp = _time_launches(lambda: q.q8_0_repack_r8(w, n, k), 3, 1) / 3
            wr = q.q8_0_repack_r8(w, n, k)
            tn = _time_launches(lambda: q.q8_0_matvec(w, x, n, k, y=y), args.steps,
                                args.warmup) / args.steps
            tr = _time_launches(lambda: q.q8_0_matvec_r8(wr, x, n, k, y=y), args.steps,
                                args.warmup) / args.steps
            nbytes = q8_bytes(n, k) + q8_bytes(1, k) + 4 * n
            rows_out.append({"shape": [n, k], "bytes_per_launch": nbytes,
                             "native_us": round(tn * 1e6, 3), "r8_us": round(tr * 1e6, 3),
                             "native_gbs": round(nbytes / tn / 1e9, 1),
                             "r8_gbs": round(nbytes / tr / 1e9, 1),
                             "r8_over_native_time": round(tr / tn, 4),
                             "repack_us_once": round(t_rp * 1e6, 1)})
            del w, wr
        big = rows_out[0]
        res.update(shapes=rows_out, us_per_matvec=big["r8_us"], gbs=big["r8_gbs"],
                   pct_of_hbm_peak=round(big["r8_gbs"] / HBM_PEAK_GBS * 100, 2),
                   roofline={"bound": "hbm", "achieved": big["r8_gbs"], "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(big["r8_gbs"] / HBM_PEAK_GBS, 4),
                             "traffic": None, "kernel": "r8_matvec_kernel"})
        if not args.no_cpu_baseline:
            # the oracle's R8 matvec on 4096 rows of the vocabulary shape
            import oracle
            n, k = 4096, 2048
            wh = oracle.quantize_rows(synth.normal_f32((n, k), 0.02, "cpu-r8", n))
            xh = oracle.quantize_rows(synth.normal_f32((1, k), 1.0, "cpu-r8-x", n))
            wrh = oracle.repack_r8(wh, n, k)
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < 5.0:
                oracle.matvec_r8(wrh, xh, n, k)
                reps += 1
            dt = time.perf_counter() - t0
            nb_cpu = q8_bytes(n, k) + q8_bytes(1, k) + 4 * n
            res["cpu_baseline"] = {"value": round(reps * nb_cpu / dt / 1e9, 3), "unit": "GB/s",
                                   "cores": 1, "kind": "oracle",
                                   "sample": f"{reps} R8 matvecs of 4096 x 2048, {dt:.1f} s"}
    elif wl == "kq":
        # 4/5-bit K-quant weights (Q4_K, Q5_K) against Q8_1 activations: the
        # vocabulary projection and the Llama-110M-shaped step (85 products:
        # one Q8_1 quantize launch + one kq_matvec_batched launch)
        out_t = {}
        for t in (4, 5):
            bb = synth.KQ_BYTES[t]
            n, k = 262144, 2048
            w = synth.kq_blocks_torch(t, n, k, dev, 0, wl, t)
            xf = synth.normal_f32_torch((1, k), 1.0, dev, 0, wl, "x", t)
            x = q.q8_1_quantize_rows(xf)
            y = torch.empty(n, dtype=torch.float32, device=dev)
            tv = _time_launches(lambda: q.kq_matvec(t, w, x, n, k, y=y), args.steps,
                                args.warmup) / args.steps
            vb = n * (k // 256) * bb + (k // 32) * 36 + 4 * n
            del w
            # the step: stacks as in the default workload
            ws, descs = [], []
            k_tot = sum(kk * b for _, nn, kk, b in LLAMA_STACKS)
            n_tot = sum(nn * b for _, nn, kk, b in LLAMA_STACKS)
            xs = synth.normal_f32_torch((1, k_tot), 1.0, dev, 0, wl, "step-x", t)
            xq = torch.empty(k_tot // 32 * 36, dtype=torch.uint8, device=dev)
            ys = torch.empty(n_tot, dtype=torch.float32, device=dev)
            xoff = yoff = 0
            wbytes = 0
            for name, nn, kk, b in LLAMA_STACKS:
                wt = synth.kq_blocks_torch(t, b * nn, kk, dev, 0, wl, name, t)
                ws.append(wt)
                wbytes += wt.numel()
                descs.append(q.make_kq_desc(wt, (xq, xoff * 36), (ys, yoff), nn, kk, batch=b,
                                            w_batch_stride=nn * (kk // 256),
                                            x_batch_stride=kk // 32, y_batch_stride=nn))
                xoff += b * kk // 32
                yoff += b * nn

            def kstep():
                q.q8_1_quantize_rows(xs, y=xq.view(1, -1))
                q.kq_matvec_batched(t, descs, xq)
            ts = _time_launches(kstep, args.steps, args.warmup) / args.steps
            te = _time_launches(lambda: q.kq_matvec_batched(t, descs, xq), args.steps,
                                args.warmup) / args.steps
            sb = wbytes + xq.numel() + 4 * n_tot
            out_t["q4_k" if t == 4 else "q5_k"] = {
                "bits_per_weight": bb * 8 / 256,
                "vocab_262144x2048": {"us": round(tv * 1e6, 3), "bytes_per_launch": vb,
                                      "gbs": round(vb / tv / 1e9, 1),
                                      "frac": round(vb / tv / 1e9 / HBM_PEAK_GBS, 4)},
                "llama110m_step": {"us_per_step": round(ts * 1e6, 3),
                                   "tokens_per_s": round(1 / ts, 1),
                                   "engine_us": round(te * 1e6, 3), "engine_bytes": sb,
                                   "engine_gbs": round(sb / te / 1e9, 1),
                                   "engine_frac": round(sb / te / 1e9 / HBM_PEAK_GBS, 4)}}
            del ws
        res.update(formats=out_t)
        v4 = out_t["q4_k"]["vocab_262144x2048"]
        tf = os.path.join(ROOT, "profiles", "kq_matvec_kernel_q4k_vocab.traffic.json")
        res.update(roofline={"bound": "hbm", "kernel": "kq_matvec_kernel<4> (Q4_K, vocabulary "
                             "projection 262144 x 2048)", "achieved": v4["gbs"],
                             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": v4["frac"],
                             "avg_launch_us": v4["us"], "bytes_per_launch": v4["bytes_per_launch"],
                             "traffic": read_traffic(tf) if os.path.exists(tf) else None})
        if not args.no_cpu_baseline:
            import oracle
            n, k = 2048, 2048
            wh = synth.kq_blocks(4, n, k, "cpu-kq")
            xh = oracle.quantize_rows_q8_1(synth.normal_f32((1, k), 1.0, "cpu-kq-x"))
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < 5.0:
                oracle.kq_matvec(4, wh, xh, n, k)
                reps += 1
            dt = time.perf_counter() - t0
            nb_cpu = wh.nbytes + xh.nbytes + 4 * n
            res["cpu_baseline"] = {"value": round(reps * nb_cpu / dt / 1e9, 3), "unit": "GB/s",
                                   "cores": 1, "kind": "oracle",
                                   "sample": f"{reps} Q4_K matvecs of 2048 x 2048, {dt:.1f} s"}
    elif wl == "c5a":
        m, n, k = 512, 14336, 4096
        w = q.q8_0_quantize_rows(synth.normal_f32_torch((n, k), 0.02, dev, 0, wl, "w"))
        x = q.q8_0_quantize_rows(synth.normal_f32_torch((m, k), 1.0, dev, 0, wl, "x"))
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        total = _time_launches(lambda: q.q8_0_matmul(w, x, n, k, m, y=y), args.steps,
                               args.warmup)
        t = total / args.steps
        ops = 2.0 * m * n * k
        res.update(shape=[m, n, k], us_per_gemm=round(t * 1e6, 2),
                   tops=round(ops / t / 1e12, 2), pct_of_int8_peak=round(ops / t / 5.0e15 * 100, 2),
                   prompt_tokens_per_s=round(m / t, 1))
    elif wl in ("c4b1", "c4b16"):
        n_tok = 1 if wl == "c4b1" else 16
        L, E, n_embd, n_ff, U = 30, 128, 2048, 768, 8
        layers = []
        active_bytes = 0
        for l in range(L):
            wug = q.q8_0_quantize_rows(synth.normal_f32_torch((E * 2 * n_ff, n_embd), 0.02, dev,
                                                              0, wl, "ug", l))
            wd = q.q8_0_quantize_rows(synth.normal_f32_torch((E * n_embd, n_ff), 0.02, dev, 0,
                                                             wl, "down", l))
            ids = synth.expert_ids(n_tok, U, E, 0, wl, "ids", l)
            cw = synth.combine_weights(n_tok, U, 0, wl, "cw", l)
            xf = synth.normal_f32_torch((n_tok, n_embd), 1.0, dev, 0, wl, "x", l)
            n_act = len(np.unique(ids))
            active_bytes += n_act * (q8_bytes(2 * n_ff, n_embd) + q8_bytes(n_embd, n_ff))
            layers.append(dict(wug=wug, wd=wd, ids=torch.from_numpy(ids).to(dev),
                               cw=torch.from_numpy(cw).to(dev), xf=xf,
                               h=torch.empty((n_tok, U, n_ff), dtype=torch.float32, device=dev),
                               out=torch.empty((n_tok, n_embd), dtype=torch.float32, device=dev),
                               ws=q.moe_workspace(n_tok, n_embd, n_ff, E, U, dev)))
        torch.cuda.synchronize()

        def step():
            for d in layers:
                q.moe_up_gate_swiglu(d["wug"], d["xf"], d["ids"], n_embd, n_ff, E, d["ws"],
                                     h=d["h"])
                q.moe_down_combine(d["wd"], d["h"], d["ids"], d["cw"], n_ff, n_embd, E, d["ws"],
                                   out=d["out"])
        # the same work with the layers grouped: one up_gate and one down
        # launch per step (the layers' inputs are independent synthetic rows)
        ug = [dict(w_up_gate=d["wug"], x=d["xf"], ids=d["ids"], h=d["h"], ws=d["ws"])
              for d in layers]
        dn = [dict(w_down=d["wd"], h=d["h"], ids=d["ids"], cw=d["cw"], out=d["out"], ws=d["ws"])
              for d in layers]

        def step_grouped():
            q.moe_up_gate_swiglu_batched(ug, n_embd, n_ff, E)
            q.moe_down_combine_batched(dn, n_ff, n_embd, E)
        res.update(tokens=n_tok, layers=L, active_weight_bytes=active_bytes)
        # the same layers over expert weights repacked once into the R8 layout:
        # one moe_r8_ffn_batched call per step (2 launches at one token; 3 at
        # several: up_gate, down, combine)
        r8l = []
        for d in layers:
            r8l.append(dict(w_up_gate_r8=q.q8_0_repack_r8(d["wug"], E * 2 * n_ff, n_embd),
                            w_down_r8=q.q8_0_repack_r8(d["wd"], E * n_embd, n_ff), x=d["xf"],
                            ids=d["ids"], cw=d["cw"], h=d["h"], out=d["out"],
                            ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, E, U, dev)))
        tr = _time_launches(lambda: q.moe_r8_ffn_batched(r8l, n_embd, n_ff, E), args.steps,
                            args.warmup) / args.steps
        res.update(r8_layout={"timing": "expert weights repacked once into the R8 layout; "
                                        "all layers in one moe_r8_ffn_batched call (2 launches at "
                                        "one token; 3 at several: up_gate, down, combine)",
                              "us_per_step": round(tr * 1e6, 2),
                              "gbs": round(active_bytes / tr / 1e9, 1),
                              "pct_of_hbm_peak": round(active_bytes / tr / 1e9 / HBM_PEAK_GBS * 100, 2),
                              "tokens_per_s": round(n_tok / tr, 1)})
        if n_tok == 1:
            # layer after layer over the R8 weights: two launches per layer
            # (moe_r8_ffn_batched per layer) and one (moe_r8_ffn_fused)
            fz = [dict(d, ws=q.moe_r8_fused_workspace(n_embd, n_ff, E, U, dev)) for d in r8l]

            def chained_two():
                for d in r8l:
                    q.moe_r8_ffn_batched([d], n_embd, n_ff, E)

            def chained_one():
                for d in fz:
                    q.moe_r8_ffn_fused(d, n_embd, n_ff, E)
            for key, fn, desc in (("r8_layer_after_layer", chained_two,
                                   "moe_r8_ffn_batched per layer (2 launches per layer)"),
                                  ("r8_fused_layer_after_layer", chained_one,
                                   "moe_r8_ffn_fused per layer (1 launch per layer)")):
                tl = _time_launches(fn, args.steps, args.warmup) / args.steps
                res[key] = {"timing": desc, "us_per_step": round(tl * 1e6, 2),
                            "gbs": round(active_bytes / tl / 1e9, 1),
                            "pct_of_hbm_peak": round(active_bytes / tl / 1e9 / HBM_PEAK_GBS * 100, 2),
                            "tokens_per_s": round(n_tok / tl, 1)}
            del fz
        del r8l
        if args.moe_mode in ("both", "layers"):
            t = _time_launches(step, args.steps, args.warmup) / args.steps
            res.update(us_per_step=round(t * 1e6, 2), gbs=round(active_bytes / t / 1e9, 1),
                       pct_of_hbm_peak=round(active_bytes / t / 1e9 / HBM_PEAK_GBS * 100, 2),
                       tokens_per_s=round(n_tok / t, 1),
                       timing="two launches per layer, layer after layer")
        if args.moe_mode in ("both", "grouped"):
            tg = _time_launches(step_grouped, args.steps, args.warmup) / args.steps
            res.update(grouped={"timing": "all layers in one up_gate and one down launch",
                                "us_per_step": round(tg * 1e6, 2),
                                "gbs": round(active_bytes / tg / 1e9, 1),
                                "pct_of_hbm_peak": round(active_bytes / tg / 1e9 / HBM_PEAK_GBS * 100, 2),
                                "tokens_per_s": round(n_tok / tg, 1)})
    elif wl == "c4p":
        # prompt evaluation through the same expert FFN: 512 tokens of one layer
        # (grouped int8 matrix-core GEMMs: routing, quantization, up_gate+SwiGLU,
        # quantization of h, down, combine)
        n_tok, E, n_embd, n_ff, U = 512, 128, 2048, 768, 8
        wug = q.q8_0_quantize_rows(synth.normal_f32_torch((E * 2 * n_ff, n_embd), 0.02, dev, 0,
                                                          wl, "ug"))
        wd = q.q8_0_quantize_rows(synth.normal_f32_torch((E * n_embd, n_ff), 0.02, dev, 0, wl,
                                                         "down"))
        ids_h = synth.expert_ids(n_tok, U, E, 0, wl, "ids")
        ids = torch.from_numpy(ids_h).to(dev)
        cw = torch.from_numpy(synth.combine_weights(n_tok, U, 0, wl, "cw")).to(dev)
        xf = synth.normal_f32_torch((n_tok, n_embd), 1.0, dev, 0, wl, "x")
        h = torch.empty((n_tok, U, n_ff), dtype=torch.float32, device=dev)
        out = torch.empty((n_tok, n_embd), dtype=torch.float32, device=dev)
        ws = q.moe_workspace(n_tok, n_embd, n_ff, E, U, dev)
        n_act = len(np.unique(ids_h))
        active_bytes = n_act * (q8_bytes(2 * n_ff, n_embd) + q8_bytes(n_embd, n_ff))
        macs = n_tok * U * (n_embd * 2 * n_ff + n_ff * n_embd)

        def up():
            q.moe_up_gate_swiglu(wug, xf, ids, n_embd, n_ff, E, ws, h=h)

        def down():
            q.moe_down_combine(wd, h, ids, cw, n_ff, n_embd, E, ws, out=out)
        t_up = _time_launches(up, args.steps, args.warmup) / args.steps
        t_dn = _time_launches(down, args.steps, args.warmup) / args.steps
        t = _time_launches(lambda: (up(), down()), args.steps, args.warmup) / args.steps
        res.update(tokens=n_tok, shape={"n_embd": n_embd, "n_ff": n_ff, "n_expert": E, "n_used": U},
                   active_experts=n_act, active_weight_bytes=active_bytes,
                   us_per_layer=round(t * 1e6, 2), prompt_tokens_per_s=round(n_tok / t, 1),
                   gbs=round(active_bytes / t / 1e9, 1),
                   pct_of_hbm_peak=round(active_bytes / t / 1e9 / HBM_PEAK_GBS * 100, 2),
                   tops=round(2 * macs / t / 1e12, 2),
                   us_up_gate_call=round(t_up * 1e6, 2), us_down_call=round(t_dn * 1e6, 2))
        # the same layer over expert weights repacked once into the R8 layout
        # (one moe_r8_ffn_batched call: routing, quantization, both grouped
        # products and the combine)
        r8 = dict(w_up_gate_r8=q.q8_0_repack_r8(wug, E * 2 * n_ff, n_embd),
                  w_down_r8=q.q8_0_repack_r8(wd, E * n_embd, n_ff), x=xf, ids=ids, cw=cw,
                  h=torch.empty_like(h), out=torch.empty_like(out),
                  ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, E, U, dev))
        t8 = _time_launches(lambda: q.moe_r8_ffn_batched([r8], n_embd, n_ff, E), args.steps,
                            args.warmup) / args.steps
        res["r8_layout"] = dict(us_per_layer=round(t8 * 1e6, 2),
                                prompt_tokens_per_s=round(n_tok / t8, 1),
                                gbs=round(active_bytes / t8 / 1e9, 1),
                                pct_of_hbm_peak=round(active_bytes / t8 / 1e9 / HBM_PEAK_GBS * 100, 2),
                                tops=round(2 * macs / t8 / 1e12, 2),
                                bitwise_equal_to_native=bool(torch.equal(r8["out"], out)
                                                             and torch.equal(r8["h"], h)))
    return res


def default_extras(args, q, synth):
    """Keys of the default line beyond the decode step, timed in the same run
    with the same protocol (fewer rounds): the vocabulary projection and the
    30-layer MoE expert FFN at 1 and 16 tokens, layer after layer (as a model
    runs it) and grouped."""
    import torch
    dev = "cuda"
    out = {}
    # --- the vocabulary projection 262144 x 2048 (571 MB > the Infinity Cache)
    n, k = 262144, 2048
    w = q.q8_0_quantize_rows(synth.normal_f32_torch((n, k), 0.02, dev, 0, "c5b", "w"))
    x = q.q8_0_quantize_rows(synth.normal_f32_torch((1, k), 1.0, dev, 0, "c5b", "x"))
    wr = q.q8_0_repack_r8(w, n, k)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    nbytes = q8_bytes(n, k) + q8_bytes(1, k) + 4 * n
    reps = 20

    def many_n(fn, count):
        def body():
            for _ in range(count):
                fn()
        fn()
        torch.cuda.synchronize()
        return capture(body)

    def many(fn):
        return many_n(fn, reps)
    prot = protocol({"native": many(lambda: q.q8_0_matvec(w, x, n, k, y=y)),
                     "r8": many(lambda: q.q8_0_matvec_r8(wr, x, n, k, y=y))}, rounds=6, best_of=3)
    c5b = {"shape": [n, k], "bytes_per_launch": nbytes,
           "timing": f"{reps} launches per graph; 6 rounds (first dropped), best of 3, median"}
    for key, kern in (("native", "stream_pair_kernel"), ("r8", "r8_matvec_kernel<false>")):
        tt = prot[key]["median"] / reps
        c5b[key] = {"kernel": kern, "us": round(tt * 1e6, 3), "gbs": round(nbytes / tt / 1e9, 1),
                    "frac": round(nbytes / tt / 1e9 / HBM_PEAK_GBS, 4),
                    "tokens_per_s_equiv": round(1 / tt, 1)}
    out["c5b_vocab_projection"] = c5b
    del w, x, wr, y
    # --- the MoE expert FFN: 30 layers of (n_embd 2048, n_ff 768, 128 experts, top-8)
    L, E, n_embd, n_ff, U = 30, 128, 2048, 768, 8
    wl = []
    for l in range(L):
        wug = q.q8_0_quantize_rows(synth.normal_f32_torch((E * 2 * n_ff, n_embd), 0.02, dev, 0,
                                                          "c4", "ug", l))
        wd = q.q8_0_quantize_rows(synth.normal_f32_torch((E * n_embd, n_ff), 0.02, dev, 0, "c4",
                                                         "down", l))
        wl.append(dict(wug=wug, wd=wd, wug_r8=q.q8_0_repack_r8(wug, E * 2 * n_ff, n_embd),
                       wd_r8=q.q8_0_repack_r8(wd, E * n_embd, n_ff)))
    torch.cuda.synchronize()
    steps = 10
    c4 = {"layers": L, "shape": {"n_embd": n_embd, "n_ff": n_ff, "n_expert": E, "n_used": U},
          "timing": f"HIP graph of {steps} steps of all 30 layers; 6 rounds (first dropped), "
                    "best of 3, median"}
    for n_tok in (1, 16):
        layers, active = [], 0
        for l in range(L):
            ids = synth.expert_ids(n_tok, U, E, 0, "c4", n_tok, "ids", l)
            active += len(np.unique(ids)) * (q8_bytes(2 * n_ff, n_embd) + q8_bytes(n_embd, n_ff))
            d = dict(wl[l], ids=torch.from_numpy(ids).to(dev),
                     cw=torch.from_numpy(synth.combine_weights(n_tok, U, 0, "c4", n_tok, "cw", l)).to(dev),
                     xf=synth.normal_f32_torch((n_tok, n_embd), 1.0, dev, 0, "c4", n_tok, "x", l),
                     h=torch.empty((n_tok, U, n_ff), dtype=torch.float32, device=dev),
                     out=torch.empty((n_tok, n_embd), dtype=torch.float32, device=dev),
                     ws=q.moe_workspace(n_tok, n_embd, n_ff, E, U, dev),
                     ws8=q.moe_r8_workspace(n_tok, n_embd, n_ff, E, U, dev))
            d["r8"] = dict(w_up_gate_r8=d["wug_r8"], w_down_r8=d["wd_r8"], x=d["xf"], ids=d["ids"],
                           cw=d["cw"], h=d["h"], out=d["out"], ws=d["ws8"])
            if n_tok == 1:
                d["r8f"] = dict(d["r8"], ws=q.moe_r8_fused_workspace(n_embd, n_ff, E, U, dev))
            layers.append(d)
        ug = [dict(w_up_gate=d["wug"], x=d["xf"], ids=d["ids"], h=d["h"], ws=d["ws"]) for d in layers]
        dn = [dict(w_down=d["wd"], h=d["h"], ids=d["ids"], cw=d["cw"], out=d["out"], ws=d["ws"])
              for d in layers]
        r8all = [d["r8"] for d in layers]

        def chained_native():
            for d in layers:
                q.moe_up_gate_swiglu(d["wug"], d["xf"], d["ids"], n_embd, n_ff, E, d["ws"], h=d["h"])
                q.moe_down_combine(d["wd"], d["h"], d["ids"], d["cw"], n_ff, n_embd, E, d["ws"],
                                   out=d["out"])

        def chained_r8():
            for d in layers:
                q.moe_r8_ffn_batched([d["r8"]], n_embd, n_ff, E)

        def chained_r8_fused():
            for d in layers:
                q.moe_r8_ffn_fused(d["r8f"], n_embd, n_ff, E)

        def grouped_native():
            q.moe_up_gate_swiglu_batched(ug, n_embd, n_ff, E)
            q.moe_down_combine_batched(dn, n_ff, n_embd, E)

        def grouped_r8():
            q.moe_r8_ffn_batched(r8all, n_embd, n_ff, E)

        nl = 2 if n_tok == 1 else 3         # up_gate, down (+ combine from 2 tokens on)
        forms = {"chained_native": (chained_native, f"native rows, {nl} launches per layer, layer "
                                                    "after layer"),
                 "chained_r8": (chained_r8, f"R8 expert weights, {nl} launches per layer, layer "
                                            "after layer"),
                 **({"chained_r8_fused": (chained_r8_fused, "R8 expert weights, one launch per "
                                                            "layer (moe_r8_ffn_fused), layer after "
                                                            "layer")} if n_tok == 1 else {}),
                 "grouped_native": (grouped_native, "native rows, all 30 layers in one up_gate "
                                                    "and one down call (3 launches: up_gate, down, "
                                                    "combine)"),
                 "grouped_r8": (grouped_r8, "R8 expert weights, all 30 layers in one call "
                                            f"({nl} launches)")}
        graphs = {}
        for key, (fn, _) in forms.items():
            fn()
            torch.cuda.synchronize()

            def body(fn=fn):
                for _ in range(steps):
                    fn()
            graphs[key] = capture(body)
        prot = protocol(graphs, rounds=6, best_of=3)
        res = {"tokens": n_tok, "active_weight_bytes_per_step": active}
        for key, (_, desc) in forms.items():
            tt = prot[key]["median"] / steps
            res[key] = {"timing": desc, "us_per_step": round(tt * 1e6, 2),
                        "gbs": round(active / tt / 1e9, 1),
                        "frac": round(active / tt / 1e9 / HBM_PEAK_GBS, 4),
                        "tokens_per_s": round(n_tok / tt, 1)}
        c4[f"tokens_{n_tok}"] = res
        del layers, ug, dn, r8all, graphs
    out["c4_moe_expert_ffn_30_layers"] = c4
    del wl
    torch.cuda.synchronize()
    # --- the prefill GEMM 512 x 4096 x 14336 on the int8 matrix cores
    m, n, k = 512, 14336, 4096
    w = q.q8_0_quantize_rows(synth.normal_f32_torch((n, k), 0.02, dev, 0, "c5a", "w"))
    x = q.q8_0_quantize_rows(synth.normal_f32_torch((m, k), 1.0, dev, 0, "c5a", "x"))
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    reps = 20
    prot = protocol({"gemm": many(lambda: q.q8_0_matmul(w, x, n, k, m, y=y))}, rounds=6, best_of=3)
    tt = prot["gemm"]["median"] / reps
    ops = 2 * m * n * k
    out["c5a_prefill_gemm"] = {
        "shape": [m, n, k], "kernel": "gemm_q8_kernel",
        "timing": f"{reps} launches per graph; 6 rounds (first dropped), best of 3, median",
        "us": round(tt * 1e6, 2), "tops": round(ops / tt / 1e12, 1),
        "frac_of_int8_peak": round(ops / tt / 1e12 / 5000.0, 4),
        "prompt_tokens_per_s_equiv": round(m / tt, 1)}
    del w, x, y
    # --- the expert FFN for 512 prompt tokens of one layer (grouped matrix-core
    # products), over native rows and over R8 rows
    n_tok, E, n_embd, n_ff, U = 512, 128, 2048, 768, 8
    wug = q.q8_0_quantize_rows(synth.normal_f32_torch((E * 2 * n_ff, n_embd), 0.02, dev, 0, "c4p", "ug"))
    wd = q.q8_0_quantize_rows(synth.normal_f32_torch((E * n_embd, n_ff), 0.02, dev, 0, "c4p", "down"))
    ids_h = synth.expert_ids(n_tok, U, E, 0, "c4p", "ids")
    ids = torch.from_numpy(ids_h).to(dev)
    cw = torch.from_numpy(synth.combine_weights(n_tok, U, 0, "c4p", "cw")).to(dev)
    xf = synth.normal_f32_torch((n_tok, n_embd), 1.0, dev, 0, "c4p", "x")
    h = torch.empty((n_tok, U, n_ff), dtype=torch.float32, device=dev)
    o = torch.empty((n_tok, n_embd), dtype=torch.float32, device=dev)
    ws = q.moe_workspace(n_tok, n_embd, n_ff, E, U, dev)
    r8 = dict(w_up_gate_r8=q.q8_0_repack_r8(wug, E * 2 * n_ff, n_embd),
              w_down_r8=q.q8_0_repack_r8(wd, E * n_embd, n_ff), x=xf, ids=ids, cw=cw,
              h=torch.empty_like(h), out=torch.empty_like(o),
              ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, E, U, dev))
    active = len(np.unique(ids_h)) * (q8_bytes(2 * n_ff, n_embd) + q8_bytes(n_embd, n_ff))
    macs = n_tok * U * (n_embd * 2 * n_ff + n_ff * n_embd)
    reps = 5

    def native():
        q.moe_up_gate_swiglu(wug, xf, ids, n_embd, n_ff, E, ws, h=h)
        q.moe_down_combine(wd, h, ids, cw, n_ff, n_embd, E, ws, out=o)
    prot = protocol({"r8": many_n(lambda: q.moe_r8_ffn_batched([r8], n_embd, n_ff, E), reps),
                     "native": many_n(native, reps)}, rounds=6, best_of=3)
    c4p = {"tokens": n_tok, "shape": {"n_embd": n_embd, "n_ff": n_ff, "n_expert": E, "n_used": U},
           "active_weight_bytes": active,
           "timing": f"{reps} layers per graph; 6 rounds (first dropped), best of 3, median"}
    for key, desc in (("r8", "R8 expert weights, one moe_r8_ffn_batched call (4 launches)"),
                      ("native", "native rows, moe_up_gate_swiglu + moe_down_combine (6 launches)")):
        tt = prot[key]["median"] / reps
        c4p[key] = {"timing": desc, "us_per_layer": round(tt * 1e6, 2),
                    "prompt_tokens_per_s": round(n_tok / tt, 1),
                    "gbs": round(active / tt / 1e9, 1),
                    "frac": round(active / tt / 1e9 / HBM_PEAK_GBS, 4),
                    "tops": round(2 * macs / tt / 1e12, 1)}
    out["c4p_moe_expert_ffn_prefill_512_tokens"] = c4p
    return out


def read_traffic(path):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel sources have changed since the counters were taken."""
    import hashlib
    with open(path) as f:
        t = json.load(f)
    h = hashlib.sha256()
    for fn in t["source_files"]:
        with open(os.path.join(ROOT, fn), "rb") as g:
            h.update(g.read())
    return t["bytes_per_launch"] if h.hexdigest()[:16] == t["source_hash"] else None


# ---------------------------------------------------------------------------
# profile summaries (reads a rocprofv3 rocpd database; no GPU needed)

def _short(name, width=72):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def rocpd_summary(db):
    """Per-kernel dispatch statistics and per-dispatch PMC counter means."""
    import collections
    import sqlite3
    c = sqlite3.connect(db)
    out = []
    kd = collections.defaultdict(list)
    try:
        for name, start, end in c.execute("select name, start, end from kernels"):
            kd[name].append((end - start) / 1e3)
    except sqlite3.OperationalError:
        pass
    if kd:
        tot = sum(sum(v) for v in kd.values())
        out.append(f"{'kernel':72s} {'calls':>6s} {'mean_us':>9s} {'min_us':>8s} "
                   f"{'max_us':>8s} {'total%':>7s}")
        for k, v in sorted(kd.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{_short(k):72s} {len(v):6d} {sum(v) / len(v):9.3f} {min(v):8.3f} "
                       f"{max(v):8.3f} {100 * sum(v) / tot:7.2f}")
    pm = collections.defaultdict(list)
    try:
        for name, ctr, val in c.execute("select name, counter_name, counter_value from pmc_events"):
            pm[(name, ctr)].append(val)
    except sqlite3.OperationalError:
        pass
    if pm:
        out.append(f"{'kernel':72s} {'counter':>12s} {'dispatches':>10s} {'mean/dispatch':>14s}")
        for (k, ctr), v in sorted(pm.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{_short(k):72s} {ctr:>12s} {len(v):10d} {sum(v) / len(v):14.1f}")
    return "\n".join(out)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2",
                    choices=["c1", "c2", "c3", "c4b1", "c4b16", "c4p", "c5a", "c5b", "copy", "readbw",
                             "ffn", "r8", "kq"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload: leave out the vocabulary-projection and MoE keys")
    ap.add_argument("--read-bytes", type=int, default=0,
                    help="readbw workload: bytes per read launch (default 2 GiB)")
    ap.add_argument("--moe-mode", default="both", choices=["both", "layers", "grouped"],
                    help="c4b1/c4b16: time the layer-after-layer launches, the grouped "
                         "launches, or both")
    ap.add_argument("--cpu-sample-steps", type=int, default=1700,
                    help="steps of the CPU oracle sample (about 10 s of work on 16 host threads)")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with the rocprofv3-derived HBM bytes per launch")
    ap.add_argument("--rocpd-summary", default=None, metavar="DB",
                    help="print a kernel / counter summary of a rocprofv3 database and exit")
    args = ap.parse_args()
    if args.rocpd_summary:
        print(rocpd_summary(args.rocpd_summary))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the sharding design is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import moe_expert_ffn_q8_amd as q
    import synth

    if args.workload == "c2":
        out, plan = bench_decode(args, q, synth, LLAMA_STACKS, 1, "c2",
                                 "llama2-110m-shaped Q8_0 decode step, batch 1, 85 matvecs, "
                                 "{K} sequential steps timed", 200)
        stacks, m = LLAMA_STACKS, 1
        del plan
        if not args.no_extra:
            out.update(default_extras(args, q, synth))
    elif args.workload == "c3":
        out, plan = bench_decode(args, q, synth, GPT2_STACKS, 8, "c3",
                                 "gpt2-124m-shaped Q8_0 decode step, batch 8, 49 matmuls, "
                                 "{K} sequential steps timed", 200)
        stacks, m = GPT2_STACKS, 8
    else:
        print(json.dumps(run_extra(args, q, synth)))
        return

    traffic_file = args.traffic or os.path.join(
        ROOT, "profiles", "r8_matvec_kernel_llama110m_decode_step.traffic.json"
        if args.workload == "c2" else "stream_mfma_kernel_gpt2_batch8_decode_step.traffic.json")
    if traffic_file and os.path.exists(traffic_file):
        t = read_traffic(traffic_file)
        out["roofline"]["traffic"] = t
        out["roofline"]["traffic_source"] = (
            os.path.relpath(traffic_file, ROOT) if t is not None else
            "counters taken on older kernel sources: not applicable")

    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        gbs, dt, nbytes = cpu_baseline_steps(stacks, m, args.cpu_sample_steps, threads)
        gbs1, dt1, nbytes1 = cpu_baseline_steps(stacks, m, max(1, args.cpu_sample_steps // 16), 1)
        out["cpu_baseline"] = {
            "value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{args.cpu_sample_steps} steps of the same workload shapes "
                      f"({nbytes / 1e9:.2f} GB of Q8_0 products, weights and inputs from "
                      f"the seeded numpy generator), oracle products (slices of <= 4096 "
                      f"rows) spread over {threads} threads, {dt:.1f} s wall",
            "tokens_per_s": round(m * args.cpu_sample_steps / dt, 2),
            "one_thread": {"value": round(gbs1, 3), "unit": "GB/s",
                           "sample": f"{max(1, args.cpu_sample_steps // 16)} steps, "
                                     f"{nbytes1 / 1e9:.2f} GB, {dt1:.1f} s wall"},
            "cpu_model": cpu_model(),
        }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
