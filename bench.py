#!/usr/bin/env python3
"""Benchmark of the LSA hot path on one MI355X.

Default workload (--config c5): cross-layer-index prefill of one sequence of
L = 131072 tokens over two layers; indexer H_I = 64 heads, d_I = 128, int8;
4 sinks + 1024-token window + top-k to 2048 keys; per layer 64 query heads
on one bf16 KV head of dim 128. One step = fused indexer scoring + top-k
selection for every row (lsa_select_topk), then sparse attention for every
row of both layers, which reuse the one index (lsa_sparse_attn_prefill).
--config c2 is the same step at L = 32768 with one layer and a 512 window.
Decode workloads (--config c3 / c4) time one decode step: selection for
the target row of every sequence, then split-KV attention with the merge;
the step is captured once as a HIP graph and the timed steps replay it
(per-call parts come from an eager pass of the same steps).

Inputs are synthetic and seeded, and resident in HBM before timing starts.
Prints ONE JSON line: throughput over the timed steps, per-call times from
HIP events on the stream the calls run on, per-kernel launch times from the
library's own event timing over the same number of further steps, the
roofline of the kernel with the most time per step, and the CPU oracle timed
on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c5]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_I8_TOPS = 5000.0      # MI355X dense int8, TOP/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16, TFLOP/s
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, GB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--config", default="c5", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--op", default="path", choices=["path", "backward", "kl"],
                   help="path: the hot path of the workload (default); backward / kl: the training "
                        "operators on a prefill workload's selected lists")
    p.add_argument("--fused", action="store_true",
                   help="HI decode (c4): the step as one fused call (lsa_hier_decode_step) instead of "
                        "lsa_hier_select + lsa_sparse_attn_decode")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="time budget of the oracle sample")
    p.add_argument("--copy-probe", action="store_true",
                   help="end with three plain 1 GiB device copies (HBM counter calibration)")
    return p.parse_args()


def candidate_pairs(L, n_sink, W, K_tot):
    """Scored (query, key) pairs of a causal prefill: rows t >= K_tot score
    the candidates n_sink..t-W; shorter rows keep every key unscored."""
    n = L - K_tot
    if n <= 0:
        return 0
    first = K_tot - W - n_sink + 1
    return n * first + n * (n - 1) // 2


class EventTimer:
    """HIP events recorded on torch's current stream (the stream the binding
    passes to the library) around each call of a named part."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = {}

    def __call__(self, name, fn, *a, **kw):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*a, **kw)
        e1.record()
        self.pending.setdefault(name, []).append((e0, e1))
        return r

    def ms(self, name):
        ev = self.pending.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ev) / max(1, len(ev)), len(ev)


def spread(xs):
    """Median, min and max of per-step times (event-timed)."""
    xs = sorted(xs)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"median": round(med, 4), "min": round(xs[0], 4), "max": round(xs[-1], 4)}


def copy_gbs(torch, nbytes=1 << 30, reps=5):
    """Read + write GB/s of a plain 1 GiB device-to-device copy (event-timed)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


KERNELS = ("index_prefill_kernel", "index_decode_kernel", "index_score_kernel", "select_stage_a",
           "select_stage_b", "attn_prefill_kernel", "attn_decode_partial", "attn_decode_merge",
           "fill_zero_kernel", "attn_bwd_kernel", "bwd_count_kernel", "bwd_scan_kernel", "bwd_fill_kernel",
           "bwd_reduce_kernel", "attn_bwd_finish_kernel", "kl_warmup_kernel", "hi_step_kernel",
           "filter_threshold_kernel", "filter_select_kernel", "select_stage_m")


def kernel_times(L, torch, step, steps, park=False):
    """Per-kernel launch durations over `steps` more steps, from the HIP events
    the library records on the launch stream around each of its kernel
    launches: {name: (mean ms per launch, launches per step)}. park: first
    hold the GPU on a spin kernel so that the host queues every launch before
    the GPU reaches it (short launches would otherwise include host latency
    between their two events)."""
    L.lsa_kernel_timing(True)
    try:
        if park:
            torch.cuda._sleep(50_000_000)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        out = {}
        for name in KERNELS:
            ms, n = L.lsa_kernel_time(name)
            if n:
                out[name] = (ms, n / steps)
    finally:
        L.lsa_kernel_timing(False)
    return out


def measured_mfma_peak(torch, L, kind, data=None, n_wg=256 * 8, iters=2048, reps=3):
    """TOP/s (kind 0, int8) or TFLOP/s (kind 1, bf16) of the library's
    matrix-core probe: register-only MFMA chains on every CU (two waves per
    SIMD, one round), event-timed. With data = (a, b), the operands are fragments of
    those device tensors (a different pair for every instruction) instead of
    constants."""
    sink = torch.empty(n_wg, dtype=torch.int32, device="cuda")

    def launch(it):
        if data is None:
            return L.lsa_probe_mfma(kind, n_wg, it, sink)
        return L.lsa_probe_mfma_data(kind, n_wg, it, data[0], data[1], sink)

    launch(iters // 8)  # warm the clock up
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops = launch(iters)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def probe_operands(torch, wl, kind):
    """Operand bytes with the workload's value distribution, for the probe:
    int8 -- the indexer's A operand (query bytes times the head weight, as the
    kernel folds them when every product fits int8) and its key bytes; bf16 --
    N(0, 1) keys and queries as the attention kernels multiply them."""
    from long_context_sparse_lsa_amd import synth
    if kind == 0:
        q = synth.int8_uniform((1024, wl.H_I, wl.d_I), wl.qk_lo, wl.qk_hi, synth.seed_of("probe", "q"), "cuda")
        w = torch.as_tensor(synth.int_weights(wl.H_I, wl.w_lo, wl.w_hi, synth.seed_of("probe", "w")),
                            dtype=torch.int32, device="cuda")
        a = q.to(torch.int32) * w.view(1, -1, 1)
        if wl.w_lo >= 0 and int(a.min()) >= -128 and int(a.max()) <= 127:
            q = a.to(torch.int8)
        k = synth.int8_uniform((16384, wl.d_I), wl.qk_lo, wl.qk_hi, synth.seed_of("probe", "k"), "cuda")
        return q.contiguous(), k
    a = synth.bf16_normal((16384, 128), synth.seed_of("probe", "bk"), "cuda")
    b = synth.bf16_normal((16384, 128), synth.seed_of("probe", "bq"), "cuda")
    return a, b


def roofline(bound, name, work_per_step, kt, peak, unit):
    """Roofline of one kernel: work_per_step ops (unit T*/s) or bytes (GB/s)
    done by its launches in one step, over their event-measured duration."""
    ms, per_step = kt[name]
    work = work_per_step / per_step  # per launch (mean)
    achieved = work / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None,
            "work_per_launch": work, "ms_per_launch": round(ms, 4), "launches_per_step": per_step}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def measured_traffic(workload, kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of the
    kernel on this workload from profiles/hbm_traffic.txt, or None when the
    file lacks it or was taken on other kernel sources."""
    from long_context_sparse_lsa_amd.profile_summary import sources_hash
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    head = [ln for ln in lines if ln.startswith("sources:")]
    if not head or head[0].split()[1] != sources_hash():
        return None
    for ln in lines:
        f = ln.split()
        if len(f) >= 4 and f[0] == workload and f[1] == kernel:
            kv = dict(x.split("=") for x in f[2:])
            return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def dominant(kt, candidates):
    """The candidate kernel with the most time per step."""
    have = [k for k in candidates if k in kt]
    return max(have, key=lambda k: kt[k][0] * kt[k][1])


def kernel_parts(kt):
    return {k: {"ms_per_launch": round(ms, 4), "launches_per_step": n, "ms_per_step": round(ms * n, 4)}
            for k, (ms, n) in kt.items()}


def prefill_cpu_baseline(wl, q_idx, k_idx, w, q, k, v, seconds):
    """The oracle on query rows drawn uniformly from [K_tot, L) until `seconds`
    pass: scoring against every earlier key, selection, attention per layer."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(5)
    qn = q_idx[0].cpu().numpy()
    kn = k_idx[0].cpu().numpy()
    kf, vf = k[0].cpu().double().numpy(), v[0].cpu().double().numpy()
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        t = int(rng.integers(wl.K_tot, wl.L))
        S = O.index_scores(qn[t:t + 1], kn[: t + 1], w, q_off=t)[0]
        sel = O.select_flat(S, t, wl.n_sink, wl.n_window, wl.k_dyn)
        qt = q[0, t].cpu().double().numpy()
        for _ in range(wl.n_layers):
            O.attend(qt, kf, vf, sel, wl.scale)
        n += 1
    dt = time.perf_counter() - t0
    return n / dt, n, dt


def run_prefill(args, wl, torch):
    from long_context_sparse_lsa_amd import _lib as L
    from long_context_sparse_lsa_amd import synth
    dev = "cuda"
    q_idx, k_idx, w = synth.indexer_inputs(wl, dev)
    layers = [synth.attention_inputs(wl, layer, dev) for layer in range(wl.n_layers)]
    torch.cuda.synchronize()
    timer = EventTimer(torch)

    def step(tm):
        idx, n_sel = tm("select", L.lsa_select_topk, q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
        for q, k, v in layers:   # every layer reuses the one index (CLI)
            tm("attn", L.lsa_sparse_attn_prefill, q, k, v, idx, n_sel)
        return idx, n_sel

    plain = lambda name, fn, *a, **kw: fn(*a, **kw)  # noqa: E731
    for _ in range(args.warmup):
        step(plain)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ev = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        idx, n_sel = step(timer)
        e1.record()
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    step_stats = spread([a.elapsed_time(b) for a, b in step_ev])
    sel_ms, _ = timer.ms("select")
    attn_ms, n_attn = timer.ms("attn")

    pairs = candidate_pairs(wl.L, wl.n_sink, wl.n_window, wl.K_tot)
    i8_ops = 2.0 * wl.H_I * wl.d_I * pairs
    n_sel_sum = float(n_sel.sum().item())
    attn_flop = 4.0 * wl.H * wl.D * n_sel_sum
    gathered = 2.0 * wl.D * 2 * n_sel_sum
    sel_tops = i8_ops / (sel_ms * 1e-3) / 1e12
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    kt = kernel_times(L, torch, lambda: step(plain), args.steps)
    # algorithmic work of each kernel in one step
    work = {"index_prefill_kernel": ("mfma", i8_ops, PEAK_I8_TOPS, "TOP/s"),
            "select_stage_a": ("hbm", 4.0 * pairs, PEAK_HBM_GBS, "GB/s"),  # the scores it reads
            "attn_prefill_kernel": ("mfma", attn_flop * wl.n_layers, PEAK_BF16_TFLOPS, "TFLOP/s")}
    name = dominant(kt, work)
    bound, wk, peak, unit = work[name]
    roof = roofline(bound, name, wk, kt, peak, unit)
    roof["traffic"] = measured_traffic(wl.name, name)
    out = {
        "metric": "LSA prefill tokens/s",
        "value": round(wl.L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+bf16", "data": "synthetic (seeded int8 U[lo,hi] indexer, bf16 N(0,1) q/k/v)",
        "config": {"workload": wl.name, "global_batch": wl.B, "seq_len": wl.L, "layers": wl.n_layers,
                   "H_I": wl.H_I, "d_I": wl.d_I, "H": wl.H, "D": wl.D,
                   "n_sink": wl.n_sink, "n_window": wl.n_window, "K_tot": wl.K_tot, "parallelism": "none"},
        "parts": {"select_ms": round(sel_ms, 4), "select_int8_tops": round(sel_tops, 1),
                  "scored_pairs": pairs,
                  "attn_ms_per_layer": round(attn_ms, 4), "attn_bf16_tflops": round(attn_tflops, 1),
                  "attn_gather_gbs": round(gathered / (attn_ms * 1e-3) / 1e9, 1),
                  "step_ms": step_stats,
                  "kernels": kernel_parts(kt)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        q, k, v = layers[0]
        rate, n, dt = prefill_cpu_baseline(wl, q_idx, k_idx, w, q, k, v, args.cpu_seconds)
        out["cpu_baseline"] = {"value": round(rate, 3), "unit": "tokens/s", "cores": cpu_threads(),
                               "kind": "oracle",
                               "extrapolated_s_per_step": round(wl.L / rate, 1),
                               "sample": f"{n} query rows drawn uniformly from [{wl.K_tot}, {wl.L}) in {dt:.1f} s; "
                                         f"each: exact scores against all earlier keys, top-k, "
                                         f"{wl.n_layers}x float64 attention"}
    return out


def run_training_op(args, wl, torch):
    """One training operator on a prefill workload: the selection and the
    forward (with lse) run once, untimed; a step is one call of the
    deterministic backward (--op backward) or of the warm-up KL operator
    (--op kl) over every row of one layer."""
    import numpy as np
    from long_context_sparse_lsa_amd import _lib as L
    from long_context_sparse_lsa_amd import synth
    dev = "cuda"
    q_idx, k_idx, w = synth.indexer_inputs(wl, dev)
    q, k, v = synth.attention_inputs(wl, 0, dev)
    idx, n_sel = L.lsa_select_topk(q_idx, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn, q_off=0)
    o, lse = L.lsa_sparse_attn_prefill(q, k, v, idx, n_sel, want_lse=True)
    del q_idx
    if args.op == "backward":
        d_o = synth.bf16_normal(q.shape, synth.seed_of(wl.name, "d_o"), dev)

        def step():
            return L.lsa_sparse_attn_backward(q, k, v, idx, n_sel, o, lse, d_o)
    else:
        # logits: seeded N(0, 1) per listed key (the indexer's own logits in training)
        g = torch.Generator(device=dev)
        g.manual_seed(synth.seed_of(wl.name, "logits"))
        logits = torch.randn(idx.shape, generator=g, device=dev, dtype=torch.float32)

        def step():
            return L.lsa_kl_warmup(q, k, idx, n_sel, lse, logits)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kt = kernel_times(L, torch, step, args.steps)
    pairs = float(n_sel.sum().item())
    if args.op == "backward":
        # five products per (row, key) pair and head: S, dP, dQ, dK, dV
        work = {"attn_bwd_kernel": ("mfma", 10.0 * wl.H * wl.D * pairs, PEAK_BF16_TFLOPS, "TFLOP/s"),
                # the bf16 contributions the reduce reads (512 B per pair)
                "bwd_reduce_kernel": ("hbm", 512.0 * pairs, PEAK_HBM_GBS, "GB/s")}
        metric = "LSA sparse attention backward tokens/s"
    else:
        work = {"kl_warmup_kernel": ("mfma", 2.0 * wl.H * wl.D * pairs, PEAK_BF16_TFLOPS, "TFLOP/s")}
        metric = "LSA warm-up KL tokens/s"
    name = dominant(kt, work)
    bound, wk, peak, unit = work[name]
    roof = roofline(bound, name, wk, kt, peak, unit)
    roof["traffic"] = measured_traffic(wl.name + "_" + args.op, name)
    out = {
        "metric": metric, "value": round(wl.L * wl.B / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the workload's seeded inputs; d_o / logits bf16 / fp32 N(0,1))",
        "config": {"workload": wl.name + "_" + args.op, "global_batch": wl.B, "seq_len": wl.L, "H": wl.H,
                   "D": wl.D, "K_tot": wl.K_tot, "selected_pairs": int(pairs), "parallelism": "none"},
        "parts": {"kernels": kernel_parts(kt)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        import oracle as O
        rng = np.random.default_rng(7)
        qn, kn, vn = (x[0].cpu() for x in (q, k, v))
        In, Nn = idx[0].cpu().numpy(), n_sel[0].cpu().numpy()
        kf, vf = kn.double().numpy(), vn.double().numpy()
        dof = (d_o[0].cpu().double().numpy() if args.op == "backward" else None)
        lgn = logits[0].cpu().double().numpy() if args.op == "kl" else None
        n = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            t = int(rng.integers(wl.K_tot, wl.L))
            sel = In[t, :Nn[t]]
            qt = qn[t].double().numpy()
            if args.op == "backward":
                O.attend_backward(qt, kf, vf, sel, wl.scale, dof[t])
            else:
                O.kl_warmup_row(qt, kf, sel, wl.scale, lgn[t, :Nn[t]])
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": cpu_threads(),
                               "kind": "oracle",
                               "sample": f"{n} rows drawn uniformly from [{wl.K_tot}, {wl.L}) in {dt:.1f} s; "
                                         f"each: the oracle's float64 {args.op} of the row"}
    return out


def decode_cpu_baseline(wl, q_idx, k_idx, w, q, kc, vc, seconds, blk_summary):
    """The oracle on whole sequences of the decode step until `seconds` pass."""
    import numpy as np
    import oracle as O
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < wl.B:
        b = n
        kn = k_idx[b].cpu().numpy()
        qn = q_idx[b].cpu().numpy()
        if wl.blk:
            sel = O.hier_select(qn, kn, blk_summary[b].cpu().numpy(), w, wl.blk, wl.n_blk_recall,
                                wl.n_sink, wl.n_window, wl.k_dyn)
        else:
            sel = O.decode_select(qn, kn, w, wl.n_sink, wl.n_window, wl.k_dyn)
        O.attend(q[b].reshape(-1, wl.D).cpu().double().numpy(), kc[b].cpu().double().numpy(),
                 vc[b].cpu().double().numpy(), sel, wl.scale)
        n += 1
    dt = time.perf_counter() - t0
    return n, dt


def run_decode(args, wl, torch):
    from long_context_sparse_lsa_amd import _lib as L
    from long_context_sparse_lsa_amd import synth
    dev = "cuda"
    q_idx, k_idx, w = synth.indexer_inputs(wl, dev)
    q, kc, vc = synth.attention_inputs(wl, 0, dev)
    q1 = q_idx[:, None].contiguous()
    kblk = L.lsa_block_summary(k_idx, wl.blk) if wl.blk else None
    summary_us = None
    if wl.blk:
        # the HI block summaries of the whole cache (built once per cache, then
        # kept current on append): timed apart from the step, as the kernel's
        # own launch time (the library's event timing)
        for _ in range(3):  # warm-up, as for the step
            L.lsa_block_summary(k_idx, wl.blk)
        torch.cuda.synchronize()
        L.lsa_kernel_timing(True)
        for _ in range(20):
            L.lsa_block_summary(k_idx, wl.blk)
        torch.cuda.synchronize()
        summary_us = L.lsa_kernel_time("block_summary_kernel")[0] * 1e3
        L.lsa_kernel_timing(False)
    step_ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev) if (wl.blk and args.fused) else None
    torch.cuda.synchronize()
    timer = EventTimer(torch)
    N = wl.L

    def step(tm):
        if wl.blk and args.fused:
            # the whole step in one fused call (its counters in a kept workspace)
            return tm("step", L.lsa_hier_decode_step, q_idx, k_idx, kblk, w, q, kc, vc, wl.blk, wl.n_blk_recall,
                      wl.n_sink, wl.n_window, wl.k_dyn, n_split=wl.n_split, ws=step_ws)[2]
        if wl.blk:
            idx, n_sel = tm("select", L.lsa_hier_select, q_idx, k_idx, kblk, w, wl.blk, wl.n_blk_recall,
                            wl.n_sink, wl.n_window, wl.k_dyn)
            idx, n_sel = idx[:, None], n_sel[:, None]
        else:
            idx, n_sel = tm("select", L.lsa_select_topk, q1, k_idx, w, wl.n_sink, wl.n_window, wl.k_dyn,
                            q_off=N - 1)
        # the n_q rows of a sequence (target + MTP drafts) share the one index (CLI)
        return tm("attn", L.lsa_sparse_attn_decode, q, kc, vc, idx, n_sel, n_split=wl.n_split)

    plain = lambda name, fn, *a, **kw: fn(*a, **kw)  # noqa: E731
    for _ in range(args.warmup):
        step(plain)
    torch.cuda.synchronize()
    # per-call parts from one eager pass of the steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    us_eager = (time.perf_counter() - t0) * 1e6 / args.steps
    sel_ms, _ = timer.ms("select")
    attn_ms, _ = timer.ms("attn")
    fused_ms, _ = timer.ms("step")
    # the timed steps: one decode step captured once as a HIP graph and
    # replayed, as a serving loop runs a fixed-shape step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(plain)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t0) * 1e6 / args.steps
    # the spread of single replays, from a separate untimed pass (events
    # between replays would add their host latency to the timed loop)
    step_ev = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        step_ev.append((e0, e1))
    torch.cuda.synchronize()
    step_stats = spread([a.elapsed_time(b) * 1e3 for a, b in step_ev])
    # the same replays with the last-level cache (256 MB MALL) flushed before
    # each one by reading 512 MB, untimed: a step that follows other work (a
    # read leaves clean lines, so the step pays no write-back of the flush)
    flush = torch.zeros(64 << 20, dtype=torch.int64, device=dev)
    flush.sum()
    cold = []
    for _ in range(args.steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        cold.append((e0, e1))
    torch.cuda.synchronize()
    us_cold = sum(a.elapsed_time(b) for a, b in cold) * 1e3 / len(cold)
    del flush
    K_tot = wl.K_tot
    kv_bytes = wl.B * K_tot * wl.D * 2 * 2
    qo_bytes = 2 * wl.B * wl.n_q * wl.H * wl.D * 2
    if wl.blk:
        nb = N // wl.blk
        idx_bytes = wl.B * (nb * wl.d_I + wl.n_blk_recall * wl.blk * wl.d_I)
    else:
        idx_bytes = wl.B * N * wl.d_I
    step_bytes = idx_bytes + kv_bytes + qo_bytes
    kt = kernel_times(L, torch, lambda: step(plain), args.steps, park=True)
    # algorithmic bytes of each kernel in one step: the indexer keys it scans,
    # the scores the selection reads, the K/V rows and q the attention reads
    n_scored = (N // wl.blk + wl.n_blk_recall * wl.blk) if wl.blk else N
    work = {"hi_step_kernel": ("hbm", step_bytes, PEAK_HBM_GBS, "GB/s"),
            "index_decode_kernel": ("hbm", idx_bytes, PEAK_HBM_GBS, "GB/s"),
            "select_stage_a": ("hbm", 4.0 * wl.B * n_scored, PEAK_HBM_GBS, "GB/s"),
            "attn_decode_partial": ("hbm", kv_bytes + qo_bytes // 2, PEAK_HBM_GBS, "GB/s")}
    name = dominant(kt, work)
    bound, wk, peak, unit = work[name]
    roof = roofline(bound, name, wk, kt, peak, unit)
    roof["traffic"] = measured_traffic(wl.name, name)
    out = {
        "metric": "LSA decode us/step",
        "value": round(us_step, 2), "unit": "us/step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+bf16", "data": "synthetic (seeded int8 U[-16,15] indexer, bf16 N(0,1) q and caches)",
        "config": {"workload": wl.name + ("_fused" if (wl.blk and args.fused) else ""), "global_batch": wl.B,
                   "context": N, "n_q": wl.n_q, "H": wl.H, "K_tot": K_tot, "n_split": wl.n_split,
                   "hier_blk": wl.blk, "launch": "hip_graph_replay", "parallelism": "none"},
        "parts": {"eager_us_per_step": round(us_eager, 2), "cold_cache_us_per_step": round(us_cold, 2),
                  "step_us": step_stats,
                  "select_us": round(sel_ms * 1e3, 2), "attn_us": round(attn_ms * 1e3, 2),
                  "fused_step_us": round(fused_ms * 1e3, 2),
                  "block_summary": None if summary_us is None else {
                      "us": round(summary_us, 2), "read_bytes": wl.B * N * wl.d_I,
                      "hbm_frac": round(wl.B * N * wl.d_I / (summary_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
                  "step_bytes": step_bytes,
                  "step_hbm_frac": round(step_bytes / (us_step * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "kernels": kernel_parts(kt)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        n, dt = decode_cpu_baseline(wl, q_idx, k_idx, w, q, kc, vc, args.cpu_seconds, kblk)
        out["cpu_baseline"] = {"value": round(dt / max(n, 1) * wl.B * 1e6, 1), "unit": "us/step",
                               "cores": cpu_threads(), "kind": "oracle",
                               "sample": f"{n} of {wl.B} sequences in {dt:.1f} s, scaled to the batch; "
                                         f"each: exact scores and selection, float64 attention of "
                                         f"{wl.n_q} rows"}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(how it would shard is a design note, not code). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_sparse_lsa_amd import configs
    from long_context_sparse_lsa_amd import _lib as L
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.load()
    wl = configs.BY_ID[args.config]
    if args.op != "path":
        if wl.kind != "prefill":
            print("--op backward / kl run on a prefill workload (c1, c2, c5)", file=sys.stderr)
            sys.exit(2)
        out = run_training_op(args, wl, torch)
    else:
        out = run_prefill(args, wl, torch) if wl.kind == "prefill" else run_decode(args, wl, torch)
    roof = out["roofline"]
    if roof["bound"] == "mfma":
        # the rate the matrix cores sustain for this dtype on this GPU in this
        # run (register-only probe): the attainable ceiling next to the
        # published peak
        kind = 0 if roof["unit"] == "TOP/s" else 1
        mp = measured_mfma_peak(torch, L, kind)
        roof["measured_peak"] = round(mp, 1)
        roof["frac_of_measured"] = round(roof["achieved"] / mp, 4)
        # the same on operands with the workload's values: the chip lowers
        # its clock under the power of switching operand bits, so this is
        # the ceiling for the kernel's own data
        mpd = measured_mfma_peak(torch, L, kind, data=probe_operands(torch, wl, kind))
        roof["measured_peak_data"] = round(mpd, 1)
        roof["frac_of_measured_data"] = round(roof["achieved"] / mpd, 4)
    if "attn_bf16_tflops" in out.get("parts", {}):
        # prefill attention against the bf16 probe on N(0, 1) operands
        mpa = measured_mfma_peak(torch, L, 1, data=probe_operands(torch, wl, 1))
        out["parts"]["attn_bf16_measured_peak_data"] = round(mpa, 1)
        out["parts"]["attn_frac_of_measured_data"] = round(out["parts"]["attn_bf16_tflops"] / mpa, 4)
    if roof["bound"] == "hbm":
        # the bandwidth a plain device copy reaches on this GPU in this run: the
        # attainable ceiling next to the 8 TB/s figure
        cg = copy_gbs(torch)
        roof["copy_gbs"] = round(cg, 1)
        roof["frac_of_copy"] = round(roof["achieved"] / cg, 4)
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
