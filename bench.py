"""Benchmark: ms per Mamba2 scan fwd+bwd step on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 16] [--workload pages_shape] [--no-extras]

One step = mamba2_scan_fwd + mamba2_scan_bwd over one batch of seeded synthetic input already resident in HBM.  Prints one JSON line.

Cold protocol (the headline): R input sets rotate so that no step's reads
can be served from the 256 MB Infinity Cache.  Step s runs the forward of
set s % R and the backward of set (s - R/2) % R, so between a set's forward
and its backward R/2 other steps stream far more than the cache holds.
The K timed steps are one captured HIP graph of exactly K steps (steps
0..K-1 of the rotation), timed with HIP events on the stream it is
replayed on and bracketed by device synchronisation.  Ahead of the first
event the stream runs a short spin kernel (about 0.4 ms) while the host
submits the graph, so the events bracket the K steps' kernels and not the
host's graph-launch latency (about 60 us per replay, which at K = 20 read
as 3 us per step); the wall-clock figure keeps both.  A graph's first
replay costs more than later ones (about 3 us per step), so after the W
warmup steps the timed graph is replayed once untimed; that replay's time
is reported as first_replay_ms_per_step.

Warm protocol (secondary): K steps of fwd then bwd of one set, back to back
in one graph, so the backward may find the batch in the Infinity Cache.

Per-kernel durations come from HIP events (on the stream the kernels run on)
around a captured batch of back-to-back launches of one kernel that walks the
same rotation; the dominant kernel's algorithmic bytes over its mean duration
give the roofline figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per fwd+bwd scan step at B=8192,K=8,SH2=256,D=16; % of HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published (bf16 trunk inputs run on these)
SRC = os.path.join(ROOT, "bwd_mamba2_scan_amd", "csrc", "mamba2_scan.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_pages_shape.json")
MAX_STEPS = 2000  # steps of the one captured graph that is timed
HOLD_CYCLES = 1_000_000  # GPU clock cycles of the spin ahead of a timed replay (~0.4 ms)


def hold_gpu():
    """A spin kernel on the current stream (torch's private cycle-sleep
    kernel); without it, the timed replays carry the host's graph-launch
    latency and the protocol string says so."""
    import torch

    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(HOLD_CYCLES)
    return sleep is not None
BLEND_STABILITY = 0.95  # the blend measurement's gate multiplier


def algorithmic_bytes(B, K, SH2, D, trunk_bytes=4):
    """What the method must move, fwd and bwd as separate calls (fp32; the
    trunk inputs h_history and h_s2 at trunk_bytes per value)."""
    f = 4
    H = B * K * SH2 * trunk_bytes
    hs2 = B * SH2 * trunk_bytes
    W = 3 * SH2 * D * f
    vec = B * D * f
    fwd = H + hs2 + W + vec          # read H, h_s2, W_A/B/C; write context
    bwd = H + hs2 + W + vec + W      # read H, h_s2, W_A/B/C, d_context; write dW_A/B/C
    # per kernel: the method's I/O each kernel performs (the backward reads
    # the forward's saved terms instead of the weights)
    per_kernel = {
        "fwd_kernel": fwd,
        "bwd_partials_kernel": H + hs2 + vec,
        "bwd_reduce_kernel": W,
        # optional input gradients: read W and d_context, write d_h_history and
        # d_h_s2 (fp32 whatever the trunk precision)
        "dinput_kernel": W + vec + (B * K * SH2 + B * SH2) * f,
    }
    # the backward with the input gradients: its reads and dW writes, plus the
    # d_h_history and d_h_s2 writes (fp32 whatever the trunk precision)
    per_kernel["bwd_full"] = bwd + (B * K * SH2 + B * SH2) * f
    # the optional blend step: the scan's bytes plus the h_enriched write (h_s2
    # is read already), the d_h_enriched read (in place of d_context) and the
    # temporal weights (read twice, their gradient written)
    per_kernel["blend_step"] = fwd + bwd + hs2 + hs2 - vec + 3 * SH2 * f
    return fwd + bwd, per_kernel


def algorithmic_flops(B, K, SH2, D):
    """Both contractions of both passes, one FMA = 2 flops (the O(B*K*D) scan excluded)."""
    per_pass = 2 * B * K * SH2 * 2 * D + 2 * B * SH2 * D
    per_kernel = {"fwd_kernel": per_pass, "bwd_partials_kernel": per_pass, "bwd_reduce_kernel": 0}
    return 2 * per_pass, per_kernel


def src_digest():
    with open(SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counters, if they match this source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != src_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(workload_name, budget_s=12.0):
    """The oracle, as it stands, on the host cores (rank 0 only)."""
    from oracle import mamba2_oracle as orc
    from tests.inputs import workload_inputs

    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = os.cpu_count() or 1
    inp = workload_inputs(workload_name)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        orc.fwd_bwd(inp)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 1000:
            break
    out = {
        "value": round(statistics.median(times) * 1e3, 3),
        "unit": "ms",
        "cores": cores,
        "kind": "oracle",
        "sample": f"full {workload_name} batch (fp64 numpy oracle fwd+bwd), median of {len(times)} runs "
                  f"in {time.perf_counter() - t_start:.1f} s",
    }
    # the same on one thread (BLAS limited to 1), a shorter sample
    try:
        from threadpoolctl import threadpool_limits
        one = []
        t1 = time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                t0 = time.perf_counter()
                orc.fwd_bwd(inp)
                one.append(time.perf_counter() - t0)
                if time.perf_counter() - t1 > budget_s / 2 or len(one) >= 200:
                    break
        out["single_thread"] = {"value": round(statistics.median(one) * 1e3, 3), "unit": "ms", "cores": 1,
                                "sample": f"median of {len(one)} runs"}
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return out


def parity_gate(m2, torch, t, inputs, input_grads=True):
    """Oracle parity on the benchmarked workload before any timing."""
    from oracle import mamba2_oracle as orc

    ctx, saved = m2.fwd(t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"])
    g = m2.bwd(t["h_history"], t["h_s2"], saved, t["d_context"])
    torch.cuda.synchronize()
    f, b = orc.fwd_bwd(inputs)
    c = ctx.cpu().numpy().astype(np.float64)
    ok = bool(np.all(np.abs(c - f.context) <= 1e-4 * (1 + np.abs(f.context))))
    worst_l1 = 0.0
    for k in ("dW_A", "dW_B", "dW_C"):
        ref = getattr(b, k)
        rel = float(np.sum(np.abs(g[k].cpu().numpy() - ref)) / np.sum(np.abs(ref)))
        worst_l1 = max(worst_l1, rel)
        ok = ok and rel <= 1e-3
    in_err = 0.0
    if input_grads:
        dH, dhs2 = m2.bwd_input(t["W_A"], t["W_B"], t["W_C"], saved, t["d_context"], inputs["h_history"].shape[1])
        torch.cuda.synchronize()
        ig = orc.input_grads(b, inputs["W_A"], inputs["W_B"], inputs["W_C"])
        for got, ref in ((dH, ig.d_h_history), (dhs2, ig.d_h_s2)):
            v = got.cpu().numpy().astype(np.float64)
            in_err = max(in_err, float(np.max(np.abs(v - ref) / (1 + np.abs(ref)))))
    ok = ok and in_err <= 1e-4
    if not ok:
        raise SystemExit(f"parity gate failed on the benchmarked workload (worst dW L1 {worst_l1:.3e}, "
                         f"worst input-gradient error {in_err:.3e})")
    return {"context_max_abs_err": float(np.max(np.abs(c - f.context))), "dW_worst_L1_rel": worst_l1,
            "input_grads_max_rel_err": in_err, "mean_gate": float(np.mean(f.g))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="pages_shape")
    ap.add_argument("--sets", type=int, default=8, help="rotating input sets (even, >= 2)")
    ap.add_argument("--trunk", choices=("fp32", "bf16"), default="fp32",
                    help="storage of h_history and h_s2 (bf16: the *_bf16 entry points; the headline is fp32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the blend, bf16 and long_few measurements (keeps a profile to the headline kernels)")
    args = ap.parse_args()
    if not 1 <= args.steps <= MAX_STEPS or args.warmup < 0:
        ap.error(f"--steps must be in 1..{MAX_STEPS} and --warmup >= 0")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan's batch shards with no communication in the "
              "forward and one small all-reduce of dW in the backward; the multi-GPU path is not "
              "built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bwd_mamba2_scan_amd as m2
    from tests.inputs import WORKLOADS, blend_extras, workload_inputs

    w = WORKLOADS[args.workload]
    B, K, SH2, D = w.B, w.K, w.SH2, w.D
    R = max(2, args.sets + (args.sets & 1))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inputs = workload_inputs(args.workload)
    extras = blend_extras(B, SH2, w.seed)
    base = {k: torch.from_numpy(v).to(dev) for k, v in inputs.items()}
    gate = parity_gate(m2, torch, base, inputs)
    tb = 2 if args.trunk == "bf16" else 4
    if args.trunk == "bf16":
        # the trunk inputs as bf16 (the forward and backward read them as such);
        # the oracle runs on the same rounded values
        from tests.inputs import bf16_round
        rounded = dict(inputs)
        for k in ("h_history", "h_s2"):
            bits, rounded[k] = bf16_round(inputs[k])
            base[k] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        gate["bf16"] = parity_gate(m2, torch, base, rounded, input_grads=False)

    # R distinct copies of the batch at distinct addresses, each with its own
    # context/saved/workspace/dW buffers.
    sets = []
    for r in range(R):
        s = {k: v.clone() for k, v in base.items()}
        s["context"] = torch.empty((B, D), device=dev)
        s["saved"] = m2.alloc_saved(B, K, SH2, D, dev)
        s["ws"] = m2.alloc_workspace(B, K, SH2, D, dev)
        s["dWd"] = {k: torch.empty((SH2, D), device=dev) for k in ("dW_A", "dW_B", "dW_C")}
        s["dH"] = torch.empty((B, K, SH2), device=dev)
        s["dhs2"] = torch.empty((B, SH2), device=dev)
        # the h_enriched blend (an optional step after the path)
        s["he"] = torch.empty((B, SH2), device=dev)
        s["dhe"] = torch.from_numpy(extras["d_h_enriched"]).to(dev)
        s["tw"] = torch.from_numpy(extras["temporal_weight"]).to(dev)
        s["stab"] = torch.tensor([BLEND_STABILITY], dtype=torch.float32, device=dev)
        s["bout"] = {"dW_A": torch.empty((SH2, D), device=dev), "dW_B": torch.empty((SH2, D), device=dev),
                     "dW_C": torch.empty((SH2, D), device=dev), "d_context": torch.empty((B, D), device=dev),
                     "d_temporal_weight": torch.empty((SH2,), device=dev)}
        s["bws"] = torch.empty(m2.blend_workspace_bytes(B, K, SH2, D) // 4, device=dev)
        sets.append(s)
    del base

    def fwd(s):
        m2.fwd(s["h_history"], s["h_s2"], s["W_A"], s["W_B"], s["W_C"], context=s["context"], saved=s["saved"])

    def bwd(s):
        m2.bwd(s["h_history"], s["h_s2"], s["saved"], s["d_context"], workspace=s["ws"], out=s["dWd"])

    # the backward's two kernels, each timed on its own
    def partials(s):
        m2.bwd_partials(s["h_history"], s["h_s2"], s["saved"], s["d_context"], s["ws"])

    def reduce(s):
        m2.bwd_reduce(B, K, SH2, D, s["ws"], s["dWd"]["dW_A"], s["dWd"]["dW_B"], s["dWd"]["dW_C"])

    def fwd_blend(s):
        m2.fwd_blend(s["h_history"], s["h_s2"], s["W_A"], s["W_B"], s["W_C"], stability=s["stab"],
                     temporal_weight=s["tw"], context=s["context"], h_enriched=s["he"], saved=s["saved"])

    def bwd_blend(s):
        m2.bwd_blend(s["h_history"], s["h_s2"], s["saved"], s["dhe"], D, temporal_weight=s["tw"],
                     workspace=s["bws"], out=s["bout"])

    def dinput(s):
        m2.bwd_input(s["W_A"], s["W_B"], s["W_C"], s["saved"], s["d_context"], K, d_h_history=s["dH"],
                     d_h_s2=s["dhs2"])

    # the backward with the input gradients in one call
    def bwd_full(s):
        m2.bwd_full(s["h_history"], s["h_s2"], s["saved"], s["d_context"], s["W_A"], s["W_B"], s["W_C"],
                    workspace=s["ws"], out={**s["dWd"], "d_h_history": s["dH"], "d_h_s2": s["dhs2"]})

    def step(i):
        fwd(sets[i % R])
        sb = sets[(i - R // 2) % R]
        bwd(sb)

    # prime every set's saved buffer so the first backwards read real data
    for s in sets:
        fwd(s)
    torch.cuda.synchronize()

    # ---- capture one graph per rotation phase, and one for a whole rotation
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(R):
            step(i)  # warm the path on the capture stream
        torch.cuda.synchronize()
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(i)
            graphs.append(g)
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle, stream=stream):
            for i in range(R):
                step(i)
    torch.cuda.synchronize()

    def run_steps(n):
        for _ in range(n // R):
            cycle.replay()
        for i in range(n % R):
            graphs[i].replay()

    # The K timed steps are one captured graph of exactly K steps (steps
    # 0..K-1 of the rotation), so the host's per-launch gaps stay out
    # and the figure does not depend on how K splits into graphs.  A graph's
    # first replay costs more than later ones (about 3 us per step), so it is
    # replayed once untimed after the warm-up; the timed replay is bracketed
    # by device synchronisations and timed with HIP events on its stream.
    def capture(count, fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    fn(i)
        return g

    def timed_replay(g):
        """(event ms, wall ms) of one replay, synchronised on both sides."""
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            hold_gpu()  # the host submits the graph meanwhile
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), (time.perf_counter() - t0) * 1e3

    timed = capture(args.steps, step)
    torch.cuda.synchronize()
    run_steps(args.warmup)
    first_ev, _ = timed_replay(timed)  # first replay, untimed for the headline
    ev_ms, wall_ms = timed_replay(timed)
    ms_per_step = ev_ms / args.steps
    first_ms = first_ev / args.steps
    del timed

    # ---- spread: one event pair per rotation replay (R steps each)
    rot_ms = []
    with torch.cuda.stream(stream):
        for _ in range(max(4, args.steps // R)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            hold_gpu()
            e0.record(stream)
            cycle.replay()
            e1.record(stream)
            e1.synchronize()
            rot_ms.append(e0.elapsed_time(e1) / R)
    step_pct = {k: round(float(np.percentile(rot_ms, q)), 5) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}

    # ---- warm protocol (secondary): K steps of fwd then bwd of the same set,
    # back to back in one graph, so the backward may read the batch from the
    # Infinity Cache
    def warm_step(i):
        fwd(sets[0])
        bwd(sets[0])

    warm_graph = capture(args.steps, warm_step)
    timed_replay(warm_graph)
    warm_ev, _ = timed_replay(warm_graph)
    warm_ms = warm_ev / args.steps
    del warm_graph

    # ---- per-kernel durations: HIP events around each kernel, cold rotation,
    # eager launches on the current stream (the one the kernels run on)
    # Each kernel is timed over a captured batch of back-to-back launches that
    # walks the rotation (so every launch reads a set the previous R-1 launches
    # did not touch), bracketed by one event pair on the replay stream; the
    # mean per launch is reported.
    names = ("fwd_kernel", "bwd_partials_kernel", "bwd_reduce_kernel")
    kern_fns = {"fwd_kernel": fwd, "bwd_partials_kernel": partials, "bwd_reduce_kernel": reduce,
                "dinput_kernel": dinput}
    n_launch = R * max(2, args.steps // R)
    kern_us = {}
    for name in names + ("dinput_kernel",):
        fn = kern_fns[name]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(n_launch):
                    fn(sets[i % R])
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()  # warm-up replay
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        kern_us[name] = e0.elapsed_time(e1) * 1e3 / n_launch
        del g

    # ---- optional paths (not the step): each timed as a cold rotation replayed
    # from one captured graph
    def graph_us(fn_step, count):
        with torch.cuda.stream(stream):
            for i in range(count):
                fn_step(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    fn_step(i)
            torch.cuda.synchronize()
            g.replay()
            reps = max(2, args.steps // count)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * count)


    # the blend path: fwd_blend(set s) + bwd_blend(set s - R/2)
    def blend_step(i):
        fwd_blend(sets[i % R])
        bwd_blend(sets[(i - R // 2) % R])

    # bf16 trunk inputs (the *_bf16 entry points)
    def fwd16(s):
        m2.fwd(s["h16"], s["hs16"], s["W_A"], s["W_B"], s["W_C"], context=s["context"], saved=s["saved"])

    def bwd16(s):
        m2.bwd(s["h16"], s["hs16"], s["saved"], s["d_context"], workspace=s["ws"], out=s["dWd"])

    def step16(i):
        fwd16(sets[i % R])
        sb = sets[(i - R // 2) % R]
        bwd16(sb)

    # ---- a long history with few samples (chunked forward), its own rotation
    def workload_step_us(name):
        wl = WORKLOADS[name]
        base_in = {k: torch.from_numpy(v).to(dev) for k, v in workload_inputs(name).items()}
        wsets = []
        for _ in range(R):
            x = {k: v.clone() for k, v in base_in.items()}
            x["context"] = torch.empty((wl.B, wl.D), device=dev)
            x["saved"] = m2.alloc_saved(wl.B, wl.K, wl.SH2, wl.D, dev)
            x["ws"] = m2.alloc_workspace(wl.B, wl.K, wl.SH2, wl.D, dev)
            x["dWd"] = {k: torch.empty((wl.SH2, wl.D), device=dev) for k in ("dW_A", "dW_B", "dW_C")}
            wsets.append(x)
        del base_in

        def wstep(i):
            a = wsets[i % R]
            m2.fwd(a["h_history"], a["h_s2"], a["W_A"], a["W_B"], a["W_C"], context=a["context"], saved=a["saved"])
            bset = wsets[(i - R // 2) % R]
            m2.bwd(bset["h_history"], bset["h_s2"], bset["saved"], bset["d_context"], workspace=bset["ws"],
                   out=bset["dWd"])

        for i in range(R):
            a = wsets[i]
            m2.fwd(a["h_history"], a["h_s2"], a["W_A"], a["W_B"], a["W_C"], context=a["context"], saved=a["saved"])
        us = graph_us(wstep, R)
        wbytes, _ = algorithmic_bytes(wl.B, wl.K, wl.SH2, wl.D)
        del wsets
        torch.cuda.empty_cache()
        gbps = wbytes / (us * 1e-6) / 1e9
        return {"workload": name, "B": wl.B, "K": wl.K, "SH2": wl.SH2, "STATE_D": wl.D, "us": round(us, 2),
                "algorithmic_bytes": wbytes, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBS, 4)}

    # the backward with the input gradients: one call against the two separate
    # calls, each a cold rotation replayed from one captured graph
    full_us = graph_us(lambda i: bwd_full(sets[i % R]), 8 * R)
    sep_us = graph_us(lambda i: (bwd(sets[i % R]), dinput(sets[i % R])), 8 * R)

    blend_step_us = bf16_step_us = None
    bf16_kern_us = {}
    long_few = None
    if not args.no_extras and args.trunk == "fp32":
        blend_step_us = graph_us(blend_step, R)
        for st_ in sets:
            st_["h16"] = st_["h_history"].to(torch.bfloat16)
            st_["hs16"] = st_["h_s2"].to(torch.bfloat16)
        bf16_step_us = graph_us(step16, R)
        bf16_kern_us = {"fwd_kernel": graph_us(lambda i: fwd16(sets[i % R]), 8 * R),
                        "bwd": graph_us(lambda i: bwd16(sets[i % R]), 8 * R)}
        for st_ in sets:
            del st_["h16"], st_["hs16"]
        if args.workload == "pages_shape":
            long_few = workload_step_us("long_few")

    # ---- copy ceiling: a 1 GiB device-to-device copy (read + write bytes)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    copy_ms = []
    with torch.cuda.stream(stream):
        for _ in range(6):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            e1.synchronize()
            copy_ms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * src.numel() * 4 / (min(copy_ms[1:]) * 1e-3) / 1e9
    del src, dst

    step_bytes, per_kernel_bytes = algorithmic_bytes(B, K, SH2, D, tb)
    # bf16 trunk inputs: h_history and h_s2 move half the bytes, twice per step
    bf16_bytes = step_bytes - (B * K * SH2 + B * SH2) * 4
    blend_out = bf16_out = None
    if blend_step_us is not None:
        blend_gbps = per_kernel_bytes["blend_step"] / (blend_step_us * 1e-6) / 1e9
        blend_out = {"us": round(blend_step_us, 2), "stability": BLEND_STABILITY,
                     "temporal_weight": "U(0.5, 1.5)", "algorithmic_bytes": per_kernel_bytes["blend_step"],
                     "achieved": round(blend_gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(blend_gbps / HBM_PEAK_GBS, 4)}
        bf16_gbps = bf16_bytes / (bf16_step_us * 1e-6) / 1e9
        bf16_out = {"us": round(bf16_step_us, 2), "algorithmic_bytes": bf16_bytes,
                    "achieved": round(bf16_gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(bf16_gbps / HBM_PEAK_GBS, 4),
                    "kernel_us": {k: round(v, 2) for k, v in bf16_kern_us.items()}}
    flops, per_kernel_flops = algorithmic_flops(B, K, SH2, D)
    dom = max(names, key=lambda n: kern_us[n])
    hbm_us = step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    # the matrix-core peak of the contraction's own type: fp32 trunk inputs
    # give an fp32 contraction, bf16 trunk inputs run on bf16 MFMAs
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if args.trunk == "bf16" else MFMA_FP32_PEAK_TFLOPS
    mfma_us = flops / (mfma_peak * 1e12) * 1e6
    roofline_us = max(hbm_us, mfma_us)
    # the dominant kernel's own bound: bytes at HBM peak vs flops at the MFMA peak
    k_mfma = per_kernel_flops[dom] / (mfma_peak * 1e12) > per_kernel_bytes[dom] / (HBM_PEAK_GBS * 1e9)
    if k_mfma:
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(per_kernel_flops[dom] / (kern_us[dom] * 1e-6) / 1e12, 2),
                "peak": mfma_peak, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(per_kernel_bytes[dom] / (kern_us[dom] * 1e-6) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom) if (args.workload, args.trunk) == ("pages_shape", "fp32") else None

    out = {
        "metric": METRIC,
        "value": round(ms_per_step, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.trunk == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "B": B, "K": K, "SH2": SH2, "STATE_D": D, "trunk": args.trunk,
            "protocol": f"cold: {R} rotating input sets, fwd(set s) + bwd(set s-{R // 2}) per step; "
                        f"the {args.steps} timed steps are one HIP graph, replayed once untimed, then timed "
                        + ("with HIP events after a ~0.4 ms GPU spin that covers the host's graph submission"
                           if hasattr(torch.cuda, "_sleep") else
                           "with HIP events (no GPU spin available: the host's graph submission is included)"),
        },
        "hbm_roofline_frac": round(hbm_us / (ms_per_step * 1e3), 4),
        "roofline_frac_step": round(roofline_us / (ms_per_step * 1e3), 4),
        "step_bound": "mfma" if mfma_us > hbm_us else "hbm",
        "samples_per_s": round(B / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": step_bytes,
        "algorithmic_flops_per_step": flops,
        "achieved_GBps_step": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_ms_per_rotation": step_pct,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "achieved_over_copy_ceiling": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / copy_gbps, 4),
        "wall_ms_per_step": round(wall_ms / args.steps, 5),
        "warm_ms_per_step": round(warm_ms, 5),
        "first_replay_ms_per_step": round(first_ms, 5),
        "kernel_us": {n: round(kern_us[n], 2) for n in names},
        "roofline": roof,
        # not part of the step: the optional input gradients, timed the same way
        # another workload's step, same cold protocol: a long history with few samples
        "long_few_step": long_few,
        # the same step with bf16 h_history and h_s2 (fp32 arithmetic): not the headline
        "bf16_step": bf16_out,
        # not part of the step either: the blend path, fwd_blend + bwd_blend, cold rotation
        "blend_step": blend_out,
        # the backward with the input gradients (mamba2_scan_bwd_full) against
        # mamba2_scan_bwd followed by mamba2_scan_bwd_input
        "bwd_full": {"us": round(full_us, 2), "separate_us": round(sep_us, 2),
                     "algorithmic_bytes": per_kernel_bytes["bwd_full"],
                     "achieved": round(per_kernel_bytes["bwd_full"] / (full_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(per_kernel_bytes["bwd_full"] / (full_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "input_grads": {"kernel": "dinput_kernel", "us": round(kern_us["dinput_kernel"], 2), "bound": "hbm",
                        "achieved": round(per_kernel_bytes["dinput_kernel"] / (kern_us["dinput_kernel"] * 1e-6) / 1e9, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(per_kernel_bytes["dinput_kernel"] / (kern_us["dinput_kernel"] * 1e-6) / 1e9
                                      / HBM_PEAK_GBS, 4),
                        "traffic": (measured_traffic("dinput_kernel")
                                    if (args.workload, args.trunk) == ("pages_shape", "fp32") else None)},
        "parity": gate,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
