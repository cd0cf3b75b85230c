"""Throughput of the quantized expert FFN decode layer on one MI355X.

Default workload: routed MoE expert FFN decode layer with hidden 6144, 320
experts, intermediate 2048, top-8 routing, one token, int4-g64 gate/up/down,
bf16 activations.  One step = one moe_expert_ffn layer call (gate+up+SiLU,
down, weighted combine) over a fresh routing draw.  Routing draws walk
through random permutations of the 320 experts so that an expert's weights
are re-read only after all others (6.8 GB later), far past the 256 MB
last-level cache: every step streams its 8 experts from HBM.

Prints one JSON line:  value = algorithmic bytes per step (routed experts'
weights + scales, each read once, plus x and y) / time per step, in GB/s.
`roofline` reports the dominant kernel (fused gate+up+SiLU, about two thirds
of the bytes): its stage entry point is launched back to back over the same
routing draws, timed with HIP events recorded on the launch stream.  `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same steps.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s + µs/layer for int4-g64 MoE expert FFN decode (B=1)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--config", default="moe_large", choices=["moe_large", "moe_35b", "moe_prefill", "gemv", "qprep", "copy"],
                   help="copy: a plain 1 GiB device-to-device copy, the reference kernel for scaling the "
                        "FETCH_SIZE / WRITE_SIZE counters")
    p.add_argument("--tokens", type=int, default=1)
    p.add_argument("--shared", type=int, default=0,
                   help="moe configs: fold a shared expert into the routed group as one more slot (weight 1); "
                        "the value is the number of rotating copies of it (one per layer of a model)")
    p.add_argument("--batch", type=int, default=1, help="gemv: activations per weight read (qgemm_small when > 1)")
    p.add_argument("--gs", type=int, default=64, help="int4 group size (0 = per-row)")
    p.add_argument("--fmt", type=int, default=4, help="4 = int4, 1 = int8 per-row, 5 = int3-g64 two-plane "
                                                      "(gemv and the moe decode configs)")
    p.add_argument("--n", type=int, default=6144)
    p.add_argument("--pair", type=int, default=0,
                   help="gemv: rows of a second matrix of the same x and format, run with qgemv_pair "
                        "(one launch for both projections); also times the two as separate qgemv calls")
    p.add_argument("--k", type=int, default=6144)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--scales", default="unit", choices=["unit", "wide"],
                   help="expert weight scale draws: 'unit' gives unit-variance gate/up pre-activations (as a trained "
                        "model's normalised layers do), 'wide' the fixed U(0.005, 0.02) range of the tests")
    p.add_argument("--graph", action="store_true",
                   help="gemv / qprep: time the calls as one HIP graph replay (no per-call host launch cost) "
                        "instead of back-to-back launches from Python")
    return p.parse_args()


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def expert_bytes(fmt, H, I, gs):
    """Weights + scales of one expert (gate, up, down), as stored."""
    return 2 * I * row_bytes(fmt, H, gs) + H * row_bytes(fmt, I, gs)


def row_bytes(fmt, k, gs):
    """Weights + scales of one row of k inputs, as stored."""
    if fmt == 4:
        return k // 2 + 4 * (k // gs if gs else 1)
    if fmt == 5:  # int3-g64: 24 bytes + one scale per 64 inputs
        return (k + 63) // 64 * 28
    return k + 4


def counter_traffic(name, sources=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (profiles/<name>.txt: FETCH_SIZE and WRITE_SIZE per dispatch, each scaled
    by the factor a plain 1 GiB copy gives), or None when the summary is
    missing or was taken from other kernel sources than the ones built now
    (`sources`: the source files its digest covers; the decode kernels'
    by default)."""
    from int4_expert_gemv_amd import build as hipbuild
    sources = hipbuild.DECODE_SOURCES if sources is None else sources
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_digest") != hipbuild.source_digest(sources) or \
            "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def routing_schedule(seed, n_steps, T, E, k):
    """Per step: T tokens' top-k ids (distinct within a token) and softmax
    gate weights.  One token: a walk over random permutations of the experts
    (an expert comes back only after all others, so no step finds its weights
    in the last-level cache).  Several tokens: every token draws its k experts
    independently (uniformly, without replacement within the token), so
    tokens share experts as independent routing does (about 58.7 distinct
    experts of 320 for 8 tokens of top-8)."""
    g = np.random.default_rng([seed, 1234])
    if T == 1:
        need = n_steps * k
        perm = np.concatenate([g.permutation(E) for _ in range(need // E + 2)])
        ids = perm[:need].reshape(n_steps, 1, k).astype(np.int32)
    else:
        ids = np.stack([np.stack([g.choice(E, size=k, replace=False) for _ in range(T)])
                        for _ in range(n_steps)]).astype(np.int32)
    logits = g.standard_normal(size=(n_steps, T, k))
    w = np.exp(logits - logits.max(axis=2, keepdims=True))
    w = (w / w.sum(axis=2, keepdims=True)).astype(np.float32)
    return ids, w


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(o, run, units_per_call, unit_bytes, seconds, what):
    """The oracle as it stands, timed on the host: run(i) is one call over
    sample i (units_per_call of the metric's units each, unit_bytes bytes per
    unit); first with every host thread (OpenMP over rows), then on one
    thread, each for about `seconds` (at least one call)."""
    threads = len(os.sched_getaffinity(0))
    out = {}
    for label, nthr in (("multi", threads), ("single", 1)):
        o.set_threads(nthr)
        t0 = time.time()
        done = 0
        while done == 0 or (time.time() - t0) < seconds:
            run(done)
            done += 1
        el = time.time() - t0
        out[label] = (done, el, nthr)
    o.set_threads(threads)
    (dm, em, tm), (ds, es, _) = out["multi"], out["single"]
    gbs = lambda d, e: round(d * units_per_call * unit_bytes / e / 1e9, 4)
    return {"value": gbs(dm, em), "unit": "GB/s", "cores": tm, "kind": "oracle",
            "sample": "%s: %d calls on %d threads, %.2f ms per call" % (what, dm, tm, 1e3 * em / dm),
            "single_thread": {"value": gbs(ds, es), "unit": "GB/s", "cores": 1,
                              "sample": "%s: %d calls on 1 thread, %.2f ms per call" % (what, ds, 1e3 * es / ds)},
            "cpu_model": cpu_model()}


def stream_read_gbs():
    """A measured streaming-read rate of this GPU: torch's row sums over a
    2 GiB fp32 tensor viewed as 512 rows of 2^20 (the fastest plain read
    among torch's reductions here), best of 10; the denominator next to the
    published peak."""
    import torch
    a = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    rows = a.view(-1, 1 << 20)
    for _ in range(3):
        rows.sum(dim=1)
    torch.cuda.synchronize()
    best = None
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rows.sum(dim=1)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    nbytes = a.numel() * 4
    del a, rows
    return round(nbytes / (best * 1e-3) / 1e9, 1)


def stream_fields(achieved):
    sr = stream_read_gbs()
    return {"measured_stream_read_gbs": sr, "frac_of_measured_stream": round(achieved / sr, 4)}


def back_to_back_ms(launch, n):
    """Average time per launch(j), j < n, enqueued back to back between two
    events on the launch stream (torch's current stream): the kernel's own
    time plus the gap between consecutive kernels."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for j in range(n):
        launch(j)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def per_launch_ms(launch, n):
    """Average duration of launch(j), j < n, each bracketed by its own pair
    of events on the launch stream (torch's current stream): the kernel's
    own time plus the event granularity, without the gaps between calls."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for j in range(n):
        ev[j][0].record()
        launch(j)
        ev[j][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_moe(args, E, H, I):
    import torch
    from int4_expert_gemv_amd import qmoe, synth
    from oracle import ref

    T, k, fmt = args.tokens, 8, args.fmt
    gs = {1: 0, 5: 64}.get(fmt, args.gs)
    wname = {1: "int8-row", 5: "int3-g64"}.get(fmt, "int4-" + ("g%d" % gs if gs else "row"))
    nsh = max(0, args.shared)
    n_steps = args.warmup + args.steps
    print("generating %d experts (hidden %d, inter %d, %s)" % (E + nsh, H, I, wname), file=sys.stderr, flush=True)
    t0 = time.time()
    ex = synth.expert_set(args.seed, fmt, E + nsh, H, I, gs, threads=min(16, os.cpu_count() or 4), scales=args.scales)
    d = {key: dev(ex[key]) for key in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}
    torch.cuda.synchronize()
    print("generated+uploaded in %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)
    e = qmoe.experts(fmt, gs, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    ids_h, w_h = routing_schedule(args.seed, n_steps, T, E, k)
    if nsh:  # the shared expert (copy i % nsh at step i) as an always-on slot with weight 1
        sh_ids = (E + np.arange(n_steps) % nsh).astype(np.int32)
        ids_h = np.concatenate([ids_h, np.broadcast_to(sh_ids[:, None, None], (n_steps, T, 1))], axis=2)
        w_h = np.concatenate([w_h, np.ones((n_steps, T, 1), np.float32)], axis=2)
        k += 1
    x_h = synth.activations(np.random.default_rng([args.seed, 5]), (n_steps, T, H), "bf16")
    ids_d, w_d, x_d = dev(ids_h), dev(w_h), dev(x_h)
    ws = torch.empty(qmoe.moe_expert_ffn_workspace(e, T, k), dtype=torch.uint8, device="cuda")
    h = torch.empty((T * k, I), dtype=torch.float32, device="cuda")
    y = torch.empty((n_steps, T, H), dtype=torch.float32, device="cuda")

    def step(i):
        qmoe.moe_expert_ffn(e, x_d[i], ids_d[i], w_d[i], y[i], ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for j in range(args.steps):
        step(args.warmup + j)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps

    separate_us = None
    if nsh:  # the same layer with the shared expert as a second call, added by the caller
        y1 = torch.empty((T, H), dtype=torch.float32, device="cuda")
        y2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ids_r, w_r = ids_d[:, :, :k - 1].contiguous(), w_d[:, :, :k - 1].contiguous()
        ids_s, w_s = ids_d[:, :, k - 1:].contiguous(), w_d[:, :, k - 1:].contiguous()

        def sep(i):
            qmoe.moe_expert_ffn(e, x_d[i], ids_r[i], w_r[i], y1, ws)
            qmoe.moe_expert_ffn(e, x_d[i], ids_s[i], w_s[i], y2, ws)
            torch.add(y1, y2, out=y[i])

        for i in range(args.warmup):
            sep(i)
        torch.cuda.synchronize()
        start.record()
        for j in range(args.steps):
            sep(args.warmup + j)
        end.record()
        torch.cuda.synchronize()
        separate_us = start.elapsed_time(end) / args.steps * 1e3
        for j in range(n_steps):  # restore the folded results for the parity check below
            step(j)
        torch.cuda.synchronize()

    # dominant kernel: the fused gate+up+SiLU stage (one launch), over the
    # same routing draws, each launch bracketed by its own events
    gu_launch = lambda j: qmoe.moe_gate_up(e, x_d[args.warmup + j], ids_d[args.warmup + j], h, ws)
    gu_ms = back_to_back_ms(gu_launch, args.steps)
    gu_ms_bracketed = per_launch_ms(gu_launch, args.steps)

    # the two stage entry points on the last step, untimed (the layer call may
    # run them as one launch: then the two agree to fp32 rounding, not bit for bit)
    y2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    last = n_steps - 1
    qmoe.moe_gate_up(e, x_d[last], ids_d[last], h, ws)
    qmoe.moe_down(e, h, ids_d[last], w_d[last], y2, ws)
    torch.cuda.synchronize()
    same = bool(torch.equal(y2, y[last]))

    # parity of the last step (layer call and stage calls) against the oracle
    o = ref.oracle()
    yr, _, nr = o.moe_ffn(ex, x_h[last], ids_h[last], w_h[last])
    err = ref.max_norm_err(y[last].cpu().numpy(), yr, nr)
    err_stages = ref.max_norm_err(y2.cpu().numpy(), yr, nr)

    ebytes = expert_bytes(fmt, H, I, gs)
    uniq = [len(np.unique(ids_h[args.warmup + j])) for j in range(args.steps)]
    step_bytes = float(np.mean(uniq)) * ebytes + T * H * 2 + T * H * 4 + T * k * 8
    gu_bytes = float(np.mean(uniq)) * (2 * I * row_bytes(fmt, H, gs)) + T * H * 2
    value = step_bytes / (ms_step * 1e-3) / 1e9
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(o, lambda i: o.moe_ffn(ex, x_h[i % n_steps], ids_h[i % n_steps], w_h[i % n_steps],
                                                  want_norm=False),
                           1, step_bytes, args.cpu_seconds / 2, "the same decode steps (routing draws 0, 1, ...), "
                                                                 "fp64 oracle")

    gname = {1: "int8", 5: "int3"}.get(fmt, "g%d" % gs if gs else "row")
    tag = "%s_%s_t%d%s" % (args.config, gname, T, "_shared" if nsh else "")
    arith = ("bf16 dot products (v_dot2: weight codes as exact bf16, x as bf16 hi + lo where it is fp32), "
             "fp32 accumulation" if fmt == 5 else
             "integer dot products (int4 x int4 digits, int8 matrix instructions) into int32, combined in fp32")
    routing = "top-%d" % k
    if nsh:
        routing = ("top-%d + 1 shared expert folded in as an always-on slot with weight 1 (%d rotating copies)"
                   % (k - 1, nsh))
    return {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "us_per_layer": round(ms_step * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i32+f32",
        "data": "synthetic (seeded; weight scales '%s')" % args.scales,
        "config": {"workload": "moe_expert_ffn decode: hidden %d, %d experts, inter %d, %s, %d token(s)%s, "
                               "%s weights, bf16 x" % (H, E, I, routing, T,
                                                      " routed independently" if T > 1 else "", wname),
                   "tokens": T, "hidden": H, "experts": E, "inter": I, "top_k": k, "weights": wname,
                   "unique_experts_per_step": round(float(np.mean(uniq)), 2),
                   "bytes_per_step": int(step_bytes), "hbm_fraction_of_step": round(value / HBM_PEAK_GBS, 4),
                   "arithmetic": arith},
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("moe_gate_up_%s_counters" % tag),
                     "kernel": "fused gate+up+SiLU (moe_gate_up stage, one launch)",
                     "us_per_launch": round(gu_ms * 1e3, 3), "bytes_per_launch": int(gu_bytes),
                     "timing": "launches back to back between two HIP events on the launch stream",
                     "us_per_launch_bracketed": round(gu_ms_bracketed * 1e3, 3),
                     **stream_fields(gu_gbs)},
        "parity": {"max_norm_err": err, "tol": 2e-4, "stage_entry_points_max_norm_err": err_stages,
                   "stage_entry_points_identical": same},
        "cpu_baseline": cpu,
        **({"shared_expert": {"separate_call_us_per_layer": round(separate_us, 3),
                              "folded_us_per_layer": round(ms_step * 1e3, 3)}} if nsh else {}),
    }


def bench_prefill(args):
    """The expert-grouped prefill layer: 512 tokens, 256 experts, hidden 6144,
    inter 2048, top-8 with Zipf-skewed routing, int4-g64, bf16 x.  Each step
    uses one of 4 routing draws; every call streams the ~252 experts it
    touches (5.3 GB, far past the last-level cache)."""
    import torch
    from int4_expert_gemv_amd import build as hipbuild, qmoe, synth
    from oracle import ref

    T, E, H, I, k, gs, fmt = 512, 256, 6144, 2048, 8, 64, 4
    MFMA_PEAK = 2500.0  # dense bf16 TFLOP/s
    draws = 4
    g = np.random.default_rng([args.seed, 17])
    routes = [synth.zipf_routing(g, T, E, k) for _ in range(draws)]
    print("generating %d experts (hidden %d, inter %d, int4 gs=%d)" % (E, H, I, gs), file=sys.stderr, flush=True)
    ex = synth.expert_set(args.seed, fmt, E, H, I, gs, threads=min(16, os.cpu_count() or 4))
    d = {key: dev(ex[key]) for key in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")}
    e = qmoe.experts(fmt, gs, d["gate_q"], d["up_q"], d["down_q"], d["gate_s"], d["up_s"], d["down_s"])
    xs = [synth.activations(np.random.default_rng([args.seed, 18, i]), (T, H), "bf16") for i in range(draws)]
    x_d = [dev(x) for x in xs]
    ids_d = [dev(r[0]) for r in routes]
    w_d = [dev(r[1]) for r in routes]
    ws = torch.empty(qmoe.moe_expert_ffn_workspace(e, T, k), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def step(i):
        j = i % draws
        qmoe.moe_expert_ffn(e, x_d[j], ids_d[j], w_d[j], y, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    ebytes = expert_bytes(fmt, H, I, gs)
    touched = [len(np.unique(r[0])) for r in routes]
    per_step = [touched[i % draws] * ebytes + T * H * 2 + T * H * 4 + T * k * 8 for i in range(args.steps)]
    step_bytes = float(np.mean(per_step))
    flops = 2.0 * 3 * H * I * T * k
    gbs = step_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12

    # parity of a few tokens of the last draw (prefill precision: bf16 activations and hidden vector)
    j = (args.steps - 1) % draws
    step(args.steps - 1)
    torch.cuda.synchronize()
    pick = np.array([0, 1, T // 2, T - 1])
    yr, _, nr = ref.oracle().moe_ffn(ex, xs[j][pick], routes[j][0][pick], routes[j][1][pick], flags=ref.BF16_ACT)
    err = ref.max_norm_err(y.cpu().numpy()[pick], yr, nr)
    cpu = None
    if not args.no_cpu:
        # the oracle on 32 of the step's 512 tokens (a full step takes minutes
        # on the host), scaled to the step's bytes per token
        sub = np.arange(32) * (T // 32)
        o = ref.oracle()
        cpu = cpu_baseline(o, lambda i: o.moe_ffn(ex, xs[i % draws][sub], routes[i % draws][0][sub],
                                                  routes[i % draws][1][sub], flags=ref.BF16_ACT, want_norm=False),
                           32, step_bytes / T, args.cpu_seconds / 2,
                           "32 tokens (every 16th) of a prefill step, fp64 oracle; bytes counted as the step's "
                           "bytes per token")
    return {"metric": "achieved HBM GB/s + us/layer for int4-g64 MoE expert FFN prefill (512 tokens)",
            "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "us_per_layer": round(ms * 1e3, 2), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "moe_expert_ffn prefill: 512 tokens, hidden 6144, 256 experts, inter 2048, "
                                   "top-8 Zipf routing, int4-g64 weights, bf16 MFMA",
                       "experts_touched": touched, "bytes_per_step": int(step_bytes), "gflop_per_step": flops / 1e9},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": counter_traffic("moe_prefill_512tok_g64_counters", hipbuild.PREFILL_SOURCES),
                         "kernel": "whole prefill layer (5 kernels)",
                         "mfma_tflops": round(tflops, 2), "mfma_peak_tflops": MFMA_PEAK,
                         "mfma_utilisation": round(tflops / MFMA_PEAK, 4)},
            "parity": {"max_norm_err": err, "tol": 2e-4, "tokens_checked": pick.tolist()},
            "cpu_baseline": cpu}


def graph_ms(fn, steps):
    """ms per call of fn(0..steps-1) captured into one HIP graph and replayed
    (events on the replay stream around the second replay)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for j in range(steps):
            fn(j)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def bench_gemv(args):
    import torch
    from int4_expert_gemv_amd import qmoe, synth
    from oracle import ref

    fmt, n, k, B = args.fmt, args.n, args.k, args.batch
    gs = args.gs if fmt == 4 else (64 if fmt == 5 else 0)
    n2 = args.pair if B == 1 else 0

    def row_b(rows):
        if fmt == 5:  # int3-g64: 24 bytes + one fp32 scale per 64 inputs
            return rows * ((k + 63) // 64) * (24 + 4)
        return (rows * (k // 2 + 4 * (k // gs if gs else 1))) if fmt == 4 else rows * (k + 4)

    mb = row_b(n) + row_b(n2)
    copies = max(1, -(-(1 << 30) // mb))  # at least 1 GiB of distinct weights in rotation
    g = np.random.default_rng([args.seed, 77])
    qw, s = synth.quant_matrix(g, fmt, n, k, gs)
    mats = []
    for c in range(copies):
        mats.append(qmoe.qmat(fmt, dev(qw), dev(s), n, k, gs))
    if n2:
        qw2, s2 = synth.quant_matrix(np.random.default_rng([args.seed, 78]), fmt, n2, k, gs)
        mats2 = [qmoe.qmat(fmt, dev(qw2), dev(s2), n2, k, gs) for c in range(copies)]
        y2 = torch.empty((n2,), device="cuda")
    x_h = synth.activations(g, (B, k), "bf16")
    x = dev(x_h)
    y = torch.empty((B, n), device="cuda")

    def call(i):
        if n2:
            qmoe.qgemv_pair(mats[i], mats2[i], x[0], y[0], y2)
        elif B == 1:
            qmoe.qgemv(mats[i], x[0], y[0])
        else:
            qmoe.qgemm_small(mats[i], x, y)

    def call_separate(i):
        qmoe.qgemv(mats[i], x[0], y[0])
        qmoe.qgemv(mats2[i], x[0], y2)

    def timed(fn):
        for i in range(args.warmup):
            fn(i % copies)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.graph:
            return graph_ms(lambda j: fn(j % copies), args.steps)
        start.record()
        for j in range(args.steps):
            fn(j % copies)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    sep_ms = timed(call_separate) if n2 else None
    ms = timed(call)
    o = ref.oracle()
    err = 0.0
    yh = y.cpu().numpy()
    for b in range(B):
        yr, nr = o.gemv(fmt, n, k, gs, qw, s, x_h[b])
        err = max(err, ref.max_norm_err(yh[b], yr, nr))
    if n2:
        yr, nr = o.gemv(fmt, n2, k, gs, qw2, s2, x_h[0])
        err = max(err, ref.max_norm_err(y2.cpu().numpy(), yr, nr))
    byts = mb + B * k * 2 + B * (n + n2) * 4
    gbs = byts / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        def cpu_call(i):
            for b in range(B):
                o.gemv(fmt, n, k, gs, qw, s, x_h[b], want_norm=False)
            if n2:
                o.gemv(fmt, n2, k, gs, qw2, s2, x_h[0], want_norm=False)
        cpu = cpu_baseline(o, cpu_call, 1, byts, args.cpu_seconds / 2, "the same call, fp64 oracle")
    wname = ("int4-g%d" % gs if gs else "int4-row") if fmt == 4 else ("int3-g64" if fmt == 5 else "int8-row")
    return {"metric": "achieved HBM GB/s for quantized GEMV", "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "us_per_call": round(ms * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": ("qgemv_pair %dx%d + %dx%d" % (n, k, n2, k) if n2 else
                                    "%s %dx%d" % ("qgemv" if B == 1 else "qgemm_small", n, k)) +
                                   " %s, bf16 x, batch %d, %d weight copies in rotation" % (wname, B, copies),
                       "timing": "HIP graph replay" if args.graph else "back-to-back launches from Python"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "parity": {"max_norm_err": err, "tol": 2e-4}, "cpu_baseline": cpu,
            **({"separate_calls_us": round(sep_ms * 1e3, 3)} if n2 else {})}


def bench_qprep(args):
    """The q-prep chain: [W_a (6144 -> 2048) + W_kv (6144 -> 576)] x in one
    launch, RMS norm of the latent, W_b (2048 -> 16384), int4-g64, bf16 x;
    weight sets in rotation over >= 1 GiB.  Also times the same chain with
    the norm on the host (a synchronisation and two copies in the middle)."""
    import torch
    from int4_expert_gemv_amd import qmoe, synth
    from oracle import ref

    k, na, nkv, nq, gs = 6144, 2048, 576, 16384, 64
    row_b = lambda rows, kk: rows * (kk // 2 + 4 * (kk // gs))
    mb = row_b(na, k) + row_b(nkv, k) + row_b(nq, na)
    copies = max(1, -(-(1 << 30) // mb))
    g = np.random.default_rng([args.seed, 91])
    mats = []
    for tag, n, kk in ((1, na, k), (2, nkv, k), (3, nq, na)):
        qw, sc = synth.quant_matrix(np.random.default_rng([args.seed, 91, tag]), 4, n, kk, gs)
        mats.append(((4, n, kk, gs, qw, sc), [qmoe.qmat(4, dev(qw), dev(sc), n, kk, gs) for _ in range(copies)]))
    gw_h = (1.0 + 0.1 * g.standard_normal(na)).astype(np.float32)
    gw = dev(gw_h)
    eps = 1e-6
    x_h = synth.activations(g, (k,), "bf16")
    x = dev(x_h)
    u = torch.empty(na, device="cuda")
    kv = torch.empty(nkv, device="cuda")
    qo = torch.empty(nq, device="cuda")

    def chain(i):
        qmoe.qgemv_norm_chain(mats[0][1][i], mats[1][1][i], gw, eps, mats[2][1][i], x, u, kv, qo)

    def host_norm(i):
        qmoe.qgemv_pair(mats[0][1][i], mats[1][1][i], x, u, kv)
        uh = u.cpu().numpy()
        un = uh / np.sqrt(np.mean(uh * uh) + eps) * gw_h
        u.copy_(torch.from_numpy(un.astype(np.float32)))
        qmoe.qgemv(mats[2][1][i], u, qo)

    def timed(fn):
        for i in range(args.warmup):
            fn(i % copies)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.graph:
            return graph_ms(lambda j: fn(j % copies), args.steps)
        start.record()
        for j in range(args.steps):
            fn(j % copies)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    g_flag, args.graph = args.graph, False
    host_ms = timed(host_norm)  # synchronises with the host on every call: never captured
    args.graph = g_flag
    ms = timed(chain)
    o = ref.oracle()
    ur, _ = o.gemv(*mats[0][0], x_h)
    un = o.rmsnorm(ur, gw_h, eps)
    yq, nrq = o.gemv(*mats[2][0], un)
    yk, nrk = o.gemv(*mats[1][0], x_h)
    err = max(ref.max_norm_err(qo.cpu().numpy(), yq, nrq), ref.max_norm_err(kv.cpu().numpy(), yk, nrk))
    byts = mb + k * 2 + (na + nkv + nq) * 4 + na * 4
    gbs = byts / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        def cpu_call(i):
            u0, _ = o.gemv(*mats[0][0], x_h, want_norm=False)
            o.gemv(*mats[1][0], x_h, want_norm=False)
            o.gemv(*mats[2][0], o.rmsnorm(u0, gw_h, eps), want_norm=False)
        cpu = cpu_baseline(o, cpu_call, 1, byts, args.cpu_seconds / 2, "the same chain, fp64 oracle")
    return {"metric": "achieved HBM GB/s for the q-prep chain (pair GEMV, RMS norm, GEMV)", "value": round(gbs, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "us_per_call": round(ms * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "qgemv_norm_chain: %d -> (%d, %d), rmsnorm, %d -> %d, int4-g64, bf16 x, "
                                   "%d weight sets in rotation" % (k, na, nkv, na, nq, copies),
                       "timing": "HIP graph replay" if args.graph else "back-to-back launches from Python"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "parity": {"max_norm_err": err, "tol": 2e-4}, "cpu_baseline": cpu,
            "norm_on_host_us": round(host_ms * 1e3, 3)}


def bench_copy(args):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    return {"metric": "device copy bandwidth (read + write)", "value": round(2 * n / (ms * 1e-3) / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "1 GiB device-to-device copy"}}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in the design "
              "notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.config == "moe_large":
        out = bench_moe(args, 320, 6144, 2048)
    elif args.config == "moe_35b":
        out = bench_moe(args, 256, 2048, 512)
    elif args.config == "moe_prefill":
        out = bench_prefill(args)
    elif args.config == "qprep":
        out = bench_qprep(args)
    elif args.config == "copy":
        out = bench_copy(args)
    else:
        out = bench_gemv(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
