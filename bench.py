"""MoE-layer forward benchmark on one MI355X.

One step = one pass of the whole layer (moe_layer: the router, the
permutation, moe_forward and moe_combine in one call; a single token is
routed inside the forward's first launch) over one batch of seeded
synthetic tokens, with all inputs already resident in HBM.  Decode workloads rotate over several
resident layers and a pool of activation batches so that neither the 256 MB
Infinity Cache nor L2 holds the expert weights between steps.

The rotation of steps is captured as one HIP graph of moe_layer calls (a
model captures its layers the same way), plus one graph per step for runs
that do not fill whole rotations, and replayed, so neither host launches
nor graph launches between steps enter the timing.

Prints ONE JSON line (the driver's contract).  The top level is the headline
workload (mid layer, T = 1 by default): `value` is MoE-layer tokens/s.
`roofline` reports the expert-FFN stage (moe_forward) against HBM bandwidth
(decode) or the bf16/fp16 MFMA peak (prefill), timed with HIP events on the
stream the kernels run on around replays of a graph of moe_forward calls.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
With the default workload, `additional_workloads` holds the same figures for
the 256-expert layer at T = 1 (HBM roof) and at T = 8192 with int4 weights
(MFMA roof), each timed the same way in the same run, then the residency
tier (decode from pinned host memory behind a per-layer HBM expert cache,
`--tiered`) and the sparse-attention indexer at decode and prefill
(`--index`).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2516.6  # dense bf16/fp16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz

# the workloads timed beside the headline one by default: (workload, T)
ADDITIONAL = (("large", 1), ("prefill_int4_uniform", 8192))
# workloads whose oracle is also timed on one thread (configs 0-2)
ONE_THREAD = (("tiny", 16), ("mid", 1), ("large", 1))


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mid", help="workload name (routed_expert_ffn_sigmoid_amd.synth.CONFIGS)")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default: first of the workload's T list)")
    ap.add_argument("--layers", type=int, default=None, help="resident layers rotated per step")
    ap.add_argument("--pool", type=int, default=None, help="activation batches rotated per step (16 decode, 2 prefill)")
    ap.add_argument("--path", default="auto", choices=["auto", "gemv", "gemm"])
    ap.add_argument("--invariant", action="store_true", help="the batch-shape-invariant mode (MOE_FLAG_BATCH_INVARIANT)")
    ap.add_argument("--router", default="sigmoid", choices=["sigmoid", "softmax", "expert-choice"],
                    help="router variant (expert choice runs the layer with one slot per expert, k = E)")
    ap.add_argument("--capacity-factor", type=float, default=0.0)
    ap.add_argument("--only", action="store_true", help="the named workload alone (no additional workloads)")
    ap.add_argument("--index", default=None, metavar="T,S",
                    help="time the sparse-attention indexer's top-2048 (dsa_index_topk) for T queries at the end of "
                         "an S-key cache (64 heads of 128) instead of the MoE layer")
    ap.add_argument("--tiered", action="store_true",
                    help="decode with the routed experts in pinned host memory behind a per-layer HBM cache")
    ap.add_argument("--slots", type=int, default=None,
                    help="HBM slots per layer (--tiered; default 4 k, at least a step's experts + the pinned ones)")
    ap.add_argument("--pinned", type=int, default=None, help="pinned hot experts per layer (--tiered; default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of each oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three plain 1 GiB device-to-device copies (torch copy_), whose HBM counter "
                         "readings scale the counters read for the MoE kernels")
    return ap.parse_args(argv)


def measured_traffic(config, T, gemm=False):
    """HBM bytes per moe_forward launch from the committed rocprofv3 counter summary of this workload
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is none or when the kernel sources
    have changed since the counters were taken."""
    kind = "gemm" if gemm else "decode"
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kind}_{config}_T{T}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        for key in ("source_sha256:", "traffic_bytes_per_launch:"):
            if line.startswith(key):
                vals[key[:-1]] = line[len(key):].strip()
    h = hashlib.sha256()
    for f in ("ffn_gemm.hip" if gemm else "ffn_decode.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "routed_expert_ffn_sigmoid_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sample_inputs(spec, T, n):
    """The first n tokens of the workload's first batch, with router and bias, and a host expert set in which only
    the experts those tokens hit (and the shared one) are generated: np.zeros leaves the other experts' pages
    untouched, and the oracle reads only the experts it applies."""
    from oracle import oracle as orc
    from routed_expert_ffn_sigmoid_amd import synth
    x = synth.gen_x(spec, T, 0, 0)[:n]
    W_r, bias = synth.gen_router(spec, 0, 0), synth.gen_bias(spec, 0, 0)
    r = orc.router_select(orc.router_logits(orc.decode_act(x, spec.act), W_r), bias, spec.k, spec.routed_scale)
    one = synth.stack_experts([synth.gen_expert(spec, 0)])
    routed = synth.QExpertSet(*[np.zeros((spec.E,) + getattr(one, f).shape[1:], getattr(one, f).dtype)
                                for f in ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down",
                                          "z_gate", "z_up", "z_down")])
    for e in sorted(set(int(v) for v in r.idx.ravel())):
        ex = synth.stack_experts([synth.gen_expert(spec, e)])
        for f in ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down"):
            getattr(routed, f)[e] = getattr(ex, f)[0]
    return x, W_r, bias, routed, synth.gen_shared_expert(spec)


def cpu_baseline(spec, T, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload: whole oracle layers (route, batch union,
    experts, shared expert, combine) over the first n tokens of its first batch.  Tokens are independent, so
    tokens/s of a sample is that of the workload (the oracle gains nothing from weight reuse)."""
    from oracle import oracle as orc
    n = min(T, 16)
    x, W_r, bias, routed, shared = _sample_inputs(spec, T, n)
    cores = orc.max_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.moe_layer(spec, x, W_r, bias, routed, shared)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    return {"value": round(reps * n / el, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} oracle layers of the first {n} tokens of the {spec.name} T={T} batch (layer 0), "
                      f"{el:.1f} s, fp64 C with OpenMP on {cores} threads"}


def one_thread_oracle():
    """The oracle on one host thread, one whole layer each of configs 0-2 (tiny T=16, mid T=1, large T=1)."""
    from oracle import oracle as orc
    from routed_expert_ffn_sigmoid_amd import synth
    out = {}
    cores = orc.max_threads()
    orc.set_threads(1)
    try:
        for name, T in ONE_THREAD:
            spec = synth.CONFIGS[name]
            x, W_r, bias, routed, shared = _sample_inputs(spec, T, T)
            t0 = time.perf_counter()
            orc.moe_layer(spec, x, W_r, bias, routed, shared)
            el = time.perf_counter() - t0
            out[f"{name}_T{T}"] = {"tokens_per_s": round(T / el, 3), "seconds": round(el, 3)}
    finally:
        orc.set_threads(cores)
    return out


def measure(spec, T, args, dev):
    """Time one workload; returns the figures of its JSON object (without the top-level contract fields)."""
    import torch
    from routed_expert_ffn_sigmoid_amd import binding as B
    from routed_expert_ffn_sigmoid_amd import layer as L
    from routed_expert_ffn_sigmoid_amd import synth

    decode = T * spec.k <= 4 * spec.E or T <= 64
    n_layers = args.layers or (4 if decode else 1)
    pool_n = args.pool or (16 if decode else 2)
    path = {"auto": B.MOE_PATH_AUTO, "gemv": B.MOE_PATH_GEMV, "gemm": B.MOE_PATH_GEMM}[args.path]
    flags = B.MOE_FLAG_BATCH_INVARIANT if args.invariant else 0
    router = {"sigmoid": B.MOE_ROUTER_SIGMOID_BIAS, "softmax": B.MOE_ROUTER_SOFTMAX,
              "expert-choice": B.MOE_ROUTER_EXPERT_CHOICE}[args.router]
    if router == B.MOE_ROUTER_EXPERT_CHOICE:
        spec = synth.small_spec(spec, k=spec.E)

    t_setup = time.perf_counter()
    layers = [L.DeviceLayerWeights(spec, 0, l, dev) for l in range(n_layers)]
    pool = [L.upload_x(spec, synth.gen_x(spec, T, 0, b), dev) for b in range(pool_n)]
    cycle = n_layers * pool_n // math.gcd(n_layers, pool_n)
    # one set of output/workspace buffers per step of the rotation, so each step can be a captured graph
    runs = [L.MoeRun(spec, T, dev, path, flags, router, args.capacity_factor) for _ in range(cycle)]
    setup_s = time.perf_counter() - t_setup

    def operands(i):
        return pool[i % pool_n], layers[i % n_layers]

    # eager pass over the rotation: realized unique experts per step
    n_uniq = np.zeros(cycle, dtype=np.int64)
    for i in range(cycle):
        x, W = operands(i)
        runs[i].run(x, W)
        n_uniq[i] = int(runs[i].n_uniq.item())
    torch.cuda.synchronize()

    # HIP graphs: one per step of the rotation (the moe_layer call), and one of a whole rotation of
    # moe_forward calls for the expert-FFN stage timing
    side = torch.cuda.Stream()
    step_graphs = []
    for i in range(cycle):
        g = torch.cuda.CUDAGraph()
        x, W = operands(i)
        with torch.cuda.graph(g, stream=side):
            runs[i].run(x, W)
        step_graphs.append(g)
    fwd_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(fwd_graph, stream=side):
        for i in range(cycle):
            x, W = operands(i)
            runs[i].forward(x, W)
    perm_graph = torch.cuda.CUDAGraph()  # the permutation alone (it rewrites the same outputs)
    with torch.cuda.graph(perm_graph, stream=side):
        for i in range(cycle):
            runs[i].permute()
    route_graph = torch.cuda.CUDAGraph()  # the router alone
    with torch.cuda.graph(route_graph, stream=side):
        for i in range(cycle):
            x, W = operands(i)
            runs[i].route(x, W)
    rp_graph = torch.cuda.CUDAGraph()  # router and permutation in one call
    with torch.cuda.graph(rp_graph, stream=side):
        for i in range(cycle):
            x, W = operands(i)
            runs[i].route_permute(x, W)
    torch.cuda.synchronize()

    # a whole rotation of steps in one graph, as a model captures its layers: no graph launch between steps
    rot_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rot_graph, stream=side):
        for i in range(cycle):
            x, W = operands(i)
            runs[i].run(x, W)
    torch.cuda.synchronize()

    def replay_steps(i0, n):
        """Steps i0 .. i0 + n - 1 of the rotation, in order: whole rotations where they start at step 0 of it,
        single-step graphs elsewhere."""
        i = i0
        while i < i0 + n:
            if i % cycle == 0 and i + cycle <= i0 + n:
                rot_graph.replay()
                i += cycle
            else:
                step_graphs[i % cycle].replay()
                i += 1

    replay_steps(0, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    replay_steps(args.warmup, args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # expert-FFN stage alone, timed with HIP events on the stream the kernels run on
    fwd_reps = max(1, (args.steps + cycle - 1) // cycle)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fwd_graph.replay()
    e0.record(stream)
    for _ in range(fwd_reps):
        fwd_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_s = e0.elapsed_time(e1) / 1e3
    n_fwd = fwd_reps * cycle
    fwd_us = fwd_s / n_fwd * 1e6
    perm_graph.replay()
    e0.record(stream)
    for _ in range(fwd_reps):
        perm_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    perm_us = e0.elapsed_time(e1) * 1e3 / n_fwd
    route_graph.replay()
    e0.record(stream)
    for _ in range(fwd_reps):
        route_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    route_us = e0.elapsed_time(e1) * 1e3 / n_fwd
    rp_graph.replay()
    e0.record(stream)
    for _ in range(fwd_reps):
        rp_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    rp_us = e0.elapsed_time(e1) * 1e3 / n_fwd

    # distribution of the step time: each step's graph replay between its own pair of events (a separate
    # pass after the timed one, so the events do not enter the reported throughput)
    n_dist = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for j in range(n_dist):
        evs[j][0].record(stream)
        step_graphs[(args.warmup + j) % cycle].replay()
        evs[j][1].record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in evs])

    ebytes = spec.expert_bytes()
    sbytes = spec.expert_bytes(spec.I_shared) if spec.I_shared else 0
    bytes_per_fwd = float(np.mean(n_uniq)) * ebytes + sbytes
    flops_per_step = 2.0 * 3 * spec.d * (T * spec.k * spec.I + T * spec.I_shared)
    # the roof that binds: HBM when the expert FFNs do fewer flops per expert-weight byte than the ridge
    # point of the two peaks (2516.6 TFLOP/s / 8 TB/s = 315 flop/B), the matrix cores otherwise
    ridge = PEAK_MFMA_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    # the auto path runs the matrix-core GEMM above B.MOE_AUTO_DECODE_MAX_T tokens (outside the invariant mode)
    gemm = args.path == "gemm" or (args.path == "auto" and not args.invariant and T > B.MOE_AUTO_DECODE_MAX_T)
    traffic = (None if args.invariant or args.path == "gemv" and T > B.MOE_AUTO_DECODE_MAX_T
               else measured_traffic(spec.name, T, gemm))
    if flops_per_step / bytes_per_fwd < ridge:
        achieved = bytes_per_fwd / (fwd_s / n_fwd) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "moe_forward (gate/up + down expert-FFN kernels)",
                "algorithmic_bytes_per_launch": round(bytes_per_fwd),
                "avg_launch_us": round(fwd_us, 2)}
    else:
        achieved = flops_per_step / (fwd_s / n_fwd) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "moe_forward (x to fp16, gate/up and down grouped-GEMM kernels)",
                "algorithmic_flops_per_launch": flops_per_step,
                "avg_launch_us": round(fwd_us, 2)}
    steps_idx = range(args.warmup, args.warmup + args.steps)
    res = {
        "value": round(T * args.steps / elapsed, 2),
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "dtype": ("bf16-act/" if spec.act == synth.ACT_BF16 else "f32-act/") + f"int{spec.wbits}-weights/f32-accum",
        "config": {"workload": f"{spec.name}: d={spec.d} E={spec.E} top-{spec.k} I={spec.I} "
                               f"shared={spec.I_shared} int{spec.wbits} T={T}",
                   "T": T, "layers_resident": n_layers, "x_pool": pool_n,
                   "mean_unique_experts": round(float(np.mean([n_uniq[i % cycle] for i in steps_idx])), 2),
                   "assignments_per_unique_expert": round(T * spec.k / float(np.mean(n_uniq)), 2),
                   "permute_us_alone": round(perm_us, 2), "route_us_alone": round(route_us, 2),
                   "route_permute_us_alone": round(rp_us, 2),
                   "router": args.router, "capacity_factor": args.capacity_factor,
                   "timing": f"HIP graphs of moe_layer calls: one per rotation of {cycle} steps (layers x "
                             f"activation batches), single-step graphs where a rotation does not fit, replayed",
                   "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
                   "path": args.path, "batch_invariant": bool(args.invariant), "setup_s": round(setup_s, 1)},
        "roofline": roof,
    }
    del runs, step_graphs, rot_graph, fwd_graph, perm_graph, route_graph, rp_graph, layers, pool
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


PEAK_MFMA_INT8_TOPS = 5033.2  # dense int8 MFMA, 256 CU x 8192 op/clk x 2.4 GHz


def measure_index(args, dev):
    """The indexer's scores and top-2048 for T queries at the end of an S-key cache: one call = both kernels."""
    import torch
    from routed_expert_ffn_sigmoid_amd import binding as B
    from routed_expert_ffn_sigmoid_amd import synth
    T, S = (int(v) for v in args.index.split(","))
    H, D, K = 64, 128, 2048
    pos0 = S - T
    pool = max(1, min(8, (1 << 30) // (S * D)))  # key caches rotated so the 256 MB Infinity Cache holds none
    inps = [synth.gen_index(T, S, H, D, seed=b) for b in range(pool)]
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    bufs = [(up(i.q), up(i.w), up(i.k), up(i.kscale)) for i in inps]
    shape = B.dsa_index_shape(T, S, H, D, K, pos0)
    ws = torch.empty(B.dsa_index_workspace_size(shape), dtype=torch.uint8, device=dev)
    top = torch.empty((T, K), dtype=torch.int32, device=dev)
    gap = torch.empty(T, dtype=torch.float64, device=dev)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for q, w, k, ks in bufs:
            B.dsa_index_topk(shape, q, w, k, ks, top, gap, ws)
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup // pool)):
        g.replay()
    reps = max(1, args.steps // pool)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * pool)
    visible = sum(min(S, pos0 + t + 1) for t in range(T))
    ops = 2.0 * visible * H * D
    nbytes = S * D + S * 4 + T * H * D + T * H * 4 + T * K * 4
    if ops / nbytes < PEAK_MFMA_INT8_TOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(ops / us / 1e6, 1), "peak": PEAK_MFMA_INT8_TOPS, "unit": "TOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof.update({"kernel": "dsa_index_topk (int8 scores, then the top 2048 by radix selection)",
                 "algorithmic_bytes_per_call": nbytes, "algorithmic_int8_ops_per_call": ops, "avg_call_us": round(us, 2)})
    return {"metric": "indexer queries/s", "value": round(T / us * 1e6, 2), "unit": "queries/s", "n_gpus": 1,
            "steps": reps * pool, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8-qk/f64-score", "data": "synthetic (seeded)",
            "config": {"workload": f"indexer top-{K}: T={T} queries at the end of S={S} keys, H={H}, D={D}",
                       "T": T, "S": S, "H": H, "D": D, "K": K, "key_caches_rotated": pool}, "roofline": roof}


PEAK_PCIE_GBS = 64.0  # the host link, PCIe 5.0 x16, one direction


def cache_hit_rates(spec, W, T, dev, xs, slot_counts, pinned, warm):
    """Hit rates of the device planner for each (policy, slots) over one token stream: the layer's router and
    permutation per step, then one plan per cache (no copies: the rates do not depend on them).  xs: [n*T][d];
    the first `warm` steps fill the caches and are not counted."""
    import torch
    from routed_expert_ffn_sigmoid_amd import binding as B
    from routed_expert_ffn_sigmoid_amd import layer as L
    run = L.MoeRun(spec, T, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    caches = []
    for policy in (B.MOE_CACHE_WEIGHTED_LRU, B.MOE_CACHE_LRU):
        for S in slot_counts:
            c = B.make_cache_shape(spec.E, S, len(pinned), policy)
            st = torch.empty(B.moe_cache_state_size(c), dtype=torch.uint8, device=dev)
            lists = [torch.empty(spec.E, **i32), torch.empty(1, **i32), torch.empty(spec.E, **i32),
                     torch.empty(1, **i32)]
            B.moe_cache_init(c, pinned, st, lists[2], lists[3])
            caches.append((policy, S, c, st, lists))
    n = xs.shape[0] // T
    base = {}
    for i in range(n):
        if i == warm:
            torch.cuda.synchronize()
            base = {(p, S): B.moe_cache_stats(c, st) for p, S, c, st, _ in caches}
        run.route(xs[i * T:(i + 1) * T], W)
        run.permute()
        for _, _, c, st, (h, nh, m, nm) in caches:
            B.moe_cache_plan(c, T, spec.k, run.uniq, run.n_uniq, st, h, nh, m, nm)
    torch.cuda.synchronize()
    out = {}
    for p, S, c, st, _ in caches:
        s1 = B.moe_cache_stats(c, st)
        s0 = base[(p, S)]
        hits, misses = s1[1] - s0[1], s1[2] - s0[2]
        out[f"{'weighted_lru' if p == B.MOE_CACHE_WEIGHTED_LRU else 'lru'}_slots{S}"] = round(hits / (hits + misses), 4)
    return out


def measure_tiered(args, dev):
    """Decode through the residency tier: every routed expert of each layer in pinned host memory, a weighted-LRU
    cache of HBM slots per layer in front of it.  One step = one layer call (route, permute, plan, the missed
    experts copied from host memory on a second stream while the resident ones compute, the missed ones, combine)
    for T fresh tokens, layers rotated."""
    import torch
    from routed_expert_ffn_sigmoid_amd import binding as B
    from routed_expert_ffn_sigmoid_amd import layer as L
    from routed_expert_ffn_sigmoid_amd import synth
    spec = synth.CONFIGS["large_zipf"]
    T = args.T or 1
    nl = args.layers or 2
    npin = 4 if args.pinned is None else args.pinned
    # four times the experts a token activates, and room for a whole step's misses
    slots = args.slots or max(4 * spec.k, min(spec.E, T * spec.k) + npin)
    t0 = time.time()
    copy_stream = torch.cuda.Stream()
    tiers, Ws, runs, tq = [], [], [], []
    for l in range(nl):
        tiers.append(L.HostTier(spec, layer=l))
        tq.append(tiers[-1].qffn())
        Ws.append(L.DeviceLayerWeights(spec, layer=l, device=dev, routed=False))
        pinned = synth.popularity_order(spec, layer=l)[:npin].tolist()
        runs.append(L.CachedMoeRun(spec, T, slots, pinned, device=dev, copy_stream=copy_stream))
        runs[-1].init(tiers[-1])
    setup_s = time.time() - t0
    steps, warm = args.steps, max(args.warmup, 8 * nl)
    xs = L.upload_x(spec, synth.gen_x(spec, (steps + warm) * T, 0, 1000), dev)  # a fresh token every step
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]

    def one(i, ev=None):
        l = i % nl
        runs[l].step(xs[i * T:(i + 1) * T], Ws[l], tiers[l], tq[l], ev)

    for i in range(warm):
        one(i)
    torch.cuda.synchronize()
    s0 = [r.stats() for r in runs]
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        one(warm + i, fev[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    s1 = [r.stats() for r in runs]
    hits = sum(b[1] - a[1] for a, b in zip(s0, s1))
    misses = sum(b[2] - a[2] for a, b in zip(s0, s1))
    eb = spec.expert_bytes()
    fetch_ms = sum(a.elapsed_time(b) for a, b in fev)
    fetched = misses * eb
    # the host link through the DMA engines (hipMemcpyAsync from the same pinned tier), for comparison
    dst = L.DeviceExperts(spec, 1, spec.I, dev)
    names = ("q_gate", "q_up", "q_down", "s_gate", "s_up", "s_down", "z_gate", "z_up", "z_down")
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 8
    c0.record(stream)
    for r in range(reps):
        for n in names:
            getattr(dst, n)[0].copy_(getattr(tiers[0], n)[5 + r], non_blocking=True)
    c1.record(stream)
    torch.cuda.synchronize()
    dma_gbs = reps * eb / (c0.elapsed_time(c1) * 1e6)
    # hit rates by policy and slot count on one stream of independent tokens and one of correlated tokens
    nrate, wrate = 2048, 512
    pin0 = synth.popularity_order(spec, layer=0)[:npin].tolist()
    sc = sorted({16, 2 * spec.k * T + npin, slots, 64, 128})
    sc = [S for S in sc if S - npin >= min(spec.E, T * spec.k)]
    x_iid = L.upload_x(spec, synth.gen_x(spec, nrate * T, 0, 2000), dev)
    x_ar = L.upload_x(spec, synth.gen_x_correlated(spec, nrate * T, 0.9, 0, 0), dev)
    rates = {"independent_tokens": cache_hit_rates(spec, Ws[0], T, dev, x_iid, sc, pin0, wrate),
             "correlated_tokens_rho0.9": cache_hit_rates(spec, Ws[0], T, dev, x_ar, sc, pin0, wrate)}
    achieved = fetched / (fetch_ms * 1e6) if fetch_ms > 0 else 0.0
    return {"metric": "MoE-layer tokens/s, routed experts in a host tier behind an HBM cache",
            "value": round(T / ms * 1e3, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int4-weights/bf16-act/f32-out", "data": "synthetic (seeded; random-init quantised weights)",
            "config": {"workload": f"256-expert top-8 int4 layer (d=7168, I=2048, shared 2048), Zipf(1.1) bias, "
                                   f"T={T} per step, {nl} layers rotated, every routed expert in pinned host memory",
                       "T": T, "slots_per_layer": slots, "pinned_per_layer": npin, "policy": "weighted LRU",
                       "setup_s": round(setup_s, 1)},
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "experts_fetched_per_step": round(misses / steps, 3),
            "roofline": {"bound": "pcie", "achieved": round(achieved, 2), "peak": PEAK_PCIE_GBS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_PCIE_GBS, 4), "traffic": None,
                         "kernel": "cache_fetch_kernel (missed experts, host tier -> HBM slots)",
                         "algorithmic_bytes_per_expert": eb, "fetch_ms_per_step": round(fetch_ms / steps, 4),
                         "dma_engine_gbs": round(dma_gbs, 2)},
            "hit_rates_by_policy": rates}


def index_cpu_baseline(sub, target_s):
    """The oracle's indexer (scores of every visible key, full sort) on queries of the same shape: the last query
    of the batch, repeated for about target_s."""
    from oracle import oracle as orc
    from routed_expert_ffn_sigmoid_amd import synth
    T, S = sub["config"]["T"], sub["config"]["S"]
    H, D, K = sub["config"]["H"], sub["config"]["D"], sub["config"]["K"]
    inp = synth.gen_index(1, S, H, D, seed=0)
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.index_topk(inp.q, inp.w, inp.k, inp.kscale, K, S - 1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    cores = orc.max_threads()
    return {"value": round(reps / el, 3), "unit": "queries/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} oracle calls of one query at the end of S={S} keys (H={H}, D={D}, K={K}), "
                      f"{el:.1f} s, fp64 C with OpenMP over queries (one query: one thread)"}


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.tiered:
        import torch
        from routed_expert_ffn_sigmoid_amd import binding as B
        B.lib()
        print(json.dumps(measure_tiered(args, torch.device("cuda:0"))), flush=True)
        return
    if args.index:
        import torch
        from routed_expert_ffn_sigmoid_amd import binding as B
        B.lib()
        print(json.dumps(measure_index(args, torch.device("cuda:0"))), flush=True)
        return
    import torch
    from routed_expert_ffn_sigmoid_amd import binding as B
    from routed_expert_ffn_sigmoid_amd import synth

    spec = synth.CONFIGS[args.config]
    T = args.T or synth.WORKLOAD_T[args.config][0]
    dev = torch.device("cuda:0")
    B.lib()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = measure(spec, T, args, dev)
    out = {
        "metric": "MoE-layer tokens/s",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; random-init quantised weights)",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    default_run = args.config == "mid" and args.T is None and not args.only and args.path == "auto" \
        and not args.invariant and args.layers is None and args.pool is None and args.router == "sigmoid" \
        and args.capacity_factor == 0
    extra = []
    if default_run:
        for name, Tw in ADDITIONAL:
            sub = measure(synth.CONFIGS[name], Tw, args, dev)
            sub = {"metric": "MoE-layer tokens/s", "unit": "tokens/s", "steps": args.steps, "warmup": args.warmup,
                   **sub}
            extra.append((name, Tw, sub))
        # the hot path's other rows: the residency tier (decode from a host tier behind the HBM cache) and the
        # sparse-attention indexer (decode and a prefill chunk)
        rows = [measure_tiered(argparse.Namespace(**{**vars(args), "T": 1, "layers": None}), dev)]
        for ix in ("1,32768", "512,16384"):
            rows.append(measure_index(argparse.Namespace(**{**vars(args), "index": ix}), dev))
        out["additional_workloads"] = [s for _, _, s in extra] + rows
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, T, args.cpu_seconds)
        for name, Tw, sub in extra:
            sub["cpu_baseline"] = cpu_baseline(synth.CONFIGS[name], Tw, args.cpu_seconds)
        if default_run:
            out["cpu_baseline"]["one_thread"] = one_thread_oracle()
            for sub in out["additional_workloads"]:
                if sub.get("metric") == "indexer queries/s":
                    sub["cpu_baseline"] = index_cpu_baseline(sub, args.cpu_seconds)
                elif sub.get("metric", "").startswith("MoE-layer tokens/s, routed experts in a host tier"):
                    # the oracle keeps every expert in host memory, the tier's own setting
                    sub["cpu_baseline"] = cpu_baseline(synth.CONFIGS["large_zipf"], sub["config"]["T"],
                                                       args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
