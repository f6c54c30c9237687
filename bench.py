"""Benchmark of the MoE expert-FFN layer on one MI355X.

Default workload: the GLM-5.2-shaped MoE layer at decode, T = 1 token
(H=6144, I=2048, 256 routed experts + 1 shared, sigmoid router top-8, int4
experts, Q8_0-style activations). A step is one pass of the whole hot path
for one batch through one layer: router logits + Q8(x), top-k + batch union,
gate/up IDOT + SwiGLU + Q8(h), down IDOT, combine with the shared expert.
Inputs (weights, tokens) are resident in HBM before timing starts.

The 256 MB Infinity Cache would hold one layer's 170 MB: steps therefore walk
round-robin over 16 independently seeded layer instances of that exact shape
(78 GB resident), so every step streams its experts from HBM as a real
multi-layer decode does. The steps are captured once in a HIP graph (16
steps, one per layer instance, 16 different token batches) and replayed.

Other workloads: glm52_mtp_verify_T4 (T=4), glm52_prefill_T512 (T=512, the
grouped int8-MFMA path), glm52_chain16_T1 (one token through 16 layers:
RMSNorm, then the layer with its output added to the residual stream; a step
is the whole 16-layer stack, restarted from the same input token), and
glm52_int8_mtp_T1 / glm52_int8_T4 (the same layer with int8 experts, the
MTP head's format, at T=1 and T=4), glm52_hot8_T512 (prefill with every
token on the same 8 experts: a compute-bound grouped GEMM, whose roofline
field is the int8 matrix-core rate), and glm52_dense_T1 / glm52_dense_T4
(the dense SwiGLU MLP of the first layers, int8, H 6144, I 12288).

Prints ONE JSON line (metric, value, roofline of the dominant kernel,
cpu_baseline of the oracle on a bounded sample).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published
# committed counter runs (HBM bytes per launch of the roofline kernel) and the
# sources that kernel is built from: a reading counts only while they are unchanged
TRAFFIC = {
    "glm52_decode_T1": ("decode_T1_glm52_traffic.json",
                        ["csrc/kernels_decode.hip", "csrc/gemv_device.hpp", "csrc/route_device.hpp",
                         "csrc/device_common.hpp", "csrc/internal.hpp", "build.py"]),
    "glm52_prefill_T512": ("prefill_T512_glm52_traffic.json",
                           ["csrc/kernels_grouped.hip", "csrc/device_common.hpp", "csrc/internal.hpp",
                            "build.py"]),
}



def kernel_source_hash(workload):
    import hashlib
    h = hashlib.sha256()
    for n in TRAFFIC[workload][1]:
        with open(os.path.join(ROOT, "int4_quantized_expert_sigmoid_amd", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the roofline kernel from the committed counter
    runs, or None when there are none for this workload or they were taken on
    other kernel sources."""
    if workload not in TRAFFIC:
        return None
    path = os.path.join(ROOT, "profiles", TRAFFIC[workload][0])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("workload") != workload or t.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return t.get("traffic_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4096)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="glm52_decode_T1")
    p.add_argument("--instances", type=int, default=16, help="resident layer instances (MALL defeat)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch every step eagerly")
    p.add_argument("--copy-probe", action="store_true",
                   help="after timing, copy a 1 GiB buffer once (a known-size kernel for HBM counter scaling)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu():
    """The host's CPU model and logical core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(spec, tokens_np, n_tokens=3, reps=3):
    """The oracle as it stands on a bounded sample, in both builds: n_tokens
    tokens through layer instance 0, each timed reps times (median), first on
    one thread (liboracle.so), then with its row loops on every host core
    (liboracle_omp.so, the same arithmetic). The threaded figure is the
    headline value; both are reported."""
    import numpy as np
    from oracle import layers as OL
    from oracle import oracle as O
    from synth import synth as S

    W, b = S.router(spec, 0, 0)
    cache = OL.ExpertCache(spec, 0, 0)
    for t in range(n_tokens):
        OL.forward_token(spec, cache, W, b, tokens_np[t])          # regenerate experts (untimed)

    def leg(threaded):
        O.use_threads(threaded)
        try:
            times = []
            for t in range(n_tokens):
                per = []
                for _ in range(reps):
                    t0 = time.perf_counter()
                    OL.forward_token(spec, cache, W, b, tokens_np[t])
                    per.append(time.perf_counter() - t0)
                times.append(sorted(per)[len(per) // 2])
            return float(np.mean(times)), O.threads()
        finally:
            O.use_threads(False)

    s1, _ = leg(False)
    sN, nthr = leg(True)
    model, nproc = host_cpu()
    sample = (f"{n_tokens} tokens through one layer of this shape, median of {reps} runs each; "
              f"C oracle, -O2; expert generation and packing untimed")
    return {"value": 1.0 / sN, "unit": "tokens*layers/s", "cores": nthr, "kind": "oracle",
            "sample": sample + f"; OpenMP build, {nthr} threads ({sN:.3f} s/token)",
            "single_thread": {"value": 1.0 / s1, "unit": "tokens*layers/s", "cores": 1,
                              "sample": sample + f"; plain build, one thread ({s1:.3f} s/token)"},
            "nproc": nproc, "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    from synth import synth as S0
    if args.workload in S0.DENSE_WORKLOADS:
        return bench_dense(args)

    import numpy as np
    import torch

    from int4_quantized_expert_sigmoid_amd import api, COLI_ACCUMULATE
    from int4_quantized_expert_sigmoid_amd._lib import lib
    from int4_quantized_expert_sigmoid_amd.synthetic import device_layer
    from synth import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = S.WORKLOADS[args.workload]
    spec, T = wl.layer, wl.tokens.T
    chain = wl.n_layers > 1
    decode = T <= 8                              # token-GEMV path; larger batches take the MFMA path
    n_inst = wl.n_layers if chain else args.instances
    log(f"bench: {args.workload} T={T}, building {n_inst} layer instances on device")
    t0 = time.time()
    scratch = torch.empty(spec.H * spec.I, dtype=torch.float32, device="cuda")
    layers = [device_layer(spec, wl.seed, li, scratch=scratch) for li in range(n_inst)]
    del scratch
    torch.cuda.synchronize()
    log(f"bench: layers ready in {time.time() - t0:.1f} s "
        f"({n_inst * spec.n_experts_stored * spec.expert_bytes / 1e9:.1f} GB of int{spec.weight_bits} experts resident)")

    ws = [api.workspace(L, T) for L in layers]
    cls = [L.c() for L in layers]
    stream = torch.cuda.Stream()
    from dataclasses import replace

    if chain:
        # one step = the token through all layers, restarted from the same input
        G = 1
        x0 = torch.from_numpy(S.tokens(wl.tokens, spec.H, wl.seed)).cuda()
        xr = torch.empty_like(x0)                 # residual stream
        gam = [torch.from_numpy(S.rms_gamma(spec.H, wl.seed, li)).cuda() for li in range(n_inst)]
        toks = x0.cpu().numpy()

        def step(i, s):
            with torch.cuda.stream(s):
                xr.copy_(x0)
            for l in range(n_inst):      # x <- x + MoE(RMSNorm(x) * gamma): the router launch takes the norm
                api.moe_forward_rms(layers[l], xr, gam[l], wl.rms_eps, ws[l], y=xr, flags=COLI_ACCUMULATE,
                                    stream=s, c_layer=cls[l])
        layer_calls = lambda i: [(l, xr, xr, COLI_ACCUMULATE) for l in range(n_inst)]
    else:
        G = n_inst                               # steps per captured graph: one per instance
        toks = S.tokens(replace(wl.tokens, T=T * G), spec.H, wl.seed)
        x_all = torch.from_numpy(toks).cuda().view(G, T, spec.H)
        y_all = torch.empty_like(x_all)

        def step(i, s):
            j = i % G
            api.moe_forward(layers[j], x_all[j], ws[j], y=y_all[j], stream=s, c_layer=cls[j])
        layer_calls = lambda i: [(i % G, x_all[i % G], y_all[i % G], 0)]

    # the distinct experts each layer call reads (from the routing of one eager step)
    for i in range(G):
        step(i, stream)
    stream.synchronize()
    union = []
    for j in range(n_inst):
        lay = api.workspace_layout(layers[j], T)
        idx = ws[j][lay.idx: lay.idx + 4 * T * spec.top_k].view(torch.int32).cpu().numpy()
        union.append(len(set(idx.tolist())))
    wb = spec.weight_bits                        # 4: two codes per byte; 8: one
    # codes + f32 scales per row: one per row, or one per group of columns
    ns_gu = spec.H // spec.group_size if spec.group_size else 1
    ns_dn = spec.I // spec.group_size if spec.group_size else 1
    gu_row, dn_row = 2 * spec.I * (spec.H * wb // 8 + 4 * ns_gu), spec.H * (spec.I * wb // 8 + 4 * ns_dn)
    bytes_call = [(u + spec.has_shared) * spec.expert_bytes for u in union]
    gateup_bytes = [(u + spec.has_shared) * gu_row for u in union]
    down_bytes = [(u + spec.has_shared) * dn_row for u in union]
    calls_per_step = n_inst if chain else 1

    # ---------------- timed region: exactly K steps after exactly W
    K, W = max(1, args.steps), max(0, args.warmup)
    use_graph = not args.no_graph
    if use_graph:
        # one graph of G steps (one per layer instance), replayed; a count
        # that is not a multiple of G ends with a graph of its first steps
        graphs = {}

        def graph_of(n):
            if n not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(n):
                        step(i, torch.cuda.current_stream())
                graphs[n] = g
            return graphs[n]

        for n in {G, K % G, W % G} - {0}:
            graph_of(n)

        def run(n):
            for _ in range(n // G):
                graphs[G].replay()
            if n % G:
                graphs[n % G].replay()
    else:
        def run(n):
            for i in range(n):
                step(i, stream)
    with torch.cuda.stream(stream):
        run(W)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        t_wall = time.perf_counter()
        run(K)
        ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / K
    value = K * T * calls_per_step / (ms_total / 1e3)   # tokens x layers per second

    # ---------------- per-kernel durations: eager layer calls on the same
    # inputs through coli_moe_forward_timed, every launch recording its own
    # start and stop (the kernel's timestamps, as a kernel-trace profiler
    # reads them), on the bench stream
    calls = []
    for i in (range(8) if chain else range(min(K, 256))):
        calls += layer_calls(i)
    evs = [api.KernelEvents(16) for _ in calls]
    for (j, xin, yout, fl), ev in zip(calls, evs):
        api.moe_forward_timed(layers[j], xin, ws[j], ev, y=yout, flags=fl, stream=stream, c_layer=cls[j],
                              gamma=gam[j] if chain else None, eps=wl.rms_eps)
    stream.synchronize()
    per_call = [ev.durations_ms() for ev in evs]
    label = lambda n: n.strip("()").split("<")[0]
    names = [label(n) for n, _ in per_call[0]]
    assert all([label(n) for n, _ in d] == names for d in per_call), "launch sequence varies between calls"
    stage_avg = np.array([[ms for _, ms in d] for d in per_call]).mean(axis=0)
    del evs
    STAGES = names
    i_gu = next(i for i, n in enumerate(names) if n in ("k_select_gateup", "k_gateup_mfma", "k_gateup_quad"))
    i_dn = next(i for i, n in enumerate(names) if n in ("k_down_combine", "k_down_gemv", "k_down_mfma", "k_down_quad"))
    gu_bytes_avg = float(np.mean([gateup_bytes[j] for (j, _, _, _) in calls]))
    dn_bytes_avg = float(np.mean([down_bytes[j] for (j, _, _, _) in calls]))
    gu_gbs = gu_bytes_avg / (stage_avg[i_gu] * 1e-3) / 1e9
    dn_gbs = dn_bytes_avg / (stage_avg[i_dn] * 1e-3) / 1e9
    step_bytes = float(np.sum(bytes_call)) if chain else float(np.mean(bytes_call))
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    # int8 work of the gate/up launch: every (token, expert) pair, shared included
    gu_ops = T * (spec.top_k + spec.has_shared) * 2 * 2 * spec.H * spec.I
    gu_tops = gu_ops / (stage_avg[i_gu] * 1e-3) / 1e12
    log("bench: kernel averages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in zip(STAGES, stage_avg)))
    log(f"bench: gate/up {gu_gbs:.0f} GB/s, down {dn_gbs:.0f} GB/s, whole step {step_gbs:.0f} GB/s "
        f"on int{wb} expert bytes; {ms_step * 1e3:.2f} us/step (graph={use_graph}), wall {t_wall:.3f} s")

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy probe {src.numel() * 4} B read, {dst.numel() * 4} B written"
            + (f"; kernel source hash {kernel_source_hash(args.workload)}" if args.workload in TRAFFIC else ""))
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on a CPU sample")
        cpu = cpu_baseline(spec, np.asarray(toks).reshape(-1, spec.H))

    # the gate/up kernel's bound: its int8 ops per algorithmic byte against
    # the ridge of the two peaks (about 625 ops/B)
    ai = gu_ops / gu_bytes_avg
    mfma_bound = ai > INT8_MFMA_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "kernel": STAGES[i_gu],
                "achieved": round(gu_tops if mfma_bound else gu_gbs, 1),
                "peak": INT8_MFMA_PEAK_TOPS if mfma_bound else HBM_PEAK_GBS,
                "unit": "TOP/s (int8)" if mfma_bound else "GB/s",
                "frac": round(gu_tops / INT8_MFMA_PEAK_TOPS if mfma_bound else gu_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if chain else measured_traffic(args.workload),
                "bytes_per_launch": gu_bytes_avg, "ops_per_launch": float(gu_ops), "ops_per_byte": round(ai, 1),
                "avg_launch_ms": round(float(stage_avg[i_gu]), 5),
                "hbm_gbs": round(gu_gbs, 1), "hbm_frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                "int8_tops": round(gu_tops, 1), "int8_mfma_frac": round(gu_tops / INT8_MFMA_PEAK_TOPS, 4)}
    phase = "16-layer decode chain" if chain else ("decode" if decode else "prefill")
    config = {"workload": args.workload, "H": spec.H, "I": spec.I, "E": spec.E, "top_k": spec.top_k,
              "shared_experts": spec.has_shared, "T": T, "layers_per_step": calls_per_step,
              "layer_instances": n_inst, "hip_graph": use_graph,
              "mean_union_experts": float(np.mean(union)),
              "expert_bytes_per_step": step_bytes,
              "step_hbm_gbs": round(step_gbs, 1),
              "kernel_ms": [[n, round(float(v), 5)] for n, v in zip(STAGES, stage_avg)]}
    if chain:
        config["stack_tokens_per_s"] = round(K * T / (ms_total / 1e3), 1)
    out = {
        "metric": f"MoE-layer tokens*layers/s (GLM-5.2-shaped layer, int{wb} experts, {phase})",
        "value": round(value, 1),
        "unit": "tokens*layers/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{wb}xint8->int32, f64 block sums",
        "data": "synthetic (seeded Philox weights and tokens, no trained checkpoint)",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_dense(args):
    """A dense layer of the first ones (the dense SwiGLU MLP) at decode: a step
    is one call of coli_dense_forward on one batch, walking resident
    instances round-robin as the MoE workloads do."""
    import numpy as np
    import torch

    from int4_quantized_expert_sigmoid_amd import api
    from int4_quantized_expert_sigmoid_amd.synthetic import device_dense
    from synth import synth as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = S.DENSE_WORKLOADS[args.workload]
    spec, T = wl.dense, wl.tokens.T
    G = args.instances
    log(f"bench: {args.workload} T={T}, building {G} dense MLP instances on device")
    scratch = torch.empty(spec.H * spec.I, dtype=torch.float32, device="cuda")
    mlps = [device_dense(spec, wl.seed, li, scratch=scratch) for li in range(G)]
    del scratch
    wss = [api.dense_workspace(M, T) for M in mlps]
    cms = [M.c() for M in mlps]
    from dataclasses import replace
    toks = S.tokens(replace(wl.tokens, T=T * G), spec.H, wl.seed)
    x_all = torch.from_numpy(toks).cuda().view(G, T, spec.H)
    y_all = torch.empty_like(x_all)
    stream = torch.cuda.Stream()

    def step(i, s):
        j = i % G
        api.dense_forward(mlps[j], x_all[j], wss[j], y=y_all[j], stream=s, c_mlp=cms[j])

    K, W = max(1, args.steps), max(0, args.warmup)
    graphs = {}
    for n in {G, K % G, W % G} - {0}:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                step(i, torch.cuda.current_stream())
        graphs[n] = g

    def run(n):                                   # exactly n steps
        for _ in range(n // G):
            graphs[G].replay()
        if n % G:
            graphs[n % G].replay()

    with torch.cuda.stream(stream):
        run(W)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        run(K)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / K
    value = K * T / (ms_total / 1e3)

    # kernel-exact durations of 256 eager calls
    per_call = []
    for i in range(min(K, 256)):
        ev = api.KernelEvents(4 + 2 * ((T + 7) // 8))   # rmsnorm/quant + gate/up and down per 8-token pass
        with api.kernel_timer(ev):
            step(i, stream)
        per_call.append(ev)
    stream.synchronize()
    durs = [ev.durations_ms() for ev in per_call]
    label = lambda n: n.strip("()").split("<")[0]
    names = [label(n) for n, _ in durs[0]]
    kms = np.array([[ms for _, ms in d] for d in durs]).mean(axis=0)
    del per_call
    wb = spec.weight_bits
    # every launch of a gate/up or down kernel reads its whole matrices: the
    # token-GEMV kernels (T <= 8) or the grouped MFMA kernels (larger T, one
    # expert holding every token)
    GU, DN = ("k_dense_gateup", "k_gateup_mfma", "k_gateup_quad"), ("k_dense_down", "k_down_mfma", "k_down_quad")
    k_gu = next(n for n in names if n in GU)
    ms_gu = float(np.mean([v for n, v in zip(names, kms) if n in GU]))
    ms_dn = float(np.mean([v for n, v in zip(names, kms) if n in DN]))
    passes = sum(1 for n in names if n in GU)
    gu_bytes = 2 * spec.I * (spec.H * wb // 8 + 4)
    dn_bytes = spec.H * (spec.I * wb // 8 + 4)
    gu_gbs = gu_bytes / (ms_gu * 1e-3) / 1e9
    dn_gbs = dn_bytes / (ms_dn * 1e-3) / 1e9
    step_bytes = passes * spec.nbytes
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log("bench: kernel averages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in zip(names, kms)))
    if passes > 1:
        log(f"bench: {passes} gate/up passes per step")
    log(f"bench: gate/up {gu_gbs:.0f} GB/s, down {dn_gbs:.0f} GB/s, whole step {step_gbs:.0f} GB/s; "
        f"{ms_step * 1e3:.2f} us/step")

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        log("bench: timing the oracle on a CPU sample")
        pack = O.pack_int8_rows if wb == 8 else O.pack_int4_rows
        w = []
        for m in (S.GATE, S.UP, S.DOWN):
            w.extend(pack(S.dense_matrix(spec, wl.seed, 0, m)))
        x = np.asarray(toks).reshape(-1, spec.H)[:3]

        def leg(threaded):
            O.use_threads(threaded)
            try:
                times = []
                for t in range(3):
                    t0 = time.perf_counter()
                    O.dense_forward(*w, x[t:t + 1])
                    times.append(time.perf_counter() - t0)
                return float(np.median(times)), O.threads()
            finally:
                O.use_threads(False)

        s1, _ = leg(False)
        sN, nthr = leg(True)
        model, nproc = host_cpu()
        sample = ("3 tokens through one dense MLP of this shape, median; C oracle, -O2; "
                  "weight generation and packing untimed")
        cpu = {"value": 1.0 / sN, "unit": "tokens*layers/s", "cores": nthr, "kind": "oracle",
               "sample": sample + f"; OpenMP build, {nthr} threads ({sN:.3f} s/token)",
               "single_thread": {"value": 1.0 / s1, "unit": "tokens*layers/s", "cores": 1,
                                 "sample": sample + f"; plain build, one thread ({s1:.3f} s/token)"},
               "nproc": nproc, "cpu_model": model}
    out = {
        "metric": f"dense-MLP tokens*layers/s (GLM-5.2-shaped first-layer MLP, int{wb} weights, "
                  f"{'decode' if T <= 8 else 'prefill chunk'})",
        "value": round(value, 1), "unit": "tokens*layers/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"int{wb}xint8->int32, f64 block sums",
        "data": "synthetic (seeded Philox weights and tokens, no trained checkpoint)",
        "config": {"workload": args.workload, "H": spec.H, "I": spec.I, "T": T, "layer_instances": G,
                   "hip_graph": True, "weight_bytes_per_step": step_bytes, "gemv_passes": passes,
                   "step_hbm_gbs": round(step_gbs, 1),
                   "kernel_ms": [[n, round(float(v), 5)] for n, v in zip(names, kms)]},
        "roofline": {"bound": "hbm", "kernel": k_gu, "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": gu_bytes, "avg_launch_ms": round(ms_gu, 5),
                     "down_gbs": round(dn_gbs, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
