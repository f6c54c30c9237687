"""Per-workgroup timeline of the three-launch decode layer (T <= 8).

Loads the profiling build of the library (`python -m
int4_quantized_expert_sigmoid_amd.build --trace`, _trace/libcoli_moe.so:
the same sources with COLI_TRACE), installs a device buffer for its stamps,
runs one layer call per repetition on seeded synthetic layers of a named
workload, and prints, for each phase, the spread of the workgroups' stamps
in us from the router launch's first workgroup:

  router:        start, end
  gate/up:       shared-expert workgroups' start and end; routed workgroups'
                 start, end of selection and union, end; the selection steps
                 (keys in and groups scored, keys ordered, k rounds, union)
  down+combine:  start, end of the streamed rows, end (the T <= 2 form)

The stamps are the 100 MHz real-time counter read by the first lane of
each workgroup (10 ns resolution).

    python -m int4_quantized_expert_sigmoid_amd.trace_decode [workload] [--dump FILE.npz]

--dump also writes the raw stamps of every call (launch stamps [call][3][4096][4]
and selection marks [call][4096][8], 100 MHz ticks) for offline analysis.
"""
import ctypes
import os
import sys

import numpy as np
import torch

from . import _lib, build

REPS = 8          # traced calls
N_LAYERS = 4      # distinct layers, walked in turn so no call finds its weights in the MALL
TRACE_WG = 4096   # stamp slots per launch


def main(argv):
    from dataclasses import replace
    from synth import synth as S
    from .synthetic import device_layer
    from . import api

    if not os.path.exists(build.TRACE_LIB):
        raise SystemExit(f"{build.TRACE_LIB} is not built: run python -m int4_quantized_expert_sigmoid_amd.build --trace")
    _lib.LIB_PATH = build.TRACE_LIB
    L = _lib.lib()
    L.coli_trace_decode_set.argtypes = [ctypes.c_void_p]
    dump = None
    if "--dump" in argv:
        i = argv.index("--dump")
        dump = argv[i + 1]
        argv = argv[:i] + argv[i + 2:]
    name = argv[0] if argv else "glm52_decode_T1"
    wl = S.WORKLOADS[name]
    spec, T = wl.layer, wl.tokens.T
    if T > 8:
        raise SystemExit("the decode launches serve T <= 8")
    torch.cuda.set_device(0)
    layers = [device_layer(spec, 0, i) for i in range(N_LAYERS)]
    toks = torch.from_numpy(S.tokens(replace(wl.tokens, T=T * N_LAYERS), spec.H, 0)).cuda().view(N_LAYERS, T, spec.H)
    ws = [api.workspace(Lr, T) for Lr in layers]
    stamps = torch.zeros(3 * TRACE_WG * 4 + TRACE_WG * 8, dtype=torch.int64, device="cuda")
    y = torch.empty_like(toks[0])

    def call(i):
        api.moe_forward(layers[i % N_LAYERS], toks[i % N_LAYERS], ws[i % N_LAYERS], y=y)

    for i in range(2 * N_LAYERS):
        call(i)
    torch.cuda.synchronize()
    res = []
    for rep in range(REPS):
        stamps.zero_()
        torch.cuda.synchronize()
        L.coli_trace_decode_set(ctypes.c_void_p(stamps.data_ptr()))
        call(rep)
        torch.cuda.synchronize()
        L.coli_trace_decode_set(None)
        for j in range(1, N_LAYERS):
            call(rep + j)
        torch.cuda.synchronize()
        a = stamps.cpu().numpy()
        res.append((a[:3 * TRACE_WG * 4].reshape(3, TRACE_WG, 4).copy(), a[3 * TRACE_WG * 4:].reshape(TRACE_WG, 8).copy()))

    if dump:
        np.savez_compressed(dump, launches=np.stack([r[0] for r in res]), marks=np.stack([r[1] for r in res]))
    E, I, H = spec.E, spec.I, spec.H
    nrb = I // 32
    nsh = nrb if spec.has_shared else 0
    n_gu = nsh + T * spec.top_k * nrb          # grid of the gate/up launch
    n_dn = H // 8 if T <= 1 else H // 4        # grid of the down + combine launch (T <= 2)
    phases = {}

    def put(k, v):
        phases.setdefault(k, []).append(np.asarray(v, float))

    for launches, marks in res:
        r0 = launches[0, :E, 0]
        t0 = r0[r0 > 0].min()
        us = lambda a: np.where(a > 0, (a - t0) * 0.01, np.nan)
        put("router start", us(launches[0, :E, 0]))
        put("router end", us(launches[0, :E, 2]))
        put("shared GU start", us(launches[1, :nsh, 0]))
        put("shared GU end", us(launches[1, :nsh, 2]))
        rg = slice(nsh, n_gu)
        put("routed GU start", us(launches[1, rg, 0]))
        put("routed GU routed", us(launches[1, rg, 1]))
        put("routed GU end", us(launches[1, rg, 2]))
        for m, lab in ((0, "sel keys issued"), (1, "sel ordered"), (2, "sel rounds"), (4, "sel union")):
            put("  " + lab, us(marks[rg, m]))
        if T <= 2:
            put("down start", us(launches[2, :n_dn, 0]))
            put("down streamed", us(launches[2, :n_dn, 1]))
            put("down end", us(launches[2, :n_dn, 2]))

    def spread(v):
        v = v[np.isfinite(v)]
        if len(v) == 0:
            return "   -  "
        return f"min {v.min():6.2f} p50 {np.median(v):6.2f} p90 {np.percentile(v, 90):6.2f} max {v.max():6.2f}"

    print(f"{name}: per-workgroup timestamps, us from the router launch's first workgroup, {REPS} calls pooled")
    for k, v in phases.items():
        print(f"{k:18s}", spread(np.concatenate(v)))
    print("per-call medians:")
    for k, v in phases.items():
        ok = [x[np.isfinite(x)] for x in v if np.isfinite(x).any()]
        if ok:
            print(f"{k:18s} {np.median([np.median(x) for x in ok]):6.2f}  "
                  f"(last of call, median {np.median([x.max() for x in ok]):6.2f})")


if __name__ == "__main__":
    main(sys.argv[1:])
