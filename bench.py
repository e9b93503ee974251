#!/usr/bin/env python3
"""DeepSeekMoE layer forward on one MI355X: tokens/s and expert-GEMM TFLOP/s.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 16b]

A step is one moe_forward (router, dispatch, routed gate/up and down grouped
GEMMs, shared experts, combine) over one batch of seeded synthetic inputs
that are resident in HBM before timing starts.  By default the expert
weights are converted once to the packed layout (moe_pack_weights) before
timing, as a server would at load time; --weights row_major times the plain
layout, and the JSON line carries the other layout's time beside it.  The timed steps run through
moe_forward_timed with a HIP event pair for the gate/up kernel only, bound
to its launch on the launch stream (the kernel's own start and end); the
per-stage breakdown comes from a few further steps with every marker set,
outside the timed region.

Warm-up runs at least --warmup steps and keeps going until WARMUP_MIN_S of
back-to-back steps have passed: from an idle GPU the step time falls for
the first 25-50 ms of sustained load (2b-shaped layer 0.67 -> 0.55 ms, 16B
2.73 -> 2.30 ms, measured step by step) as the clocks come up, and a few
steps do not cover that.  The JSON line gives the count actually run.

Prints one JSON line.  `roofline` is for the dominant kernel, the gate/up
grouped GEMM, whose launch does 4*R*d*I FLOPs (R = T*K' routed rows, plus
K_s*T rows when the shared experts of the routed width ride in the same
launch) and must move, at the least, the W1/W3 rows of every expert it
uses, the x rows it reads and the R*I outputs it writes.  Above the ridge
point (peak FLOP/s over peak bytes/s) it is priced against the bf16 dense
MFMA peak, below it against HBM bandwidth.  `expert_gemm_tflops` counts all expert FLOPs (routed 6*T*K'*d*I
and shared 6*T*d*K_s*I_s) over the four GEMM stages.  `cpu_baseline` times
the fp64 oracle on the first --cpu-tokens tokens of the same workload on
the host cores, repeated until CPU_MIN_S of wall time have passed.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
WARMUP_MIN_S = 0.2            # least back-to-back warm-up before timing
CPU_MIN_S = 10.0              # least wall time of the oracle runs behind cpu_baseline

# HBM bytes per launch of the routed gate/up kernel, by (layer, weight layout),
# from rocprofv3 FETCH_SIZE (x2) and WRITE_SIZE (x1) in KiB, the factors taken
# from a plain 1 GiB copy in the same run
# (profiles/grouped_gemm_gate_up_16b_fetch_write.md).  None whenever the
# kernel has changed since the counters were taken.
TRAFFIC_BYTES = {("16b", "packed"): (1751334 * 2 + 360448) * 1024,
                 ("16b", "row_major"): (1751347 * 2 + 360450) * 1024}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="16b", help="layer shape from synth.configs")
    ap.add_argument("--weights", choices=("packed", "row_major"), default="packed",
                    help="expert weight layout the timed forward reads (packed: converted once by "
                         "moe_pack_weights before timing, like loading a checkpoint)")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the workload the oracle is timed on (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    return ap.parse_args()


def hip_runtime():
    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


def upload(a, device):
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def cpu_baseline(cfg, inputs, n_tokens):
    """The fp64 oracle, as it stands, on the first n_tokens tokens of the workload,
    run again until CPU_MIN_S of wall time have passed."""
    import oracle
    from threadpoolctl import threadpool_info
    n = min(n_tokens, cfg.tokens)
    sub = dict(inputs)
    sub["x"] = inputs["x"][:n]
    c = cfg.with_(tokens=n)
    runs, t0, c0 = 0, time.perf_counter(), time.process_time()
    while True:
        oracle.forward(c, sub)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_MIN_S:
            break
    cpu = time.process_time() - c0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": runs * n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.tokens} tokens of the same layer, fp64 numpy "
                      f"(routing + dispatch + all chosen experts + shared + combine), "
                      f"{runs} runs, {dt:.1f} s wall, {cpu:.1f} s CPU"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is run and timed on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_43_amd import _lib, ops
    from synth import get_config, make_inputs

    cfg = get_config(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    inputs = make_inputs(cfg)
    d = {k: upload(v, dev) for k, v in inputs.items()}
    torch.cuda.synchronize()
    print(f"[bench] inputs for {cfg.name} ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    lay_rm = ops.Layer.of(cfg)
    weight_keys = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
    packable = cfg.dtype == "bf16" and all(v % 128 == 0 for v in (cfg.d_model, cfg.d_ff, cfg.d_ff_shared))
    layout = args.weights if packable else "row_major"
    rm_args = [d["x"], d["w_router"], d["bias"], *[d[k] for k in weight_keys]]
    if layout == "packed":
        lay = dataclasses.replace(lay_rm, weight_layout="packed")
        pk = {k: ops.pack_weights(lay_rm, d[k]) for k in weight_keys}
        call_args = [d["x"], d["w_router"], d["bias"], *[pk[k] for k in weight_keys]]
    else:
        lay = lay_rm
        call_args = rm_args
    fwd = ops.Forward(lay, cfg.tokens, dev)
    fwd.check(*call_args, None)

    warmup_run, t_w = 0, time.perf_counter()
    while warmup_run < args.warmup or time.perf_counter() - t_w < WARMUP_MIN_S:
        for _ in range(max(1, args.warmup)):
            fwd(*call_args, checked=True)
        warmup_run += max(1, args.warmup)
        torch.cuda.synchronize()

    hip = hip_runtime()
    nev = 2 * _lib.MOE_NUM_STAGES
    gu_stage = _lib.STAGES.index("routed_gate_up")
    created = []

    def markers(stages):
        """Event array for moe_forward_timed with handles for `stages` only."""
        arr = (ctypes.c_void_p * nev)()
        for st_i in stages:
            for i in (2 * st_i, 2 * st_i + 1):
                ev = ctypes.c_void_p()
                assert hip.hipEventCreate(ctypes.byref(ev)) == 0
                arr[i] = ev.value
                created.append(ev.value)
        return arr

    def elapsed(arr, st_i):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), arr[2 * st_i], arr[2 * st_i + 1]) == 0
        return f.value

    p = ops._p
    lib = _lib.lib()
    c_layer = lay.c()
    stream = ops._stream()

    def step(arr):
        _lib.check("moe_forward_timed", lib.moe_forward_timed(
            ctypes.byref(c_layer), cfg.tokens, *[p(a) for a in call_args], None, p(fwd.y),
            p(fwd.topk_idx), p(fwd.topk_w), p(fwd.counts),
            p(fwd.offsets), p(fwd.ws), fwd.ws.numel(), stream, arr))

    # Timed region: whole-layer steps; HIP events mark only the gate/up kernel.
    timed = [markers([gu_stage]) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(timed[k])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    gu_ms = float(np.mean([elapsed(arr, gu_stage) for arr in timed]))

    # Per-stage breakdown from separate steps after the timed region (every
    # marker costs a few microseconds of GPU time, so they stay out of it).
    n_brk = max(3, min(args.steps, 10))
    brk = [markers(range(_lib.MOE_NUM_STAGES)) for _ in range(n_brk)]
    for arr in brk:
        step(arr)
    torch.cuda.synchronize()
    stage_ms = np.array([[elapsed(arr, st_i) for st_i in range(_lib.MOE_NUM_STAGES)] for arr in brk])
    for ev in created:
        hip.hipEventDestroy(ev)
    st = dict(zip(_lib.STAGES, stage_ms.mean(0).round(5).tolist()))

    # Routing statistics (moe_route_stats) next to the plain router on the
    # same batch, outside the timed region: the cost of the statistics.
    def per_call_ms(fn, n=20):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n_dev = 8 if cfg.n_routed % 8 == 0 else 1
    s_idx, s_w, s_stats, s_lse = ops.route_stats(lay, d["x"], d["w_router"], d["bias"], n_dev, lse=True,
                                                 ws=fwd.ws)

    def route_plain():
        _lib.check("moe_route", lib.moe_route(ctypes.byref(c_layer), cfg.tokens, p(d["x"]),
                                              p(d["w_router"]), p(d["bias"]), p(s_idx), p(s_w), stream))

    def route_with_stats():
        _lib.check("moe_route_stats", lib.moe_route_stats(
            ctypes.byref(c_layer), cfg.tokens, p(d["x"]), p(d["w_router"]), p(d["bias"]), n_dev,
            p(s_idx), p(s_w), p(s_stats), p(s_lse), p(fwd.ws), fwd.ws.numel(), stream))

    route_ms = per_call_ms(route_plain)
    route_stats_ms = per_call_ms(route_with_stats)

    # The other weight layout on the same batch (row-major when the timed
    # forward reads packed weights).
    other = "row_major" if layout == "packed" else ("packed" if packable else None)
    other_ms = None
    if other is not None:
        lay_o = dataclasses.replace(lay_rm, weight_layout=other)
        o_args = rm_args if other == "row_major" else \
            [d["x"], d["w_router"], d["bias"], *[ops.pack_weights(lay_rm, d[k]) for k in weight_keys]]
        fo = ops.Forward(lay_o, cfg.tokens, dev)
        other_ms = per_call_ms(lambda: fo(*o_args, checked=True), n=max(3, min(args.steps, 10)))
        del fo, o_args
        torch.cuda.empty_cache()

    # Expert capacity (Switch/GShard, one group of the whole batch): the same
    # layer with C = ceil(factor * T * K' / N_r) slots per expert.
    capacity = {}
    for factor in (1.0, 1.25):
        C = -(-int(factor * 100) * cfg.tokens * cfg.top_k // (100 * cfg.n_routed))
        fc = ops.Forward(dataclasses.replace(lay, capacity=C), cfg.tokens, dev)
        ms_c = per_call_ms(lambda: fc(*call_args, checked=True), n=max(3, min(args.steps, 10)))
        capacity[str(factor)] = {"capacity": C, "ms_per_step": ms_c,
                                 "kept_frac": int(fc.counts.sum()) / (cfg.tokens * cfg.top_k)}
        del fc
        torch.cuda.empty_cache()

    T, dm, I, K = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.top_k
    P = T * K
    # With I_s == I the shared experts run as K_s extra groups of T rows in
    # the routed gate/up and down launches (moe_forward's documented rule).
    fold = cfg.n_shared > 0 and cfg.d_ff_shared == I
    rows = P + (T * cfg.n_shared if fold else 0)
    gu_flop = 4.0 * rows * dm * I            # one launch of the gate/up kernel
    routed_flop = 6.0 * P * dm * I
    sh_flop = 6.0 * T * dm * cfg.n_shared * cfg.d_ff_shared
    router_flop = 2.0 * T * dm * cfg.n_routed
    expert_ms = st["routed_gate_up"] + st["routed_down"]
    if not fold:
        expert_ms += st["shared_gate_up"] + st["shared_down"]
    gu_tflops = gu_flop / (gu_ms * 1e-3) / 1e12
    # Least bytes the gate/up launch moves: W1 and W3 rows of the experts it
    # uses (all of them at these batch sizes), x once, and the R x I outputs.
    n_w = cfg.n_routed + (cfg.n_shared if fold else 0)
    gu_bytes = 2.0 * (2 * n_w * I * dm + T * dm + rows * I)
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    mfma_bound = gu_flop / gu_bytes >= (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
    expert_tflops = (routed_flop + sh_flop) / (expert_ms * 1e-3) / 1e12
    layer_tflops = (routed_flop + sh_flop + router_flop) / (ms * 1e-3) / 1e12

    # Whole-layer HBM view (the decode-shaped layer is bound by it): the
    # least bytes a forward moves are the weights of every expert it uses,
    # the router weights, x and y.
    touched = int((fwd.counts.cpu().numpy() > 0).sum())
    esz = 2 if cfg.dtype == "bf16" else 4
    layer_bytes = (3.0 * esz * dm * (touched * I + cfg.n_shared * cfg.d_ff_shared)
                   + 4.0 * cfg.n_routed * dm + 2.0 * esz * T * dm)
    layer_gbs = layer_bytes / (ms * 1e-3) / 1e9

    # The small memory-bound stages against HBM: their own algorithmic bytes
    # over their event-timed stage time.
    # rows the combine reads: routed, plus K_s folded shared rows or one y_shared row per token
    R = P + (T * cfg.n_shared if fold else (T if cfg.n_shared > 0 else 0))
    stage_bytes = {
        "route": esz * T * dm + 4.0 * cfg.n_routed * dm + 8.0 * P,        # x, W_g, idx + weights
        "dispatch": 4.0 * P + 8.0 * P + 8.0 * cfg.n_routed,              # idx; row_token, slot_row
        "combine": esz * R * dm + 8.0 * P + esz * T * dm,               # rows, idx + weights, y
    }
    stage_hbm = {k: round(v / (st[k] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) for k, v in stage_bytes.items()}

    # Cold memory-side cache: reading 512 MB between forwards evicts the
    # 256 MB MALL with clean lines, so every weight comes from HBM (the timed
    # steps above run back to back).
    junk = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)
    cold = []
    for _ in range(max(3, min(args.steps, 10))):
        torch.sum(junk, dim=0, dtype=torch.int64, out=sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fwd(*call_args, checked=True)
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del junk, sink
    cold_ms = float(np.median(cold))

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    out = {
        "metric": "MoE-layer fwd tokens/sec + expert GEMM TFLOP/s (% MFMA peak), 16B-shape layer",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": warmup_run,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"DeepSeekMoE {cfg.name} layer forward: T={T}, d={dm}, "
                        f"{cfg.n_routed} routed (top-{K}) + {cfg.n_shared} shared experts, "
                        f"SiLU FFN width {I}, {cfg.gate}",
            "tokens": T, "d_model": dm, "n_routed": cfg.n_routed, "n_shared": cfg.n_shared,
            "top_k": K, "d_ff": I, "gate": cfg.gate, "parallelism": "single GPU",
            "weights": layout,
        },
        "expert_gemm_tflops": expert_tflops,
        "expert_gemm_frac_mfma": expert_tflops / PEAK_BF16_TFLOPS,
        "layer_tflops": layer_tflops,
        "stage_ms": st,
        "routing_stats": {"route_ms": route_ms, "route_stats_ms": route_stats_ms,
                          "n_devices": n_dev},
        "capacity": capacity,
        "weights": layout,
        "other_layout": {"weights": other, "ms_per_step": other_ms},
        "layer_algorithmic_bytes": layer_bytes,
        "layer_hbm_gbs": layer_gbs,
        "layer_hbm_frac": layer_gbs / PEAK_HBM_GBS,
        "cold_mall_ms_per_step": cold_ms,
        "cold_mall_layer_hbm_frac": layer_bytes / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "stage_algorithmic_bytes": stage_bytes,
        "stage_hbm_frac": stage_hbm,
        "roofline": {
            "kernel": "gate/up grouped GEMM (grouped_gemm_bf16 gate/up, grouped; routed experts"
                      + (" + shared experts as extra groups)" if fold else ")"),
            "bound": "mfma" if mfma_bound else "hbm",
            "achieved": gu_tflops if mfma_bound else gu_gbs,
            "peak": PEAK_BF16_TFLOPS if mfma_bound else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": gu_tflops / PEAK_BF16_TFLOPS if mfma_bound else gu_gbs / PEAK_HBM_GBS,
            "traffic": TRAFFIC_BYTES.get((cfg.name, layout)),
            "algorithmic_flop_per_launch": gu_flop,
            "algorithmic_bytes_per_launch": gu_bytes,
            "avg_launch_ms": gu_ms,
        },
    }
    if args.cpu_tokens > 0:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, args.cpu_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
