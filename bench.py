#!/usr/bin/env python3
"""DeepSeekMoE layer forward on one MI355X: tokens/s and expert-GEMM TFLOP/s.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 16b]

A step is one moe_forward (router, dispatch, routed gate/up and down grouped
GEMMs, shared experts, combine) over one batch of seeded synthetic inputs
that are resident in HBM before timing starts.  By default the expert
weights and the router weights are converted once to their packed layouts
(moe_pack_weights, moe_pack_router) before timing, as a server would at load
time; --weights row_major times the plain layouts, and the JSON line carries
the other layouts' time beside it.  The timed steps run through
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
the host cores, repeated until CPU_MIN_S of wall time have passed; `cores`
is the BLAS thread count it ran with, `host_cpu_count` the host's cores.

The `decode` object times the decode-shaped layer (the same 16B layer at
T = 128) in the same run, DECODE_STEPS_MULT times as many steps (a step
is about a quarter of a millisecond long): ms per step, the layer's
fraction of the HBM roofline back to back and with a cold memory-side
cache, and its gate/up kernel against HBM bandwidth.  `decode.graph`
times the same forward captured once in a HIP graph and replayed (checked
bit for bit against the eager forward first).
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
DECODE_WORKLOAD = "16b-decode"
DECODE_STEPS_MULT = 10

# HBM bytes per launch of the routed gate/up kernel, by (layer, weight layout),
# from rocprofv3 FETCH_SIZE and WRITE_SIZE in KiB, scaled by the factors a
# plain 1 GiB copy gives in the same run (the summary under profiles/ names
# the command).  Each entry carries the SHA-256 prefix of the GEMM source it
# was taken on; when the source differs the figure no longer describes the
# kernel and roofline.traffic is null.
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_43_amd", "csrc", "gemm_bf16.hip")
TRAFFIC_BYTES = {
    # profiles/moe_layer_16b_counters.md, profiles/moe_layer_16b-decode_counters.md
    ("16b", "packed"): {"bytes": 4065112789, "gemm_sha": "4c511375cb5efa38"},
    ("16b-decode", "packed"): {"bytes": 768868651, "gemm_sha": "4c511375cb5efa38"},
}


def gemm_source_sha() -> str:
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(layer: str, layout: str):
    e = TRAFFIC_BYTES.get((layer, layout))
    if e is None or e["gemm_sha"] != gemm_source_sha():
        return None
    return e["bytes"]


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
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-shaped layer's side measurement")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure reference ceilings: a 1 GiB device copy and hipBLASLt (torch.matmul) "
                         "on the dense equivalents of the expert GEMMs")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the forward only (no breakdown, capacity, statistics or other layout)")
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
    return {"value": runs * n / dt, "unit": "tokens/s", "cores": threads,
            "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"first {n} of {cfg.tokens} tokens of the same layer, fp64 numpy "
                      f"(routing + dispatch + all chosen experts + shared + combine), "
                      f"{runs} runs, {dt:.1f} s wall, {cpu:.1f} s CPU"}


class Bench:
    """One layer shape on the GPU: inputs resident in HBM, optionally packed
    weights, a forward object and the timing helpers."""

    def __init__(self, cfg, weights, dev):
        import torch

        from mixture_experts_layer_43_amd import _lib, ops
        from synth import make_inputs
        self.cfg, self.dev = cfg, dev
        t_gen = time.perf_counter()
        self.inputs = make_inputs(cfg)
        self.d = d = {k: upload(v, dev) for k, v in self.inputs.items()}
        torch.cuda.synchronize()
        print(f"[bench] inputs for {cfg.name} ready in {time.perf_counter() - t_gen:.1f}s",
              file=sys.stderr, flush=True)
        self.lay_rm = ops.Layer.of(cfg)
        self.weight_keys = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
        self.packable = cfg.dtype == "bf16" and all(
            v % 128 == 0 for v in (cfg.d_model, cfg.d_ff, cfg.d_ff_shared))
        self.layout = weights if self.packable else "row_major"
        self.rm_args = [d["x"], d["w_router"], d["bias"], *[d[k] for k in self.weight_keys]]
        if self.layout == "packed":
            # The router's packed order needs the matrix-core router (bf16,
            # d % 64, N_r <= 128).
            rpk = cfg.d_model % 64 == 0 and cfg.n_routed <= 128
            self.lay = dataclasses.replace(self.lay_rm, weight_layout="packed",
                                           router_layout="packed" if rpk else "row_major")
            pk = {k: ops.pack_weights(self.lay_rm, d[k]) for k in self.weight_keys}
            w_router = ops.pack_router(self.lay_rm, d["w_router"]) if rpk else d["w_router"]
            self.call_args = [d["x"], w_router, d["bias"], *[pk[k] for k in self.weight_keys]]
        else:
            self.lay = self.lay_rm
            self.call_args = self.rm_args
        self.fwd = ops.Forward(self.lay, cfg.tokens, dev)
        self.fwd.check(*self.call_args, None)
        self.hip = hip_runtime()
        self.nev = 2 * _lib.MOE_NUM_STAGES
        self.created = []
        self.c_layer = self.lay.c()
        self.stream = ops._stream()
        self.lib = _lib.lib()
        self.fold = cfg.n_shared > 0 and cfg.d_ff_shared == cfg.d_ff

    def close(self):
        for ev in self.created:
            self.hip.hipEventDestroy(ev)
        self.created = []

    def warm(self, warmup):
        import torch
        n, t_w = 0, time.perf_counter()
        while n < warmup or time.perf_counter() - t_w < WARMUP_MIN_S:
            for _ in range(max(1, warmup)):
                self.fwd(*self.call_args, checked=True)
            n += max(1, warmup)
            torch.cuda.synchronize()
        return n

    def markers(self, stages):
        """Event array for moe_forward_timed with handles for `stages` only."""
        arr = (ctypes.c_void_p * self.nev)()
        for st_i in stages:
            for i in (2 * st_i, 2 * st_i + 1):
                ev = ctypes.c_void_p()
                assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
                arr[i] = ev.value
                self.created.append(ev.value)
        return arr

    def elapsed(self, arr, st_i):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), arr[2 * st_i], arr[2 * st_i + 1]) == 0
        return f.value

    def step(self, arr):
        from mixture_experts_layer_43_amd import _lib, ops
        p, fwd = ops._p, self.fwd
        _lib.check("moe_forward_timed", self.lib.moe_forward_timed(
            ctypes.byref(self.c_layer), self.cfg.tokens, *[p(a) for a in self.call_args], None,
            p(fwd.y), p(fwd.topk_idx), p(fwd.topk_w), p(fwd.counts), p(fwd.offsets), p(fwd.ws),
            fwd.ws.numel(), self.stream, arr))

    def timed(self, steps):
        """Back-to-back steps between two events on the launch stream; HIP
        events bound to the gate/up launch in each.  (ms per step, gate/up ms)."""
        import numpy as np
        import torch

        from mixture_experts_layer_43_amd import _lib
        gu = _lib.STAGES.index("routed_gate_up")
        arrs = [self.markers([gu]) for _ in range(steps)]
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for k in range(steps):
            self.step(arrs[k])
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        gu_ms = float(np.mean([self.elapsed(a, gu) for a in arrs]))
        return ms, gu_ms

    def breakdown(self, n):
        """Per-stage ms from n steps with every marker set."""
        import numpy as np
        import torch

        from mixture_experts_layer_43_amd import _lib
        brk = [self.markers(range(_lib.MOE_NUM_STAGES)) for _ in range(n)]
        for arr in brk:
            self.step(arr)
        torch.cuda.synchronize()
        st = np.array([[self.elapsed(a, i) for i in range(_lib.MOE_NUM_STAGES)] for a in brk])
        return dict(zip(_lib.STAGES, st.mean(0).round(5).tolist()))

    def cold_mall(self, n):
        """Median ms of single forwards, each right after a clean 512 MB read
        that evicts the 256 MB memory-side cache.  The read, the start event
        and the forward are enqueued together, so the forward's kernels are
        queued before the GPU reaches the start event and the time holds no
        host launch latency."""
        import numpy as np
        import torch
        junk = torch.ones(128 << 20, dtype=torch.int32, device=self.dev)
        sink = torch.empty((), dtype=torch.int64, device=self.dev)
        cold = []
        for _ in range(n):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.sum(junk, dim=0, dtype=torch.int64, out=sink)
            a.record()
            self.fwd(*self.call_args, checked=True)
            b.record()
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        del junk, sink
        return float(np.median(cold))

    def graph(self):
        """One moe_forward captured in a HIP graph (through torch.cuda.CUDAGraph on
        the launch stream), checked against the eager result."""
        import torch
        y_eager = self.fwd.y.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                self.fwd(*self.call_args, checked=True)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            self.fwd(*self.call_args, checked=True)
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(self.fwd.y, y_eager):
            raise RuntimeError("graph replay of moe_forward differs from the eager forward")
        return g

    def graph_timed(self, g, steps, warmup):
        """ms per replay of g, back to back, after warm-up replays."""
        import torch
        t_w = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t_w < WARMUP_MIN_S:
            g.replay()
            n += 1
            if n % 50 == 0:
                torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def graph_cold(self, g, n):
        """Median ms of single replays, each right after a clean 512 MB read
        (enqueued together, as in cold_mall)."""
        import numpy as np
        import torch
        junk = torch.ones(128 << 20, dtype=torch.int32, device=self.dev)
        sink = torch.empty((), dtype=torch.int64, device=self.dev)
        out = []
        for _ in range(n):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.sum(junk, dim=0, dtype=torch.int64, out=sink)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        del junk, sink
        return float(np.median(out))

    def layer_bytes(self):
        """Least bytes a forward moves: the weights of every expert it uses,
        the router weights, x and y."""
        cfg = self.cfg
        touched = int((self.fwd.counts.cpu().numpy() > 0).sum())
        esz = 2 if cfg.dtype == "bf16" else 4
        dm, I = cfg.d_model, cfg.d_ff
        return (3.0 * esz * dm * (touched * I + cfg.n_shared * cfg.d_ff_shared)
                + 4.0 * cfg.n_routed * dm + 2.0 * esz * cfg.tokens * dm)

    def gate_up_roofline(self, gu_ms):
        """The gate/up launch against its roofline: 4*R*d*I FLOPs and, at the
        least, W1/W3 of the experts it uses + x once + the R x I outputs."""
        cfg = self.cfg
        T, dm, I = cfg.tokens, cfg.d_model, cfg.d_ff
        rows = T * cfg.top_k + (T * cfg.n_shared if self.fold else 0)
        flop = 4.0 * rows * dm * I
        touched = int((self.fwd.counts.cpu().numpy() > 0).sum())
        n_w = touched + (cfg.n_shared if self.fold else 0)
        byts = 2.0 * (2 * n_w * I * dm + T * dm + rows * I)
        tflops = flop / (gu_ms * 1e-3) / 1e12
        gbs = byts / (gu_ms * 1e-3) / 1e9
        mfma = flop / byts >= (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
        return {
            "kernel": "gate/up grouped GEMM (grouped_gemm_bf16 gate/up, grouped; routed experts"
                      + (" + shared experts as extra groups)" if self.fold else ")"),
            "bound": "mfma" if mfma else "hbm",
            "achieved": tflops if mfma else gbs,
            "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": tflops / PEAK_BF16_TFLOPS if mfma else gbs / PEAK_HBM_GBS,
            "traffic": traffic_for(cfg.name, self.layout),
            "algorithmic_flop_per_launch": flop,
            "algorithmic_bytes_per_launch": byts,
            "avg_launch_ms": gu_ms,
        }


def per_call_ms(fn, n=20):
    import torch
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


def ceilings(dev):
    """Reference ceilings on this GPU, measured in the same process: the HBM
    rate of a plain 1 GiB device copy (bytes read + written), and hipBLASLt
    bf16 GEMMs (through torch.matmul, normal random data) of the dense shapes
    that the 16b layer's expert GEMMs would be without routing: M rows of
    activations (the routed rows, and routed + shared) against one weight
    matrix of the gate/up (N = 2 I) or down (N = d) shape."""
    import torch
    out = {}
    a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
    b = torch.empty_like(a)
    out["copy_1gib_gbs"] = 2.0 * a.numel() * 2 / (per_call_ms(lambda: b.copy_(a), n=10) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev).manual_seed(43)
    gemms = {}
    for name, (M, N, K) in {"gate_up_routed": (98304, 2816, 2048), "gate_up_all": (131072, 2816, 2048),
                            "down_routed": (98304, 2048, 1408), "down_all": (131072, 2048, 1408)}.items():
        x = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=g)
        w = torch.randn(K, N, device=dev, dtype=torch.bfloat16, generator=g) * (K ** -0.5)
        y = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < WARMUP_MIN_S:
            torch.matmul(x, w, out=y)
            torch.cuda.synchronize()
        ms = per_call_ms(lambda: torch.matmul(x, w, out=y), n=10)
        gemms[name] = {"M": M, "N": N, "K": K, "ms": ms, "tflops": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
        del x, w, y
        torch.cuda.empty_cache()
    out["hipblaslt_bf16"] = gemms
    return out


def decode_side(args, dev):
    """The decode-shaped layer, measured in the same run (not the bench line's value)."""
    import torch

    from synth import get_config
    cfg = get_config(DECODE_WORKLOAD)
    b = Bench(cfg, args.weights, dev)
    steps = max(1, args.steps) * DECODE_STEPS_MULT
    warm = b.warm(args.warmup)
    ms, gu_ms = b.timed(steps)
    st = b.breakdown(max(3, min(steps, 20)))
    cold_ms = b.cold_mall(max(5, min(args.steps, 20)))
    lb = b.layer_bytes()
    roof = b.gate_up_roofline(gu_ms)
    # The same forward as a HIP graph: one submission per step, the way a
    # decode loop that cannot afford per-kernel launches runs it.
    g = b.graph()
    g_ms = b.graph_timed(g, steps, args.warmup)
    g_cold = b.graph_cold(g, max(5, min(args.steps, 20)))
    del g
    b.close()
    out = {
        "workload": f"DeepSeekMoE {cfg.name} layer forward: T={cfg.tokens}, d={cfg.d_model}, "
                    f"{cfg.n_routed} routed (top-{cfg.top_k}) + {cfg.n_shared} shared experts, "
                    f"SiLU FFN width {cfg.d_ff}, {cfg.gate}",
        "tokens": cfg.tokens, "weights": b.layout, "router_weights": b.lay.router_layout,
        "steps": steps, "warmup_run": warm,
        "ms_per_step": ms, "tokens_per_s": cfg.tokens / (ms * 1e-3),
        "layer_algorithmic_bytes": lb,
        "layer_hbm_gbs": lb / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": lb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "cold_mall_ms_per_step": cold_ms,
        "cold_mall_layer_hbm_frac": lb / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "stage_ms": st,
        "roofline": roof,
        "graph": {"ms_per_step": g_ms, "layer_hbm_frac": lb / (g_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "cold_mall_ms_per_step": g_cold,
                  "cold_mall_layer_hbm_frac": lb / (g_cold * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }
    del b
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is run and timed on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_43_amd import _lib, ops
    from synth import get_config

    cfg = get_config(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    b = Bench(cfg, args.weights, dev)
    warmup_run = b.warm(args.warmup)

    # Timed region: whole-layer steps; HIP events mark only the gate/up kernel.
    ms, gu_ms = b.timed(args.steps)
    print(f"[bench] {cfg.name}: {ms:.4f} ms per step, gate/up {gu_ms:.4f} ms", file=sys.stderr,
          flush=True)

    T, dm, I, K = cfg.tokens, cfg.d_model, cfg.d_ff, cfg.top_k
    P = T * K
    fold = b.fold
    routed_flop = 6.0 * P * dm * I
    sh_flop = 6.0 * T * dm * cfg.n_shared * cfg.d_ff_shared
    router_flop = 2.0 * T * dm * cfg.n_routed
    layer_bytes = b.layer_bytes()
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
            "weights": b.layout, "router_weights": b.lay.router_layout,
        },
        "weights": b.layout,
        "layer_algorithmic_bytes": layer_bytes,
        "layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": b.gate_up_roofline(gu_ms),
    }

    if not args.no_extras:
        # Per-stage breakdown from separate steps after the timed region
        # (every marker costs a few microseconds of GPU time).
        st = b.breakdown(max(3, min(args.steps, 10)))
        expert_ms = st["routed_gate_up"] + st["routed_down"]
        if not fold:
            expert_ms += st["shared_gate_up"] + st["shared_down"]
        expert_tflops = (routed_flop + sh_flop) / (expert_ms * 1e-3) / 1e12
        out["expert_gemm_tflops"] = expert_tflops
        out["expert_gemm_frac_mfma"] = expert_tflops / PEAK_BF16_TFLOPS
        out["layer_tflops"] = (routed_flop + sh_flop + router_flop) / (ms * 1e-3) / 1e12
        out["stage_ms"] = st
        # The small memory-bound stages against HBM, with their own bytes.
        R = P + (T * cfg.n_shared if fold else (T if cfg.n_shared > 0 else 0))
        esz = 2 if cfg.dtype == "bf16" else 4
        stage_bytes = {
            "route": esz * T * dm + 4.0 * cfg.n_routed * dm + 8.0 * P,   # x, W_g, idx + weights
            "dispatch": 4.0 * P + 8.0 * P + 8.0 * cfg.n_routed,         # idx; row_token, slot_row
            "combine": esz * R * dm + 8.0 * P + esz * T * dm,           # rows, idx + weights, y
        }
        out["stage_algorithmic_bytes"] = stage_bytes
        out["stage_hbm_frac"] = {k: round(v / (st[k] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                                 for k, v in stage_bytes.items()}

        # Routing statistics next to the plain router on the same batch.
        d, p, lib, c_layer, stream = b.d, ops._p, b.lib, b.c_layer, b.stream
        n_dev = 8 if cfg.n_routed % 8 == 0 else 1
        w_router = b.call_args[1]     # in the timed forward's router layout
        s_idx, s_w, s_stats, s_lse = ops.route_stats(b.lay, d["x"], w_router, d["bias"], n_dev,
                                                     lse=True, ws=b.fwd.ws)

        def route_plain():
            _lib.check("moe_route", lib.moe_route(ctypes.byref(c_layer), T, p(d["x"]),
                                                  p(w_router), p(d["bias"]), p(s_idx), p(s_w),
                                                  stream))

        def route_with_stats():
            _lib.check("moe_route_stats", lib.moe_route_stats(
                ctypes.byref(c_layer), T, p(d["x"]), p(w_router), p(d["bias"]), n_dev,
                p(s_idx), p(s_w), p(s_stats), p(s_lse), p(b.fwd.ws), b.fwd.ws.numel(), stream))

        out["routing_stats"] = {"route_ms": per_call_ms(route_plain),
                                "route_stats_ms": per_call_ms(route_with_stats), "n_devices": n_dev}

        # The other weight layout on the same batch.
        other = "row_major" if b.layout == "packed" else ("packed" if b.packable else None)
        other_ms = None
        if other is not None:
            lay_o = dataclasses.replace(b.lay_rm, weight_layout=other)
            o_args = b.rm_args if other == "row_major" else \
                [d["x"], d["w_router"], d["bias"],
                 *[ops.pack_weights(b.lay_rm, d[k]) for k in b.weight_keys]]
            fo = ops.Forward(lay_o, T, dev)
            other_ms = per_call_ms(lambda: fo(*o_args, checked=True), n=max(3, min(args.steps, 10)))
            del fo, o_args
            torch.cuda.empty_cache()
        out["other_layout"] = {"weights": other, "ms_per_step": other_ms}

        # Expert capacity (Switch/GShard, one group of the whole batch): the
        # same layer with C = ceil(factor * T * K' / N_r) slots per expert.
        capacity = {}
        for factor in (1.0, 1.25):
            C = -(-int(factor * 100) * T * K // (100 * cfg.n_routed))
            fc = ops.Forward(dataclasses.replace(b.lay, capacity=C), T, dev)
            ms_c = per_call_ms(lambda: fc(*b.call_args, checked=True), n=max(3, min(args.steps, 10)))
            capacity[str(factor)] = {"capacity": C, "ms_per_step": ms_c,
                                     "kept_frac": int(fc.counts.sum()) / (T * K)}
            del fc
            torch.cuda.empty_cache()
        out["capacity"] = capacity

        cold_ms = b.cold_mall(max(3, min(args.steps, 10)))
        out["cold_mall_ms_per_step"] = cold_ms
        out["cold_mall_layer_hbm_frac"] = layer_bytes / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        c = torch.empty_like(a)
        for _ in range(3):
            c.copy_(a)
        torch.cuda.synchronize()
        del a, c
    b.close()
    inputs = b.inputs
    del b
    torch.cuda.empty_cache()

    if args.ceilings:
        print("[bench] reference ceilings", file=sys.stderr, flush=True)
        out["ceilings"] = ceilings(dev)

    if not args.no_decode and cfg.name != DECODE_WORKLOAD:
        print(f"[bench] decode-shaped layer {DECODE_WORKLOAD}", file=sys.stderr, flush=True)
        out["decode"] = decode_side(args, dev)

    if args.cpu_tokens > 0:
        print("[bench] timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, inputs, args.cpu_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
