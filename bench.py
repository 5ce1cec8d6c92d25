#!/usr/bin/env python3
"""Throughput of one Edge0-145B-shaped latent-MoE layer on one MI355X; prints one JSON line.

A step is one lmoe_forward (D projection, router, top-k, permutation, expert SwiGLU with the
shared expert, combine, U projection) over one batch of synthetic tokens already resident
in HBM.  The timed steps are enqueued back to back on one stream and cycle through
`--rotate` byte-identical copies of the layer's weights at different HBM addresses, so the
256 MB last-level cache cannot serve a step from the previous one.  HIP events recorded by
the library around the dominant kernel of every timed step give its duration.  The same
steps replayed from captured HIP graphs are timed afterwards and reported beside it.

Workloads (lmoe_data.WORKLOADS): decode_t8 (default, HBM-bound), prefill_t4096,
prefill_t16384 (MFMA-bound; measured as the secondary line by default), stack48_mxfp4_t8.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-MoE layer tok/s: decode T=8 (%HBM BW), 16K prefill (%MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 (the block-scaled MXFP8 x MXFP4 products run at the fp8 rate)
MX_MIN_T = 96  # batches from which MXFP4 experts take the block-scaled MFMA kernels (kMxMinT in the library)
STAGE_UP = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """hipEvent handles for the stage-event hook (created through the HIP runtime)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipGetLastError.restype = ctypes.c_int

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b, required=True):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            assert not required, f"hipEventElapsedTime {rc}"
            self.lib.hipGetLastError()
            return None
        return ms.value


def algorithmic_counts(wl, ids: np.ndarray, T=None):
    """Bytes and flops the method itself needs for one layer step, from the step's own routing."""
    s = wl.shape
    T = wl.T if T is None else T
    H, L, E, k, F, Fs = s.hidden, s.latent, s.n_experts, s.top_k, s.ffn, s.shared_ffn
    G = s.groups  # expert groups, each with its own D and U (all of them read: z of every group is formed)
    nd = int(np.unique(ids).size)
    wb = 2  # bf16 dense weights
    rec = {"mxfp4": s.mxfp4_record_bytes(), "nvfp4": s.nvfp4_record_bytes()}.get(wl.expert, 3 * F * L * 2)
    up_w = {"mxfp4": 2 * F * L // 2 + 2 * F * L // 32,
            "nvfp4": 2 * F * L // 2 + 2 * F * L // 16 + 8}.get(wl.expert, 2 * F * L * 2)
    dense = (2 * H * L * G + E * L) * wb + E * 4 + 3 * Fs * L * wb
    xin = T * H * (4 if wl.layers > 1 else 2)
    yout = T * H * (4 if wl.layers > 1 else 2)
    layer_bytes = dense + nd * rec + xin + yout
    flops_tok = 2 * (H * L * G + L * E + k * 3 * F * L + 3 * Fs * L + L * H * G)
    rows = T * k + (T if Fs else 0)
    up_bytes = nd * up_w + 2 * Fs * L * wb + T * L * G * 2 + rows * max(F, Fs) * 2
    up_flops = 2 * (T * k * 2 * F * L + (T * 2 * Fs * L if Fs else 0))
    # gate/up launch: the gate and up rows of every touched expert and of the shared expert once,
    # the latent tokens in, SiLU(g) * u out (bf16, one row of the SwiGLU width per segment row)
    return dict(n_distinct_experts=nd, layer_bytes=layer_bytes, layer_flops=flops_tok * T, up_bytes=up_bytes,
                up_flops=up_flops)


def layer_copies(wl, rotate):
    """`rotate` byte-identical device copies of the workload's layer 0."""
    import lmoe_data as gen
    from sparse_moe_proj_amd.device import DeviceLayer

    t0 = time.time()
    lw = gen.make_layer(wl, 0)
    log(f"[bench] {wl.name}: generated layer in {time.time() - t0:.1f}s")
    base = DeviceLayer(lw, act=wl.act)
    del lw
    return [base] + [base.clone() for _ in range(rotate - 1)]


def measure(wl, steps, warmup, rotate, profile_stages=True, copies=None, T=None, graphs=True):
    """Times `steps` forward steps of T tokens (default: the workload's T) over the weight copies."""
    import torch

    import lmoe_data as gen
    import sparse_moe_proj_amd as lm
    from sparse_moe_proj_amd.device import Workspace, to_device

    hip = Hip()
    if copies is None:
        copies = layer_copies(wl, rotate)
    rotate = len(copies)
    base = copies[0]
    T = wl.T if T is None else T
    x = to_device(gen.make_tokens(wl, T=T))
    y = torch.empty((T, wl.shape.hidden), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, wl.shape.top_k), dtype=torch.int32, device="cuda")
    nbytes = lm.lmoe_workspace_bytes(base.cfg, T)
    ws = Workspace("cuda").get(nbytes)

    def fwd(dl, opts=None):
        lm.check(lm.lmoe_forward(dl.cfg, dl.weights, x, T, y, opts, ws, ws.numel()))

    fwd(base, lm.make_opts(aux_ids=ids))
    torch.cuda.synchronize()
    counts = algorithmic_counts(wl, ids.cpu().numpy(), T)
    for i in range(warmup):
        fwd(copies[i % rotate])
    torch.cuda.synchronize()

    # per-stage breakdown (eager, untimed): every stage bracketed by events
    stages_us = {}
    if profile_stages:
        acc = np.zeros(lm.LMOE_N_STAGES)
        seen = np.zeros(lm.LMOE_N_STAGES, dtype=bool)
        n = max(rotate, 4)
        for i in range(n):
            evs = [hip.event() for _ in range(2 * lm.LMOE_N_STAGES)]  # fresh: stages not launched stay unrecorded
            arr = (ctypes.c_void_p * len(evs))(*evs)
            fwd(copies[i % rotate], lm.make_opts(stage_events=arr))
            torch.cuda.synchronize()
            for s_ in range(1, lm.LMOE_N_STAGES):
                ms = hip.elapsed_ms(evs[2 * s_], evs[2 * s_ + 1], required=False)
                if ms is not None:
                    acc[s_] += ms
                    seen[s_] = True
        stages_us = {lm.STAGES[s_]: round(1e3 * acc[s_] / n, 2) for s_ in range(1, lm.LMOE_N_STAGES) if seen[s_]}

    # timed region: K eager steps on one stream, events around the dominant stage of each
    stream = torch.cuda.current_stream()
    ev_pairs, keep = [], []
    for i in range(steps):
        e0, e1 = hip.event(), hip.event()
        arr = (ctypes.c_void_p * (2 * lm.LMOE_N_STAGES))()
        arr[2 * STAGE_UP], arr[2 * STAGE_UP + 1] = e0, e1
        ev_pairs.append((e0, e1))
        keep.append((arr, lm.make_opts(stage_events=arr)))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        fwd(copies[i % rotate], keep[i][1])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = 1e3 * (t_end - t_start) / steps
    up_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev_pairs]))

    if not graphs:
        return dict(ms_per_step=ms_per_step, tok_s=T / (ms_per_step / 1e3), up_ms=up_ms, counts=counts,
                    stages_us=stages_us, weight_bytes_per_copy=base.nbytes(), graph_ms_per_step=None)
    # the same steps replayed from captured HIP graphs (one per weight copy), for comparison
    graphs = []
    for r in range(rotate):
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=s2):
            fwd(copies[r])
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for i in range(steps):
        graphs[i % rotate].replay()
    torch.cuda.synchronize()
    graph_ms = 1e3 * (time.perf_counter() - g0) / steps
    return dict(ms_per_step=ms_per_step, tok_s=T / (ms_per_step / 1e3), up_ms=up_ms, counts=counts,
                stages_us=stages_us, weight_bytes_per_copy=base.nbytes(), graph_ms_per_step=graph_ms)


def measure_stack(wl, steps, warmup):
    """The multi-layer stack (pre-RMSNorm, fp32 residual updated in place): every layer's weights
    resident at their own HBM addresses (layers sharing an expert bank hold separate copies), a
    step is one pass of the T tokens through all layers; reported per layer."""
    import torch

    import lmoe_data as gen
    import sparse_moe_proj_amd as lm
    from sparse_moe_proj_amd.device import DeviceLayer, Workspace, to_device

    hip = Hip()
    t0 = time.time()
    banks = {b: gen.make_experts(wl, b) for b in range(max(wl.expert_banks, 1))}
    layers = []
    for l in range(wl.layers):
        lw = gen.make_layer(wl, l, experts=banks[gen.expert_bank(wl, l)] if wl.expert_banks else None)
        layers.append(DeviceLayer(lw, act="bf16"))
    del banks
    log(f"[bench] {wl.name}: {wl.layers} layers generated and uploaded in {time.time() - t0:.1f}s")
    T = wl.T
    h = to_device(gen.make_residual(wl))
    ws = Workspace("cuda").get(lm.lmoe_workspace_bytes(layers[0].cfg, T))
    ids = [torch.empty((T, wl.shape.top_k), dtype=torch.int32, device="cuda") for _ in layers]

    def layer_fwd(dl, opts):
        lm.check(lm.lmoe_forward(dl.cfg, dl.weights, h, T, h, opts, ws, ws.numel()))

    # routing of one pass (for the algorithmic byte counts), then warmup passes
    for dl, idt in zip(layers, ids):
        layer_fwd(dl, lm.make_opts(prenorm=1, residual=1, aux_ids=idt))
    torch.cuda.synchronize()
    counts = [algorithmic_counts(wl, idt.cpu().numpy()) for idt in ids]
    for _ in range(warmup):
        for dl in layers:
            layer_fwd(dl, lm.make_opts(prenorm=1, residual=1))
    torch.cuda.synchronize()
    opts, evs = [], []
    for _ in range(steps):
        for _l in layers:
            e0, e1 = hip.event(), hip.event()
            arr = (ctypes.c_void_p * (2 * lm.LMOE_N_STAGES))()
            arr[2 * STAGE_UP], arr[2 * STAGE_UP + 1] = e0, e1
            evs.append((e0, e1))
            opts.append((arr, lm.make_opts(prenorm=1, residual=1, stage_events=arr)))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    i = 0
    for _ in range(steps):
        for dl in layers:
            layer_fwd(dl, opts[i][1])
            i += 1
    torch.cuda.synchronize()
    ms_per_layer = 1e3 * (time.perf_counter() - t_start) / (steps * wl.layers)
    up_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in evs]))
    mean = {key: float(np.mean([c[key] for c in counts])) for key in ("layer_bytes", "layer_flops", "up_bytes",
                                                                      "up_flops", "n_distinct_experts")}
    return dict(ms_per_step=ms_per_layer, tok_s=T / (ms_per_layer / 1e3), up_ms=up_ms, counts=mean,
                stages_us={}, graph_ms_per_step=None)


def cpu_baseline(wl, seconds):
    """The oracle as it stands (float64 numpy), on the host's cores, on whole decode steps."""
    import lmoe_data as gen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    lw = gen.make_layer(wl, 0)
    x = oracle.decode(gen.make_tokens(wl), wl.act)
    reps, tok = 0, 0
    t0 = time.perf_counter()
    while True:
        L = oracle.Layer(lw)  # includes promoting the touched weights to float64
        oracle.block_forward(L, x)
        reps += 1
        tok += x.shape[0]
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(tok / dt, 3), "unit": "tok/s per layer", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} whole {wl.name} steps (T={x.shape[0]}), float64 numpy, weights promoted per step",
            "seconds": round(dt, 2)}


def measured_traffic(workload):
    """HBM bytes per launch of the small-batch gate/up kernel from the committed rocprofv3 counter
    passes (FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size), or None when the kernel's
    sources have changed since the counters were taken or no pass covers this workload."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_decode_gu_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, "sparse_moe_proj_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes"] if h.hexdigest() == rec["sources_sha256"] else None


def roofline_hbm(counts, up_ms, traffic=None):
    achieved = counts["up_bytes"] / (up_ms / 1e3) / 1e9
    return {"bound": "hbm", "kernel": "decode_gu_kernel (expert gate/up and SwiGLU)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": counts["up_bytes"], "avg_launch_us": round(up_ms * 1e3, 2)}


def mx_mfma_path(wl):
    """Whether the workload's expert products take the block-scaled MXFP8 x MXFP4 MFMA kernels."""
    min_t = int(os.environ.get("LMOE_MX_MIN_T", "0") or 0) or MX_MIN_T
    return wl.expert == "mxfp4" and wl.T >= max(min_t, 17) and os.environ.get("LMOE_MX_MFMA", "1")[:1] != "0"


def roofline_mfma(counts, up_ms, wl=None):
    achieved = counts["up_flops"] / (up_ms / 1e3) / 1e12
    if wl is not None and mx_mfma_path(wl):
        kernel, peak = ("expert gate/up (mx_gemm_persistent MxUp, MXFP8 z + MXFP4 residual x MXFP4 records; "
                        "with the z quantization and the bf16 shared expert)"), MFMA_FP8_PEAK_TFLOPS
    else:
        kernel, peak = "expert gate/up (pipe_gemm_persistent PipeUp)", MFMA_BF16_PEAK_TFLOPS
    return {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1),
            "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": None, "flops_per_launch": counts["up_flops"], "avg_launch_us": round(up_ms * 1e3, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_t8")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--secondary", default="prefill_t16384", help="second workload line ('' = none)")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (calibrates HBM traffic counters)")
    ap.add_argument("--tsweep", default="",
                    help="comma-separated token counts: also time the workload's layer at each T (a 'tsweep' list)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the latent-MoE block is built and measured on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import lmoe_data as gen
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = gen.WORKLOADS[args.workload]
    if wl.layers > 1:  # the stack streams its own distinct layers: no weight copies to rotate
        copies = None
        m = measure_stack(wl, args.steps, args.warmup)
        args.rotate = 1
    else:
        copies = layer_copies(wl, args.rotate)
        m = measure(wl, args.steps, args.warmup, args.rotate, copies=copies)
    c = m["counts"]
    mfma_bound = c["layer_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > c["layer_bytes"] / (HBM_PEAK_GBS * 1e9)
    rl = roofline_mfma(c, m["up_ms"], wl) if mfma_bound else roofline_hbm(c, m["up_ms"], measured_traffic(wl.name))
    layer_s = m["ms_per_step"] / 1e3
    out = {
        "metric": METRIC,
        "value": round(m["tok_s"], 1),
        "unit": "tok/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 x mxfp4" if mx_mfma_path(wl) else "bf16",
        "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) tokens, Zipf(1.1) router bias)",
        "config": {"workload": wl.name, "T": wl.T, "hidden": wl.shape.hidden, "latent": wl.shape.latent,
                   "n_experts": wl.shape.n_experts, "top_k": wl.shape.top_k, "ffn": wl.shape.ffn,
                   "shared_ffn": wl.shape.shared_ffn, "router_bias": wl.bias, "weights": wl.expert,
                   "weight_copies": args.rotate, "timed": "eager lmoe_forward calls on one stream"},
        "roofline": rl,
        "layer": {"bytes": c["layer_bytes"], "flops": c["layer_flops"], "n_distinct_experts": c["n_distinct_experts"],
                  "hbm_frac": round(c["layer_bytes"] / layer_s / (HBM_PEAK_GBS * 1e9), 4),
                  "mfma_frac": round(c["layer_flops"] / layer_s / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)},
        "stages_us": m["stages_us"],
        "graph_ms_per_step": round(m["graph_ms_per_step"], 5) if m["graph_ms_per_step"] is not None else None,
    }
    if wl.layers > 1:
        out["config"]["layers"] = wl.layers
        out["config"]["timed"] = "eager lmoe_forward calls, all layers in order, per-layer figures"
    if args.tsweep and copies is not None:
        sweep = []
        for T in [int(v) for v in args.tsweep.split(",") if v]:
            mt = measure(wl, args.steps, args.warmup, args.rotate, profile_stages=False, copies=copies, T=T,
                         graphs=False)
            ct = mt["counts"]
            sweep.append({"T": T, "tok_s": round(mt["tok_s"], 1), "us_per_step": round(1e3 * mt["ms_per_step"], 2),
                          "n_distinct_experts": ct["n_distinct_experts"],
                          "layer_hbm_frac": round(ct["layer_bytes"] / (mt["ms_per_step"] / 1e3) / (HBM_PEAK_GBS * 1e9), 4),
                          "gate_up_us": round(1e3 * mt["up_ms"], 2),
                          "gate_up_gbs": round(ct["up_bytes"] / (mt["up_ms"] / 1e3) / 1e9, 1)})
            log(f"[bench] tsweep {sweep[-1]}")
        out["tsweep"] = sweep
    del copies
    if args.secondary:
        del m
        torch.cuda.empty_cache()
        wl2 = gen.WORKLOADS[args.secondary]
        m2 = measure(wl2, args.secondary_steps, 3, 2)
        c2 = m2["counts"]
        s2 = m2["ms_per_step"] / 1e3
        out["secondary"] = {
            "workload": wl2.name, "T": wl2.T, "value": round(m2["tok_s"], 1), "unit": "tok/s per layer",
            "ms_per_step": round(m2["ms_per_step"], 4),
            "roofline": roofline_mfma(c2, m2["up_ms"]),
            "layer": {"flops": c2["layer_flops"], "bytes": c2["layer_bytes"],
                      "n_distinct_experts": c2["n_distinct_experts"],
                      "mfma_frac": round(c2["layer_flops"] / s2 / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                      "hbm_frac": round(c2["layer_bytes"] / s2 / (HBM_PEAK_GBS * 1e9), 4)},
            "stages_us": m2["stages_us"],
            "graph_ms_per_step": round(m2["graph_ms_per_step"], 4),
        }
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
