#!/usr/bin/env python3
"""Throughput of one Edge0-145B-shaped latent-MoE layer on one MI355X; prints one JSON line.

A step is one lmoe_forward (D projection, router, top-k, permutation, expert SwiGLU with the
shared expert, combine, U projection) over one batch of synthetic tokens already resident
in HBM.  The timed steps are enqueued back to back on one stream and cycle through
`--rotate` byte-identical copies of the layer's weights at different HBM addresses, so the
256 MB last-level cache cannot serve a step from the previous one.

What is measured:
  * value / ms_per_step: exactly --steps eager steps after --warmup untimed ones, bracketed by
    device synchronisation (wall clock);
  * roofline: the dominant kernel (decode: the gate/up launch; prefill: the expert gate/up
    GEMM), its duration from HIP events the library attaches to that launch in every timed
    step, against the published peak and against the rate this part reaches in a plain
    streaming-read or matrix-core loop (libpeaks.so, timed in the same run); the whole layer's
    fraction beside it;
  * timing: at least --graph-reps replays of captured HIP graphs (after 20 untimed ones), each
    bracketed by events: median, p10, p90;
  * clocks: the shader clock read by the matrix-core loop (s_memtime against the 100 MHz
    real-time counter) and, where the driver exposes it, the current SCLK level sampled while
    the graph replays run;
  * cpu_baseline: the oracle on the host's cores for the headline workload, and oracle_baselines
    for every workload on a bounded sample, with the CPU model and host memory.

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


def host_info():
    """CPU model, host memory and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    mem_gb = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    mem_gb = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return {"cpu_model": model, "host_mem_gib": mem_gb, "cores_available": cores}


class SclkSampler:
    """Samples the GPU's current SCLK level (the line the driver marks with '*' in pp_dpm_sclk)
    from a thread while the measured work runs; inactive where the file is not readable."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.path = None
        for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                with open(p) as f:
                    if "*" in f.read():
                        self.path = p
                        break
            except OSError:
                continue
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if self.path else None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if "*" in line:
                        tok = [t for t in line.replace(":", " ").split() if t.lower().endswith("mhz")]
                        return int(tok[0][:-3]) if tok else None
        except (OSError, ValueError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.array(self.samples)
        return {"source": self.path, "samples": int(a.size), "median_mhz": float(np.median(a)),
                "min_mhz": int(a.min()), "max_mhz": int(a.max())}


def measure_peaks():
    """Rates this part reaches in plain loops (libpeaks.so): HBM streaming read, bf16 32x32x16 and
    scaled FP8 x FP4 32x32x64 matrix-core issue, with the shader clock read inside the loops."""
    import torch
    path = os.path.join(ROOT, "sparse_moe_proj_amd", "libpeaks.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python sparse_moe_proj_amd/build.py` first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.peak_stream_read.argtypes = [P, ctypes.c_size_t, P, ctypes.c_int, P]
    lib.peak_mfma.argtypes = [ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, P]
    per_wave = lib.peak_mfma_per_wave()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = {"compute_units": cus}

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return ts

    nbytes = 4 << 30  # well beyond the 256 MB last-level cache
    buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    best = None
    for wg_per_cu in (4, 8, 16):
        grid = cus * wg_per_cu
        sink = torch.zeros(grid, dtype=torch.int32, device="cuda")

        def run():
            assert lib.peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream.cuda_stream) == 0

        ms = float(np.median(timed(run, 7)[2:]))
        gbs = nbytes / (ms / 1e3) / 1e9
        if best is None or gbs > best["GBs"]:
            best = {"GBs": round(gbs, 1), "bytes": nbytes, "workgroups": grid, "ms": round(ms, 4)}
    out["stream_read"] = best
    del buf
    for kind, name, flop in ((0, "mfma_bf16_32x32x16", 32768), (1, "mfma_scale_fp8xfp4_32x32x64", 131072)):
        res = torch.zeros(cus * 256, dtype=torch.float32, device="cuda")
        clk = torch.zeros(4, dtype=torch.int64, device="cuda")
        iters = 4000 if kind == 0 else 2000

        def run():
            assert lib.peak_mfma(kind, res.data_ptr(), iters, clk.data_ptr(), cus, stream.cuda_stream) == 0

        ms = float(np.median(timed(run, 7)[2:]))
        flops = cus * 4 * iters * per_wave * flop
        c = clk.cpu().numpy().astype(np.int64)
        sclk = (c[2] - c[0]) / ((c[3] - c[1]) / 100e6) / 1e6 if c[3] > c[1] else None
        out[name] = {"TFLOPs": round(flops / (ms / 1e3) / 1e12, 1), "ms": round(ms, 4),
                     "sclk_mhz_in_loop": round(sclk, 1) if sclk else None}
    return out


def graph_timing(run_graph, samples, warmup=20, group_us=1000.0):
    """Replays of captured HIP graphs (`run_graph(i)` launches replay i) on the current stream.

    An event recorded between two replays costs the step about 4.6 us at decode size (measured:
    79.3 us per replay with an event around every replay, 74.7 us without), so the spread is taken
    over `samples` groups of g consecutive replays each (g = ceil(group_us / step), at least 1):
    events bracket each group, a sample is the group's time / g, and median, p10 and p90 are
    over the samples (g * samples >= 100 replays).  Then the same number of replays runs with
    events only at its two ends (mean), and a further untimed run of about 200 ms has the SCLK
    level sampled (reading the driver's clock file while timing could perturb what is timed)."""
    import torch
    for i in range(warmup):
        run_graph(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(10):
        run_graph(i)
    b.record()
    torch.cuda.synchronize()
    step_us = 1e3 * a.elapsed_time(b) / 10
    g = max(1, int(np.ceil(group_us / step_us)))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    evs[0].record()
    for i in range(samples):
        for j in range(g):
            run_graph(i * g + j)
        evs[i + 1].record()
    torch.cuda.synchronize()
    us = np.array([1e3 * evs[i].elapsed_time(evs[i + 1]) / g for i in range(samples)])
    n = samples * g
    a.record()
    for i in range(n):
        run_graph(i)
    b.record()
    torch.cuda.synchronize()
    mean_run = 1e3 * a.elapsed_time(b) / n
    with SclkSampler() as sampler:
        for i in range(max(1, int(2e5 / step_us))):
            run_graph(i)
        torch.cuda.synchronize()
    return {"replays": n, "samples": samples, "replays_per_sample": g,
            "median_us": round(float(np.median(us)), 2), "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2), "mean_us": round(mean_run, 2),
            "sclk": sampler.summary()}


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
    base = DeviceLayer(lw, act=wl.act, mx_mfma_min_t=MX_MFMA_MIN_T)
    del lw
    return [base] + [base.clone() for _ in range(rotate - 1)]


def measure(wl, steps, warmup, rotate, profile_stages=True, copies=None, T=None, graphs=True, graph_reps=100):
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
                    stages_us=stages_us, weight_bytes_per_copy=base.nbytes(), graph=None)
    # the same steps replayed from captured HIP graphs (one per weight copy): per-replay events
    graphs = []
    for r in range(rotate):
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=s2):
            fwd(copies[r])
        graphs.append(g)
    torch.cuda.synchronize()
    gt = graph_timing(lambda i: graphs[i % rotate].replay(), max(graph_reps, 100))  # >= 100 replays
    return dict(ms_per_step=ms_per_step, tok_s=T / (ms_per_step / 1e3), up_ms=up_ms, counts=counts,
                stages_us=stages_us, weight_bytes_per_copy=base.nbytes(), graph=gt)


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
    banks = {b: gen.make_experts(wl, b) for b in range(wl.expert_banks)}
    layers = []
    for l in range(wl.layers):
        lw = gen.make_layer(wl, l, experts=banks[gen.expert_bank(wl, l)] if wl.expert_banks else None)
        layers.append(DeviceLayer(lw, act="bf16", mx_mfma_min_t=MX_MFMA_MIN_T))
        del lw
        if l % 8 == 7:
            log(f"[bench] {wl.name}: {l + 1} layers generated and uploaded ({time.time() - t0:.1f}s)")
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
                stages_us={}, graph=None)


class LazyExperts:
    """A layer's routed expert records, each drawn from its own seed on first access: the oracle
    reads only the records of the experts its tokens route to."""

    def __init__(self, wl, bank):
        self.wl, self.bank, self.cache = wl, bank, {}

    def __getitem__(self, e):
        import lmoe_data as gen
        e = int(e)
        if e not in self.cache:
            self.cache[e] = gen.expert_record(self.wl.shape, gen.rng_for(self.wl.wid, self.bank, gen.T_EXPERT, e),
                                              self.wl.expert)
        return self.cache[e]

    def draw(self, ids):
        from concurrent.futures import ThreadPoolExecutor

        import lmoe_data as gen
        with ThreadPoolExecutor(gen.n_threads()) as ex:
            list(ex.map(self.__getitem__, sorted(set(int(e) for e in np.asarray(ids).ravel()))))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def oracle_rate(wl, seconds, ntok=None):
    """The oracle as it stands (float64 numpy) on one layer of `wl`, on the host's cores: passes over
    the workload's T tokens (ntok None) or over its first ntok tokens (tokens are independent units
    of the block, so a sample of them does the same work per token).  Generating the data and drawing
    the routed experts' records happen before the timed passes; every timed pass builds a fresh
    oracle.Layer, so promoting the touched weights to float64 is inside."""
    import lmoe_data as gen
    import oracle
    lazy = LazyExperts(wl, gen.expert_bank(wl, 0))
    lw = gen.make_layer(wl, 0, experts=lazy)
    T = wl.T if ntok is None else min(ntok, wl.T)
    if wl.layers > 1:  # one layer of the stack: bf16(RMSNorm(h)) in, the fp32 residual updated
        h = gen.make_residual(wl, T=T).astype(np.float64)
        x = oracle.round_to_bf16(oracle.rmsnorm(h))

        def step(L):
            return oracle.stack_step(L, h)
    else:
        x = oracle.decode(gen.make_tokens(wl, T=T), wl.act)

        def step(L):
            return oracle.block_forward(L, x)
    L0 = oracle.Layer(lw)
    lazy.draw(oracle.route(x @ L0.D.T, L0.Wr, L0.br, wl.shape.top_k, wl.shape.groups)[0])
    passes = 0
    t0 = time.perf_counter()
    while True:
        step(oracle.Layer(lw))
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    what = "whole steps" if T == wl.T else f"the first {T} of its {wl.T} tokens per pass"
    if wl.layers > 1:
        what = f"one layer of the {wl.layers}-layer stack, T={T}"
    return {"workload": wl.name, "value": round(passes * T / dt, 3), "unit": "tok/s per layer", "tokens_per_pass": T,
            "passes": passes, "seconds": round(dt, 2), "sample": what}


def cpu_baseline(wl, seconds):
    """The headline workload's oracle rate (bounded in time) with the host it ran on."""
    r = oracle_rate(wl, seconds)
    hi = host_info()
    return {"value": r["value"], "unit": r["unit"], "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{r['passes']} passes of {r['sample']} (T={r['tokens_per_pass']}), float64 numpy, weights "
                      f"promoted per pass", "seconds": r["seconds"], "cpu_model": hi["cpu_model"],
            "host_mem_gib": hi["host_mem_gib"]}


# every workload the layer is specified on, with the oracle's token sample (None: whole steps)
ORACLE_SAMPLES = (("tiny_f32", None, 2.0), ("decode_t8", None, 3.0), ("prefill_t4096", 16, 3.0),
                  ("prefill_t16384", 16, 3.0), ("stack48_mxfp4_t8", None, 3.0))


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


def roofline_hbm(counts, up_ms, layer_s, peaks=None, traffic=None):
    """The decode gate/up launch against HBM: algorithmic bytes / its mean duration, as a fraction of
    the published 8 TB/s (frac) and of the streaming-read rate measured in the same run; the
    whole layer's fraction beside it."""
    achieved = counts["up_bytes"] / (up_ms / 1e3) / 1e9
    layer_gbs = counts["layer_bytes"] / layer_s / 1e9
    meas = peaks["stream_read"]["GBs"] if peaks else None
    return {"bound": "hbm", "kernel": "decode_gu_kernel (expert gate/up and SwiGLU)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": counts["up_bytes"], "avg_launch_us": round(up_ms * 1e3, 2),
            "measured_peak": meas, "frac_of_measured": round(achieved / meas, 4) if meas else None,
            "layer_achieved": round(layer_gbs, 1), "layer_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
            "layer_frac_of_measured": round(layer_gbs / meas, 4) if meas else None}


# lmoe_config.mx_mfma_min_t of every layer the benchmark builds (--mx-mfma-min-t)
MX_MFMA_MIN_T = 0


def mx_mfma_path(wl):
    """Whether the workload's expert products take the block-scaled MXFP8 x MXFP4 MFMA kernels."""
    if wl.expert != "mxfp4" or MX_MFMA_MIN_T < 0:
        return False
    return wl.T >= max(MX_MFMA_MIN_T or MX_MIN_T, 65)


def roofline_mfma(counts, up_ms, layer_s, peaks=None, wl=None):
    """The prefill expert gate/up launch against the matrix cores: algorithmic flops / its mean
    duration, as a fraction of the published peak of its operand type (frac) and of the issue rate
    a plain MFMA loop of the same instruction reaches in the same run; the layer beside it (bf16)."""
    achieved = counts["up_flops"] / (up_ms / 1e3) / 1e12
    layer_tf = counts["layer_flops"] / layer_s / 1e12
    if wl is not None and mx_mfma_path(wl):
        kernel, peak, key = ("expert gate/up (mx_gemm_persistent MxUp, MXFP8 z + MXFP4 residual x MXFP4 records; "
                             "with the z quantization and the bf16 shared expert)"), MFMA_FP8_PEAK_TFLOPS, \
            "mfma_scale_fp8xfp4_32x32x64"
    else:
        kernel, peak, key = "expert gate/up (pipe_gemm_persistent PipeUp)", MFMA_BF16_PEAK_TFLOPS, "mfma_bf16_32x32x16"
    meas = peaks[key]["TFLOPs"] if peaks else None
    meas_bf16 = peaks["mfma_bf16_32x32x16"]["TFLOPs"] if peaks else None
    return {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1),
            "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": None, "flops_per_launch": counts["up_flops"], "avg_launch_us": round(up_ms * 1e3, 2),
            "measured_peak": meas, "frac_of_measured": round(achieved / meas, 4) if meas else None,
            "layer_achieved": round(layer_tf, 1), "layer_frac": round(layer_tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "layer_frac_of_measured": round(layer_tf / meas_bf16, 4) if meas_bf16 else None}


def roofline_of(wl, c, m, peaks):
    layer_s = m["ms_per_step"] / 1e3
    mfma_bound = c["layer_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12) > c["layer_bytes"] / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        return roofline_mfma(c, m["up_ms"], layer_s, peaks, wl)
    return roofline_hbm(c, m["up_ms"], layer_s, peaks, measured_traffic(wl.name))


def layer_line(c, m):
    layer_s = m["ms_per_step"] / 1e3
    return {"bytes": c["layer_bytes"], "flops": c["layer_flops"], "n_distinct_experts": c["n_distinct_experts"],
            "hbm_frac": round(c["layer_bytes"] / layer_s / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(c["layer_flops"] / layer_s / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_t8")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--graph-samples", type=int, default=100,
                    help="timed samples of HIP-graph replays (groups of about 1 ms; at least 100 replays); "
                         "0 skips the graph timing (profiler passes)")
    ap.add_argument("--secondary", default="prefill_t16384", help="second workload line ('' = none)")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the streaming-read and MFMA-loop measurements")
    ap.add_argument("--mx-mfma-min-t", type=int, default=0,
                    help="lmoe_config.mx_mfma_min_t of MXFP4 layers (0: the library's default, -1: off)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (calibrates HBM traffic counters)")
    ap.add_argument("--tsweep", default="",
                    help="comma-separated token counts: also time the workload's layer at each T (a 'tsweep' list)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the latent-MoE block is built and measured on a single MI355X "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    global MX_MFMA_MIN_T
    MX_MFMA_MIN_T = args.mx_mfma_min_t
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
        m = measure(wl, args.steps, args.warmup, args.rotate, copies=copies, graph_reps=args.graph_samples,
                    graphs=args.graph_samples > 0)
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks()
        log(f"[bench] measured peaks {json.dumps(peaks)}")
    c = m["counts"]
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
        "roofline": roofline_of(wl, c, m, peaks),
        "layer": layer_line(c, m),
        "timing": m["graph"],
        "stages_us": m["stages_us"],
        "peaks_measured": peaks,
        "host": host_info(),
    }
    if wl.layers > 1:
        out["config"]["layers"] = wl.layers
        out["config"]["expert_sets"] = wl.expert_banks or wl.layers  # distinct sets of 512 routed experts
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
        m2 = measure(wl2, args.secondary_steps, 3, 2, graph_reps=args.graph_samples, graphs=args.graph_samples > 0)
        c2 = m2["counts"]
        out["secondary"] = {
            "workload": wl2.name, "T": wl2.T, "value": round(m2["tok_s"], 1), "unit": "tok/s per layer",
            "ms_per_step": round(m2["ms_per_step"], 4),
            "roofline": roofline_of(wl2, c2, m2, peaks),
            "layer": layer_line(c2, m2),
            "timing": m2["graph"],
            "stages_us": m2["stages_us"],
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
        out["oracle_baselines"] = [oracle_rate(gen.WORKLOADS[name], sec, ntok) for name, ntok, sec in ORACLE_SAMPLES]
        log(f"[bench] oracle baselines {json.dumps(out['oracle_baselines'])}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
