#!/usr/bin/env python3
"""Benchmark of the Mixtral sparse MoE feed-forward layer on one MI355X.

One step = one full layer forward (router + top-2 softmax, dispatch, expert
SwiGLU up/down, weighted combine) through the C ABI's moe_forward on inputs
already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--secondary A,B,..|none]
                    [--no-cpu-baseline]

The default workload is the Mixtral 8x7B layer in the decode regime (T = 16,
HBM-bound); the prefill layer (T = 4096), the Zipf-skewed layer (T = 16384)
and the 32-layer residual stack (T = 2048, one step = all 32 sublayers) are
measured too and reported under "secondary"; the small-T decode latency
sweep under "decode_latency"; the attention sublayer around the MoE (GQA with
RoPE at Mixtral widths, T = 4096) and a whole decoder layer under "attention";
one expert-parallel rank's share of the prefill layer (one local expert, 1024
rows, full width) under "ep_rank".  Per-kernel durations come from HIP events that
moe_forward records on its own stream between its kernels (timing points of
the C ABI); the roofline fraction is that of the dominant kernel.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-FFN layer tokens/s + % of MFMA/HBM roofline, Mixtral shapes, T=16/4096"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector, TFLOP/s
KERNELS = ["router", "dispatch", "expert_up", "expert_down", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_PROBE_BYTES = 1 << 30


def kernel_source(kernel: str, T: int) -> str:
    """Source file of the kernel that runs as `kernel` at T tokens (bf16)."""
    if kernel in ("expert_up", "expert_down"):
        return "expert_stream.hip" if T <= 64 else "expert_gemm.hip"
    return {"router": "router.hip", "dispatch": "dispatch.hip", "combine": "combine.hip",
            "flash_attn": "attention.hip"}[kernel]


# rocprofv3 kernel names -> step names
KERNEL_PATTERNS = [
    (r"stream_ffn_bf16_kernel<.*true>", "expert_up"), (r"stream_ffn_bf16_kernel<.*false>", "expert_down"),
    (r"gemm_bf16_kernel<true>", "expert_up"), (r"gemm_bf16_kernel<false>", "expert_down"),
    (r"router_top2_kernel", "router"), (r"dispatch_kernel", "dispatch"), (r"combine_kernel", "combine"),
    (r"flash_attn_fwd_kernel", "flash_attn"),
]
ATTN_WORKLOAD = "mixtral_attention_t4096"


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _event(hip):
    ev = ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(ev)) == 0
    return ev


def _elapsed_ms(hip, a, b) -> float:
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return float(ms.value)


def _code_only(text: str) -> str:
    """The source with comments removed (string and character literals kept)
    and runs of whitespace collapsed: what the compiler sees."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _src_sha(name: str) -> str:
    """Hash of a kernel source file's code (comments and layout ignored), so
    that counter entries stay valid across comment edits."""
    path = os.path.join(ROOT, "sparse_mixture_experts_wave_amd", "csrc", name)
    return hashlib.sha256(_code_only(open(path, encoding="utf-8").read()).encode()).hexdigest()[:16]


def _traffic(workload: str, kernel: str, T: int):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    absent or taken on a different version of the kernel's source."""
    try:
        entry = json.load(open(TRAFFIC_FILE))[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if entry.get("src_sha") != _src_sha(kernel_source(kernel, T)):
        return None
    return entry.get("bytes_per_launch")


def _counter_avgs(path: str):
    """Average counter value per (step name, counter) over the MoE kernels of a
    rocprofv3 counter_collection.csv."""
    import csv
    import re
    sums = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        for pat, step in KERNEL_PATTERNS:
            if re.search(pat, name):
                key = (step, r["Counter_Name"])
                tot, n = sums.get(key, (0.0, 0))
                sums[key] = (tot + float(r["Counter_Value"]), n + 1)
                break
    return {k: tot / n for k, (tot, n) in sums.items()}


def _copy_kib(path: str, counter: str) -> float:
    import csv
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
            return float(r["Counter_Value"])
    raise SystemExit(f"no copy kernel with {counter} in {path}")


def traffic_from(workload: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str, copy_write_csv: str):
    """Write profiles/traffic.json entries for `workload` from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) of the bench and of
    the copy probe (1 GiB read + 1 GiB written, which calibrates each counter)."""
    from synth import CONFIGS
    T, steps = (4096, ["flash_attn"]) if workload == ATTN_WORKLOAD else (CONFIGS[workload].T, KERNELS)
    f_scale = COPY_PROBE_BYTES / (_copy_kib(copy_fetch_csv, "FETCH_SIZE") * 1024)
    w_scale = COPY_PROBE_BYTES / (_copy_kib(copy_write_csv, "WRITE_SIZE") * 1024)
    fetch, write = _counter_avgs(fetch_csv), _counter_avgs(write_csv)
    try:
        out = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        out = {}
    entries = {}
    for step in steps:
        if (step, "FETCH_SIZE") not in fetch or (step, "WRITE_SIZE") not in write:
            continue
        rb = fetch[(step, "FETCH_SIZE")] * 1024 * f_scale
        wb = write[(step, "WRITE_SIZE")] * 1024 * w_scale
        entries[step] = {"bytes_per_launch": round(rb + wb), "read_bytes": round(rb), "write_bytes": round(wb),
                         "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                         "src_sha": _src_sha(kernel_source(step, T))}
    out[workload] = entries
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps({workload: entries}, indent=1))


def work_model(cfg, counts):
    """Algorithmic bytes and FLOPs per kernel launch (no padding, no re-reads)."""
    T, d, d_ff, E, k = cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k
    es = 2 if cfg.dtype == "bf16" else 4
    rows = T * k
    touched = int(sum(1 for c in counts if c > 0))
    up_bytes = touched * 2 * d_ff * d * es + T * d * es + rows * d_ff * es
    down_bytes = touched * d * d_ff * es + rows * d_ff * es + rows * d * 4
    return {
        "touched_experts": touched,
        "router": {"flops": 2 * T * d * E, "bytes": T * d * es + E * d * 4 + T * k * 8},
        "dispatch": {"flops": 0, "bytes": T * k * 4 * 3 + (E + 1) * 4},
        "expert_up": {"flops": 4 * rows * d * d_ff, "bytes": up_bytes},
        "expert_down": {"flops": 2 * rows * d * d_ff, "bytes": down_bytes},
        "combine": {"flops": 3 * rows * d, "bytes": rows * d * 4 + T * d * es + T * k * 8},
        "layer": {"flops": 6 * rows * d * d_ff + 2 * T * d * E,
                  "bytes": touched * 3 * d * d_ff * es + E * d * 4 + 2 * T * d * es},
    }


@contextlib.contextmanager
def _no_gc():
    """No Python garbage collection inside a timed region: a collection pass
    stalls the launching thread, and a region of a few milliseconds would
    count that stall as GPU time."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def measure(cfg, steps: int, warmup: int):
    """Time `steps` steps of the workload: one moe_forward call, or for a stack
    workload one moe_block_forward call per layer on a resident residual stream."""
    import numpy as np
    import torch

    import sparse_mixture_experts_wave_amd as moe
    from sparse_mixture_experts_wave_amd import _lib
    from synth import generate_torch

    lib = moe.load()
    hip = _hip()
    dev = torch.device("cuda:0")
    print(f"[bench] {cfg.name}: generating inputs ({cfg.layers} layer(s))", file=sys.stderr, flush=True)
    layers = [generate_torch(cfg, dev, layer=l) for l in range(cfg.layers)]
    x = layers[0]["x"]
    for lw in layers[1:]:
        del lw["x"]
    shape = moe.make_shape(cfg.T, cfg.d, cfg.d_ff, cfg.E, cfg.k, x.dtype)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device=dev)
    stack = cfg.layers > 1
    gamma = torch.ones(cfg.d, dtype=torch.float32, device=dev)
    y = x.clone() if stack else torch.empty_like(x)  # the stack's residual stream, updated in place

    def call(lw):
        if stack:
            moe.moe_block_forward(y, gamma, 1e-5, lw["w_gate"], lw["bias"], lw["w1"], lw["w3"], lw["w2"],
                                  workspace=ws)
        else:
            moe.moe_forward(x, lw["w_gate"], lw["bias"], lw["w1"], lw["w3"], lw["w2"], out=y, workspace=ws)

    def step():
        for lw in layers:
            call(lw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: K steps exactly as a caller runs them -> value.
    print(f"[bench] {cfg.name}: timing {steps} steps", file=sys.stderr, flush=True)
    with _no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        plain_ms = (time.perf_counter() - t0) * 1e3 / steps

    # Timed region 2: the same K steps with the C ABI timing points recording
    # HIP events on the launch stream between kernels -> per-kernel durations.
    npts = _lib.MOE_TIMING_POINTS
    evs = [[[_event(hip) for _ in range(npts)] for _ in layers] for _ in range(steps)]
    with _no_gc():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            for j, lw in enumerate(layers):
                arr = (ctypes.c_void_p * npts)(*[e.value for e in evs[i][j]])
                _lib.check(lib.moe_set_timing_events(arr, npts))
                call(lw)
        _lib.check(lib.moe_set_timing_events(None, 0))
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    calls = [e for per_step in evs for e in per_step]
    per_kernel = {name: statistics.fmean(_elapsed_ms(hip, e[j], e[j + 1]) for e in calls)
                  for j, name in enumerate(KERNELS)}
    for e in calls:
        for ev in e:
            hip.hipEventDestroy(ev)

    # Expert loads of the first layer (outside the timed regions).
    idx, _, _ = moe.moe_route(x, layers[0]["w_gate"], layers[0]["bias"])
    off, _, _ = moe.moe_dispatch(idx, cfg.E)
    counts = np.diff(off.cpu().numpy()).tolist()
    work = work_model(cfg, counts)
    return {
        "cfg": cfg, "inputs": layers[0] | {"x": x}, "layers": layers, "y": y, "ms_per_step": plain_ms,
        "ms_per_step_with_events": wall_ms, "per_kernel_ms": per_kernel, "counts": counts, "work": work,
    }


def measure_decode_latency(steps: int, Ts=(1, 2, 4, 8, 16)):
    """Per-step latency of the decode-regime layer for small T on the Mixtral
    decode weights, launched eagerly and replayed from a HIP graph that holds
    the whole moe_forward (router, dispatch, expert up/down, combine)."""
    import numpy as np
    import torch

    import sparse_mixture_experts_wave_amd as moe
    from synth import CONFIGS, generate_torch

    dev = torch.device("cuda:0")
    base = CONFIGS["mixtral_decode_t16"]
    dv = generate_torch(base, dev)
    out = []
    for T in Ts:
        cfg = base.with_(name=f"mixtral_decode_t{T}", T=T)
        x = generate_torch(cfg.with_(d_ff=64, E=2), dev)["x"]  # only x is used; seeded per T
        shape = moe.make_shape(T, cfg.d, cfg.d_ff, cfg.E, cfg.k, x.dtype)
        ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        args = (x, dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
        for _ in range(3):
            moe.moe_forward(*args, out=y, workspace=ws)
        with _no_gc():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                moe.moe_forward(*args, out=y, workspace=ws)
            torch.cuda.synchronize()
            eager_ms = (time.perf_counter() - t0) * 1e3 / steps
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            moe.moe_forward(*args, out=y, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            moe.moe_forward(*args, out=y, workspace=ws)
        for _ in range(3):
            g.replay()
        with _no_gc():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                g.replay()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - t0) * 1e3 / steps
        idx, _, _ = moe.moe_route(x, dv["w_gate"], dv["bias"])
        off, _, _ = moe.moe_dispatch(idx, cfg.E)
        counts = np.diff(off.cpu().numpy()).tolist()
        touched = sum(1 for c in counts if c > 0)
        wbytes = touched * 3 * cfg.d * cfg.d_ff * 2
        best = min(eager_ms, graph_ms)
        out.append({"T": T, "eager_us": round(eager_ms * 1e3, 1), "graph_us": round(graph_ms * 1e3, 1),
                    "tokens_per_s": round(T / (best * 1e-3), 1), "touched_experts": touched,
                    "weight_GBs": round(wbytes / (best * 1e-3) / 1e9, 1)})
        del g
    return out


def measure_ep_rank(steps: int, rows: int = 1024):
    """One expert-parallel rank's share of the prefill layer at full width.
    With expert e on GPU e, T = 4096 and top-2, a rank holds one expert and
    receives about 2T/8 = 1024 rows; its work is the grouped-GEMM expert FFN
    (up with the SiLU*gate epilogue, then down) on those rows.  Every row is
    routed to local expert 0; the layout carries a second, empty expert because
    the entry points take E >= 2."""
    import torch

    import sparse_mixture_experts_wave_amd as moe
    from synth import CONFIGS, generate_torch

    dev = torch.device("cuda:0")
    cfg = CONFIGS["mixtral_prefill_t4096"].with_(name="ep_rank_t4096", T=rows, E=2, k=1)
    dv = generate_torch(cfg, dev)
    off = torch.tensor([0, rows, rows], dtype=torch.int32, device=dev)
    st = torch.arange(rows, dtype=torch.int32, device=dev)
    y = torch.empty((rows, cfg.d), dtype=torch.float32, device=dev)
    args = (dv["x"], off, st, dv["w1"], dv["w3"], dv["w2"])
    for _ in range(3):
        moe.moe_expert_ffn(*args, k=1, y_sorted=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        moe.moe_expert_ffn(*args, k=1, y_sorted=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = 6.0 * rows * cfg.d * cfg.d_ff / (ms * 1e-3) / 1e12
    return {"workload": "ep_rank_t4096", "rows": rows, "d": cfg.d, "d_ff": cfg.d_ff, "local_experts": 1,
            "ms": round(ms, 4), "tflops": round(tflops, 1), "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def measure_attention(steps: int, T: int = 4096, d: int = 4096, H: int = 32, G: int = 8, dh: int = 128,
                      theta: float = 1e6):
    """The attention sublayer around the MoE at Mixtral 8x7B widths (32 query
    heads, 8 K/V groups, d_h = 128, rope_theta 1e6), one causal sequence of T
    tokens: the causal GQA core alone (moe_gqa_attention) and the whole
    sublayer h <- h + GQA(RMSNorm(h)) (moe_attention_block_forward), plus a
    full decoder layer = that sublayer followed by the MoE sublayer
    (moe_block_forward on the prefill workload's weights)."""
    import torch

    import sparse_mixture_experts_wave_amd as moe
    from synth import CONFIGS, attention_heads, attention_inputs, generate_torch

    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(a.view("int16")).to(dev).view(torch.bfloat16)

    inp = attention_inputs(T, d, H, G, dh)
    heads = attention_heads(T, H, G, dh)
    h0 = bf16(inp["h"])
    gamma = torch.from_numpy(inp["gamma"]).to(dev)
    wqkv, wo = bf16(inp["wqkv"]), bf16(inp["wo"])
    q, k, v = bf16(heads["q"]), bf16(heads["k"]), bf16(heads["v"])
    o = torch.empty_like(q)
    shape = moe.make_attn_shape(T, d, H, G, dh)
    ws = torch.empty(moe.attention_workspace_size(shape), dtype=torch.uint8, device=dev)
    h = h0.clone()

    # A short timed region straight after the GPU went idle reads high by a
    # fixed start-up cost (measured: the sublayer at 0.57-0.59 ms over 10
    # calls against 0.53 ms over 30 on the same GPU), so each timing warms up for
    # about 20 ms of work and times at least 30 calls (10 decoder layers).
    def timed(fn, n):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        for _ in range(max(1, int(0.02 / max(one, 1e-6)))):
            fn()
        with _no_gc():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / n

    steps = max(30, steps)
    core_ms = timed(lambda: moe.moe_gqa_attention(q, k, v, out=o), steps)
    sub_ms = timed(lambda: moe.moe_attention_block_forward(h, gamma, 1e-5, wqkv, wo, H, G, theta, 0, ws), steps)

    cfg = CONFIGS["mixtral_prefill_t4096"].with_(T=T)
    mw = generate_torch(cfg, dev)
    mshape = moe.make_shape(T, cfg.d, cfg.d_ff, cfg.E, cfg.k, torch.bfloat16)
    mws = torch.empty(moe.workspace_size(mshape), dtype=torch.uint8, device=dev)
    ones = torch.ones(cfg.d, dtype=torch.float32, device=dev)

    def layer():
        # Every step starts from the same residual stream (a 32 MiB device copy,
        # ~0.4 % of the step): applying the layer to its own output again and
        # again lets h drift and the routing with it.
        h.copy_(h0)
        moe.moe_attention_block_forward(h, gamma, 1e-5, wqkv, wo, H, G, theta, 0, ws)
        moe.moe_block_forward(h, ones, 1e-5, mw["w_gate"], mw["bias"], mw["w1"], mw["w3"], mw["w2"],
                              workspace=mws)

    layer_ms = timed(layer, max(10, steps // 3))
    core_flops = 2.0 * 2 * dh * H * T * (T + 1) / 2       # Q K^T and P V over the causal triangle
    proj_flops = 2.0 * T * d * (H + 2 * G) * dh + 2.0 * T * H * dh * d
    moe_flops = 6.0 * cfg.k * T * cfg.d * cfg.d_ff
    core_tf = core_flops / (core_ms * 1e-3) / 1e12
    return {
        "workload": f"mixtral_attention_t{T}", "T": T, "d": d, "H": H, "G": G, "d_h": dh, "rope_theta": theta,
        "core_ms": round(core_ms, 4), "sublayer_ms": round(sub_ms, 4),
        "sublayer_tokens_per_s": round(T / (sub_ms * 1e-3), 1),
        "sublayer_tflops": round((core_flops + proj_flops) / (sub_ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "kernel": "flash_attn", "achieved": round(core_tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(core_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic(ATTN_WORKLOAD, "flash_attn", T), "kernel_ms": round(core_ms, 4)},
        "decoder_layer": {"ms": round(layer_ms, 4), "tokens_per_s": round(T / (layer_ms * 1e-3), 1),
                          "tflops": round((core_flops + proj_flops + moe_flops) / (layer_ms * 1e-3) / 1e12, 2)},
    }


def roofline(res):
    cfg, work, pk = res["cfg"], res["work"], res["per_kernel_ms"]
    dom = max(("expert_up", "expert_down"), key=lambda n: pk[n])
    t = pk[dom] * 1e-3
    if cfg.T <= 64:  # decode regime: weight reads dominate
        achieved = work[dom]["bytes"] / t / 1e9
        peak, unit, bound = PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        achieved = work[dom]["flops"] / t / 1e12
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
        unit, bound = "TFLOP/s", "mfma"
    return {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": _traffic(cfg.name, dom, cfg.T),
            "kernel_ms": round(pk[dom], 4)}


def _host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS numpy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{dep.get('name', '?')} {dep.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        pass
    return model, blas


def _blas_threads():
    try:
        import threadpoolctl
        return max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _time_runs(fn, budget_s, min_runs=3, max_runs=50):
    """1 warm-up, then at least min_runs timed runs and more while within budget_s."""
    fn()
    times = []
    start = time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - start < budget_s and len(times) < max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), times


def _host(t):
    import numpy as np
    import torch

    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _oracle_leg(name, cfg, dv, n, budget_s, min_runs=3):
    """The expert-loop oracle (numpy fp32, BLAS sgemm per expert) on the first n
    tokens of a workload's inputs."""
    import oracle

    args = (_host(dv["x"][:n]), _host(dv["w_gate"]), _host(dv["bias"]), _host(dv["w1"]), _host(dv["w3"]),
            _host(dv["w2"]))
    print(f"[bench] cpu oracle on {n} tokens of {cfg.name}", file=sys.stderr, flush=True)
    med, times = _time_runs(lambda: oracle.moe_forward_expert_loop(*args), budget_s, min_runs)
    flops = 6 * cfg.k * n * cfg.d * cfg.d_ff + 2 * n * cfg.d * cfg.E
    return {"leg": name, "workload": cfg.name, "tokens": n, "tokens_per_s": round(n / med, 3),
            "gflops": round(flops / med / 1e9, 2), "median_s": round(med, 4), "runs": len(times),
            "seconds": round(sum(times), 1)}


def cpu_baseline(res, max_tokens: int, budget_s: float = 10.0, prefill_tokens: int = 256):
    """The CPU oracle on this host's cores, on bounded samples of the workloads.

    The reported value is the expert-loop oracle (numpy fp32) on the decode
    workload's tokens (tokens/s); further legs: the same oracle on the first
    prefill_tokens tokens of the prefill workload at full width, and the
    token-loop form (the definition, single BLAS thread) on the tiny fp32
    workload.  Each leg: 1 warm-up, then timed runs for about budget_s."""
    import numpy as np
    import torch

    import oracle
    from synth import CONFIGS, generate, generate_torch

    threads = _blas_threads()
    model, blas = _host_info()
    cfg, dv = res["cfg"], res["inputs"]
    legs = [_oracle_leg("expert-loop oracle, decode", cfg, dv, min(cfg.T, max_tokens), budget_s)]
    pcfg = CONFIGS["mixtral_prefill_t4096"]
    pdv = generate_torch(pcfg, torch.device("cuda"))
    legs.append(_oracle_leg("expert-loop oracle, prefill sample", pcfg, pdv, min(pcfg.T, prefill_tokens),
                            budget_s))
    del pdv
    torch.cuda.empty_cache()
    tcfg = CONFIGS["tiny_fp32"]
    tin = generate(tcfg)
    targs = (tin["x"], tin["w_gate"], tin["bias"], tin["w1"], tin["w3"], tin["w2"])
    print(f"[bench] cpu token-loop oracle on {tcfg.name}", file=sys.stderr, flush=True)
    try:
        import threadpoolctl
        limit = threadpoolctl.threadpool_limits(1)
    except Exception:  # noqa: BLE001
        limit = None
    med, times = _time_runs(lambda: oracle.moe_forward_token_loop(*targs), min(budget_s, 3.0))
    if limit is not None:
        limit.unregister()
    tflops = 6 * tcfg.k * tcfg.T * tcfg.d * tcfg.d_ff + 2 * tcfg.T * tcfg.d * tcfg.E
    legs.append({"leg": "token-loop oracle (the definition), 1 thread", "workload": tcfg.name, "tokens": tcfg.T,
                 "tokens_per_s": round(tcfg.T / med, 1), "gflops": round(tflops / med / 1e9, 3),
                 "median_s": round(med, 5), "runs": len(times), "seconds": round(sum(times), 1)})
    d0 = legs[0]
    return {"value": d0["tokens_per_s"], "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "gflops": d0["gflops"], "cpu_model": model, "blas": blas,
            "sample": f"{d0['tokens']} tokens of {cfg.name} (numpy fp32 expert-loop oracle, weights widened from "
                      f"bf16 inside), 1 warm-up + {d0['runs']} timed runs ({d0['seconds']} s), median "
                      f"{d0['median_s']} s; more legs under 'legs'",
            "legs": legs}


def summarize(res):
    cfg, work = res["cfg"], res["work"]
    ms = res["ms_per_step"]
    L = cfg.layers
    return {
        "workload": cfg.name, "T": cfg.T, "layers": L, "tokens_per_s": round(cfg.T / (ms * 1e-3), 2),
        "ms_per_step": round(ms, 4),
        "layer_tflops": round(L * work["layer"]["flops"] / (ms * 1e-3) / 1e12, 2),
        "layer_gbs": round(L * work["layer"]["bytes"] / (ms * 1e-3) / 1e9, 1),
        "roofline": roofline(res),
        "per_kernel_ms": {k: round(v, 4) for k, v in res["per_kernel_ms"].items()},
        "rows_per_expert": res["counts"], "touched_experts": work["touched_experts"],
        "ms_per_step_with_timing_events": round(res["ms_per_step_with_events"], 4),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral_decode_t16")
    ap.add_argument("--secondary", default="mixtral_prefill_t4096,mixtral_skewed_t16384,mixtral_stack32_t2048",
                    help="comma-separated workloads also measured and reported under 'secondary', or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true", help="skip the small-T decode latency sweep")
    ap.add_argument("--no-attention", action="store_true", help="skip the attention sublayer workload")
    ap.add_argument("--no-ep-rank", action="store_true", help="skip the expert-parallel rank workload")
    ap.add_argument("--attention-only", action="store_true",
                    help="measure only the attention sublayer workload and print its JSON")
    ap.add_argument("--cpu-tokens", type=int, default=16)
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json for --config from rocprofv3 --pmc CSVs (no GPU needed)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration for HBM traffic)")
    a = ap.parse_args()
    if a.traffic_from:
        traffic_from(a.config, *a.traffic_from)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} is not supported (the layer is built and "
              "measured on a single MI355X; multi-GPU sharding is a design note, not a run)", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if a.copy_probe:
        n = 1 << 28  # 1 GiB of fp32
        src = torch.empty(n, dtype=torch.float32, device="cuda")
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4}), flush=True)
        return
    if a.attention_only:
        print(json.dumps(measure_attention(a.steps)), flush=True)
        return
    cfg = CONFIGS[a.config]
    res = measure(cfg, a.steps, a.warmup)
    prim = summarize(res)
    cpu = None if a.no_cpu_baseline else cpu_baseline(res, a.cpu_tokens)
    del res
    sec = []
    for name in ([] if a.secondary in ("", "none") else a.secondary.split(",")):
        if name == a.config:
            continue
        torch.cuda.empty_cache()
        c2 = CONFIGS[name]
        r2 = measure(c2, max(3, a.steps // (4 if c2.layers > 1 else 2)), min(a.warmup, 2 if c2.layers > 1 else a.warmup))
        sec.append(summarize(r2))
        del r2
    latency = None
    if not a.no_latency:
        torch.cuda.empty_cache()
        print("[bench] decode latency sweep", file=sys.stderr, flush=True)
        latency = measure_decode_latency(a.steps)
    attention = None
    if not a.no_attention:
        torch.cuda.empty_cache()
        print("[bench] attention sublayer", file=sys.stderr, flush=True)
        attention = measure_attention(a.steps)
    ep_rank = None
    if not a.no_ep_rank:
        torch.cuda.empty_cache()
        print("[bench] expert-parallel rank share", file=sys.stderr, flush=True)
        ep_rank = measure_ep_rank(max(5, a.steps))
    out = {
        "metric": METRIC, "value": prim["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": prim["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded, Mixtral-shaped, random weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "d_ff": cfg.d_ff, "E": cfg.E, "k": cfg.k,
                   "parallelism": "single GPU"},
        "roofline": prim["roofline"], "cpu_baseline": cpu, "detail": prim, "secondary": sec,
        "decode_latency": latency, "attention": attention, "ep_rank": ep_rank,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
