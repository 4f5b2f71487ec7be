#!/usr/bin/env python3
"""Benchmark of the MI355X sparse MoE layer: decode tokens/s and % of HBM roofline.

Workload (default): real-shape decode with bf16 weights - hidden 2048, 512
routed experts, top-10 renormalized, expert intermediate 512, one shared
expert with a sigmoid gate, 1000 seeded tokens, one token per call, calls
back to back on one stream. A step is one pass of the 1000-token stream
through the layer. Dense weights (router, gate vector, shared expert) rotate
over 48 layer instances so they are re-read from HBM as in a 48-layer model;
the bf16 routed experts (3.2 GB, far beyond the 256 MB last-level cache) are
shared by the instances, while the 2-bit lines give every instance its own
copy of the routed stacks (48 x 604 MB). The calls are captured once into a
HIP graph and replayed; the timed region is K replays bracketed by device
synchronizations and HIP events on the replay stream (one event per step:
the median step is reported beside the mean).

Prints one JSON line. `roofline` covers the decode layer kernel(s):
algorithmic bytes per call (selected experts, shared expert, router, gate
vector, x, y, routing outputs) / measured time per call. `cpu_baseline` is
the plain double-precision CPU oracle on a bounded sample of the same tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


# ------------------------------------------------------------ byte models

def wbytes(fmt: str, rows: int, cols: int) -> int:
    if fmt == "f32":
        return rows * cols * 4
    if fmt == "bf16":
        return rows * cols * 2
    bits = {"q2": 2, "q3": 3, "q4": 4}[fmt]   # b-bit blocks: 4b bytes of codes + 4 of scale/min per 32 weights
    return rows * cols * (bits + 1) // 8


def expert_bytes(cfg) -> int:
    return 2 * wbytes(cfg.expert_t, cfg.I, cfg.H) + wbytes(cfg.expert_t, cfg.H, cfg.I)


def dense_bytes(cfg) -> int:
    return (wbytes(cfg.router_t, cfg.E, cfg.H) + wbytes(cfg.router_t, 1, cfg.H)
            + 2 * wbytes(cfg.shared_t, cfg.Is, cfg.H) + wbytes(cfg.shared_t, cfg.H, cfg.Is)
            + (cfg.E * 4 if cfg.bias_std > 0 else 0))


def call_bytes(cfg, rows: int, n_union: float) -> float:
    """Algorithmic bytes of one call: each distinct selected expert once, the
    dense weights once, x and y, and the routing outputs."""
    return (n_union * expert_bytes(cfg) + dense_bytes(cfg) + 2 * rows * cfg.H * 4
            + rows * (cfg.K * 8 + 4))


# ------------------------------------------------------------- workload

class Workload:
    """Device-resident layer instances, the token stream and a captured graph."""

    def __init__(self, cfg, rows_per_call: int, ncalls: int, rotate: int, x_instance: int = 0):
        import torch

        self.cfg, self.R, self.ncalls, self.rotate = cfg, rows_per_call, ncalls, rotate
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from _layers import gpu_layer_from_config
        self.dense0 = mi.dense_weights(cfg)
        self.stacks = mi.expert_stacks(cfg) if cfg.expert_t not in mi.BLOCK_FORMATS else None
        base = gpu_layer_from_config(cfg, self.dense0, self.stacks)
        self.layers = [base]
        # block-format stacks (604 MB at 2 bits) would partly stay in the
        # 256 MB last-level cache across calls: each instance gets its own copy
        self.distinct_experts = cfg.expert_t in mi.BLOCK_FORMATS and rotate > 1
        for i in range(1, rotate):
            d = mi.dense_weights(mi.layer_instance(cfg, i))
            L = base.with_dense(**d)
            self.layers.append(L.with_expert_copies() if self.distinct_experts else L)
        T = rows_per_call * ncalls
        self.x_host = mi.activations(cfg, T=T, instance=x_instance)
        self.x = torch.from_numpy(self.x_host).cuda()
        self.y = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((T, cfg.K), dtype=torch.int32, device="cuda")
        self.wts = torch.empty((T, cfg.K), dtype=torch.float32, device="cuda")
        self.gate = torch.empty((T,), dtype=torch.float32, device="cuda")
        self.ws = base.workspace(rows_per_call)
        self.graph = None

    def run_calls(self):
        import sparse_moe_decode_amd as moe
        R = self.R
        for c in range(self.ncalls):
            L = self.layers[c % self.rotate]
            s = slice(c * R, (c + 1) * R)
            moe.forward(L.desc, self.x[s], self.y[s], self.ws, ids_out=self.ids[s], wts_out=self.wts[s],
                        gate_out=self.gate[s])

    def capture(self):
        import torch
        self.run_calls()                       # eager pass (also warms up the code objects)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_calls()
        torch.cuda.synchronize()
        self.graph = g

    def step(self):
        self.graph.replay()

    def union_sizes(self):
        ids = self.ids.cpu().numpy().reshape(self.ncalls, self.R * self.cfg.K)
        return np.array([len(np.unique(r)) for r in ids], np.float64)


def time_steps(wl, steps: int, warmup: int, per_step: list | None = None):
    """Mean ms per step over `steps` graph replays (events on the replay
    stream); `per_step`, if given, receives each step's ms."""
    import torch
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        wl.step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / steps, wall


def call_latency(wl, n: int = 200):
    """Latency of one call (the first layer instance, one row group), from a
    graph of that single call replayed n times, each replay between two
    events; a long sleep kernel first lets the host queue every replay ahead
    of the GPU so that the intervals hold no host gaps. Returns microseconds
    (p50, p90, min)."""
    import torch
    import sparse_moe_decode_amd as moe
    R, L = wl.R, wl.layers[0]
    args = dict(ids_out=wl.ids[:R], wts_out=wl.wts[:R], gate_out=wl.gate[:R])
    moe.forward(L.desc, wl.x[:R], wl.y[:R], wl.ws, **args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(L.desc, wl.x[:R], wl.y[:R], wl.ws, **args)
    torch.cuda.synchronize()
    for _ in range(10):
        g.replay()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for i in range(n):
        ev[2 * i].record(stream)
        g.replay()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    us = np.sort([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(n)])
    return round(float(np.percentile(us, 50)), 3), round(float(np.percentile(us, 90)), 3), round(float(us[0]), 3)


def traffic_for(workload: str):
    """HBM bytes per call from committed rocprofv3 counter runs of this
    workload, if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec:
        return None
    if rec.get("source_sha") != source_sha():
        return None
    return rec.get("bytes_per_call")


def source_sha() -> str:
    from sparse_moe_decode_amd.profiling import source_sha as sha
    return sha()


# ---------------------------------------------------------- CPU baseline

def _oracle_rate(L, x_host, threads: int, seconds: float):
    """Tokens/s of the oracle on the token stream x_host (cycled) with the
    given OpenMP thread count, for about `seconds`."""
    import oracle
    oracle.set_threads(threads)
    threads = oracle.max_threads()
    done, chunk, n_tok = 0, 4 * threads, x_host.shape[0]
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        s0 = done % n_tok
        n = min(chunk, n_tok - s0)
        L.forward(x_host[s0:s0 + n])
        done += n
    dt = time.perf_counter() - t0
    return done, dt, threads


def cpu_baseline(wl, seconds: float, single_seconds: float):
    """The CPU oracle, as it stands, on the workload's token stream (cycled):
    with all available host cores (OpenMP over tokens) for about `seconds`,
    and on one thread for about `single_seconds`."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _layers import oracle_layer_from_config
    cfg = wl.cfg
    L = oracle_layer_from_config(cfg, dense=wl.dense0, stacks=wl.stacks)
    cores = len(os.sched_getaffinity(0))
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    n_tok = wl.x_host.shape[0]
    done, dt, threads = _oracle_rate(L, wl.x_host, cores, seconds)
    done1, dt1, _ = _oracle_rate(L, wl.x_host, 1, single_seconds)
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(done / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} tokens: the {n_tok}-token {cfg.name} stream (layer instance 0) cycled "
                      f"{done / n_tok:.1f} times, {dt:.1f} s, double-precision oracle, OpenMP over tokens; "
                      f"CPU: {cpu}",
            "single_thread": {"value": round(done1 / dt1, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"the first {done1} tokens of the same stream, {dt1:.1f} s, one thread"}}


# ------------------------------------------------------------------ main

def measure(cfg, rows, ncalls, rotate, steps, warmup, x_instance=0, per_step=None):
    wl = Workload(cfg, rows, ncalls, rotate, x_instance)
    wl.capture()
    ms, wall = time_steps(wl, steps, warmup, per_step)
    return wl, ms, wall


# (key, workload index, rows per call, calls, expert format if not the workload's)
EXTRA_WORKLOADS = [("decode_q2", 2, 1, 1000, None), ("fewrow_q2_R2", 3, 2, 500, None),
                   ("fewrow_q2_R3", 3, 3, 333, None), ("fewrow_q2_R8", 3, 8, 125, None),
                   ("prefill_q2", 4, 2048, 1, None),
                   ("decode_q3", 2, 1, 1000, "q3"), ("decode_q4", 2, 1, 1000, "q4"),
                   ("prefill_q3", 4, 2048, 1, "q3"), ("prefill_q4", 4, 2048, 1, "q4")]


def run_extra(args, keys):
    """The block-format decode, few-row and prefill workloads (all, or those in keys)."""
    import torch
    cfg = mi.CONFIGS[1]
    extra = {}
    for key, idx, rows, ncalls, fmt in EXTRA_WORKLOADS:
        if keys is not None and key not in keys:
            continue
        c = mi.CONFIGS[idx].with_(rows_per_call=rows)
        if fmt is not None:
            c = c.with_(expert_t=fmt, name=key)
        print(f"[bench] {key}", file=sys.stderr, flush=True)
        # one prefill call is about a millisecond: time more of them, after a
        # longer warm-up, so that clock ramp-up does not show in the figure
        steps, warm = (max(2, args.steps // 2), 1) if rows < 2048 else (max(20, args.steps), 5)
        per = []
        rot = args.rotate if rows < 2048 else 1
        w2, m2, _ = measure(c, rows, ncalls, rot, steps, warm, x_instance=rows if idx == 3 else 0, per_step=per)
        u = w2.union_sizes()
        per_call = m2 / 1e3 / ncalls
        rec = {"ms_per_step": round(m2, 4), "median_ms_per_step": round(float(np.median(per)), 4),
               "calls": ncalls, "rows_per_call": rows, "layer_instances": rot,
               "distinct_expert_stacks": rot if w2.distinct_experts else 1,
               "rows_per_s": round(rows * ncalls / (m2 / 1e3), 1), "us_per_call": round(per_call * 1e6, 3)}
        if rows < 2048:
            b = float(np.mean([call_bytes(c, rows, n) for n in u]))
            tr = traffic_for(key)
            rec.update({"bytes_per_call": round(b), "mean_expert_union": round(float(u.mean()), 3),
                        "GBps": round(b / per_call / 1e9, 1),
                        "hbm_frac": round(b / per_call / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic_bytes_per_call": tr,
                        "traffic_over_algorithmic": None if tr is None else round(tr / b, 4)})
            p50, p90, mn = call_latency(w2)
            rec.update({"hot_call_latency_us": {"p50": p50, "p90": p90, "min": mn}})
        else:
            tr = traffic_for(key)
            rec.update({"traffic_bytes_per_call": tr})
            flops = 2.0 * rows * (cfg.K * 3 * cfg.H * cfg.I + 3 * cfg.H * cfg.Is + cfg.E * cfg.H)
            rec.update({"useful_GFLOP": round(flops / 1e9, 2),
                        "TFLOPs": round(flops / per_call / 1e12, 2),
                        "mfma_frac": round(flops / per_call / 1e12 / BF16_PEAK_TFLOPS, 4)})
        extra[key] = rec
        del w2
        torch.cuda.empty_cache()
    return extra


class StackWorkload:
    """A 48-layer stack of 2-bit MoE layers as in the model (one per decoder
    layer): every layer with its own router, gate vector, shared expert,
    pre-MoE norm gamma and routed-expert copy, the RMS norm and the residual
    fused into the layer. Each token passes through all 48 layers, one call
    per layer (its input is the previous layer's output); the calls of all
    tokens are captured in one graph."""

    def __init__(self, cfg, tokens: int, n_layers: int = 48):
        import torch
        import sparse_moe_decode_amd as moe
        self.cfg, self.T, self.NL = cfg, tokens, n_layers
        d0 = mi.dense_weights(cfg)
        base = moe.Layer(H=cfg.H, E=cfg.E, K=cfg.K, I=cfg.I, Is=cfg.Is, router_t=cfg.router_t, expert_t=cfg.expert_t,
                         shared_t=cfg.shared_t, router_w=d0["router_w"], gate_vec=d0["gate_vec"],
                         router_bias=d0["router_bias"], sh_gate=d0["sh_gate"], sh_up=d0["sh_up"],
                         sh_down=d0["sh_down"], expert_source=lambda e, m: mi.expert_matrix_f32(cfg, e, m),
                         norm_w=mi.norm_weights(cfg, 0), norm_eps=1e-6, residual=1)
        self.layers = [base]
        for l in range(1, n_layers):
            d = mi.dense_weights(mi.layer_instance(cfg, l))
            self.layers.append(base.with_dense(**d, norm_w=mi.norm_weights(cfg, l)).with_expert_copies())
        x = mi.activations(cfg, T=tokens, instance=777)
        self.buf = [torch.from_numpy(x).cuda()] + [torch.empty((tokens, cfg.H), device="cuda")
                                                   for _ in range(n_layers)]
        self.ws = base.workspace(1)
        self.graph = None

    def run_calls(self):
        import sparse_moe_decode_amd as moe
        for t in range(self.T):
            for l, L in enumerate(self.layers):
                moe.forward(L.desc, self.buf[l][t:t + 1], self.buf[l + 1][t:t + 1], self.ws)

    def capture(self):
        import torch
        self.run_calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_calls()
        torch.cuda.synchronize()
        self.graph = g

    def step(self):
        self.graph.replay()


def run_stack(args):
    """Per-token decode through a 48-layer 2-bit stack (stack_q2_48)."""
    import torch
    cfg = mi.CONFIGS[2]
    print("[bench] stack_q2_48", file=sys.stderr, flush=True)
    tokens = 64
    wl = StackWorkload(cfg, tokens)
    wl.capture()
    per = []
    ms, _ = time_steps(wl, max(2, args.steps // 2), 1, per)
    calls = tokens * wl.NL
    per_call = ms / 1e3 / calls
    # algorithmic bytes of one layer call: as a decode call, plus gamma and the residual's x read
    b = call_bytes(cfg, 1, cfg.K) + cfg.H * 4 * 2
    rec = {"ms_per_step": round(ms, 4), "median_ms_per_step": round(float(np.median(per)), 4), "tokens": tokens,
           "layers": wl.NL, "distinct_expert_stacks": wl.NL, "tokens_per_s": round(tokens / (ms / 1e3), 1),
           "ms_per_token": round(ms / tokens, 4), "us_per_layer_call": round(per_call * 1e6, 3),
           "bytes_per_layer_call": round(b), "GBps": round(b / per_call / 1e9, 1),
           "hbm_frac": round(b / per_call / 1e9 / HBM_PEAK_GBS, 4), "traffic_bytes_per_call": traffic_for("stack_q2_48")}
    del wl
    torch.cuda.empty_cache()
    return {"stack_q2_48": rec}


def rows_sweep(args):
    """Throughput of calls of R rows on the 2-bit layer: one decode row, the
    few-row path up to 4 rows, the grouped prefill path above (the crossover
    of the two). Calls take consecutive rows of one 2048-row stream."""
    cfg = mi.CONFIGS[3].with_(rows_per_call=1)
    total = 2048
    print("[bench] rows sweep", file=sys.stderr, flush=True)
    wl = Workload(cfg, 1, total, 1)
    out = {}
    for R in (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 13, 16, 24, 32, 64, 256, 2048):
        wl.R = R
        wl.ncalls = max(1, min(total // R, 256))
        wl.ws = wl.layers[0].workspace(R)
        wl.capture()
        ms, _ = time_steps(wl, max(2, args.steps // 2), 1)
        per_call = ms / 1e3 / wl.ncalls
        # the library's choice for this layer (4-row launches fit its shapes)
        out[str(R)] = {"path": "decode" if R == 1 else ("few-row" if R <= 12 else "prefill"),
                       "calls": wl.ncalls, "us_per_call": round(per_call * 1e6, 3),
                       "rows_per_s": round(R / per_call, 1)}
    return {"workload": "rows_sweep", "config": cfg.name, "rows": out}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rotate", type=int, default=48, help="layer instances for the dense weights")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle on all host cores")
    ap.add_argument("--cpu-single-seconds", type=float, default=8.0, help="oracle on one thread")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 2-bit, few-row and prefill lines")
    ap.add_argument("--only", choices=[k for k, *_ in EXTRA_WORKLOADS] + ["stack_q2_48"],
                    help="run just this one of the other workloads (for profiling); prints its record")
    ap.add_argument("--rows-sweep", action="store_true",
                    help="rows per call from 1 to 2048 on the 2-bit layer (decode, few-row, prefill paths); "
                         "prints one record of rows/s per call size")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's kernels run on "
              f"one MI355X; several GPUs would shard experts with one all-reduce of y, not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_moe_decode_amd as moe
    moe.lib()                                     # fails loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.rows_sweep:
        print(json.dumps(rows_sweep(args)), flush=True)
        return
    if args.only:
        extra = run_stack(args) if args.only == "stack_q2_48" else run_extra(args, [args.only])
        print(json.dumps({"workload": args.only, **extra[args.only]}), flush=True)
        return

    cfg = mi.CONFIGS[1]
    print(f"[bench] building {cfg.name} workload, {args.rotate} dense-weight instances", file=sys.stderr, flush=True)
    per_step = []
    wl, ms, wall = measure(cfg, 1, cfg.T, args.rotate, args.steps, args.warmup, per_step=per_step)
    tokens = cfg.T
    tok_s = tokens / (ms / 1e3)
    per_call_s = ms / 1e3 / tokens
    bytes_call = call_bytes(cfg, 1, cfg.K + 0.0)
    achieved = bytes_call / per_call_s / 1e9
    print(f"[bench] {cfg.name}: {ms:.3f} ms/step, {tok_s:.0f} tok/s, {achieved:.0f} GB/s", file=sys.stderr,
          flush=True)

    p50, p90, mn = call_latency(wl)
    extra = {"decode_bf16_timing": {
        "median_ms_per_step": round(float(np.median(per_step)), 4),
        "min_ms_per_step": round(float(np.min(per_step)), 4), "max_ms_per_step": round(float(np.max(per_step)), 4),
        "hot_call_latency_us": {"p50": p50, "p90": p90, "min": mn,
                                "how": "one call captured alone and replayed 200 times (its weights may stay "
                                       "in the last-level cache between replays)"}}}
    if args.rotate != 1:
        wl1, ms1, _ = measure(cfg, 1, 200, 1, args.steps, args.warmup)
        extra["decode_bf16_single_instance"] = {
            "tokens_per_s": round(200 / (ms1 / 1e3), 1),
            "us_per_token": round(ms1 * 1e3 / 200, 3),
            "GBps": round(call_bytes(cfg, 1, cfg.K) / (ms1 / 1e3 / 200) / 1e9, 1)}
        del wl1

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds, args.cpu_single_seconds)
    del wl
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra.update(run_extra(args, None))
        extra.update(run_stack(args))

    line = {
        "metric": "MoE-layer decode tokens/s and % of HBM roofline (expert bytes read/s)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bf16: Qwen3-Next-shape MoE layer, hidden 2048, 512 experts, top-10, "
                               "inter 512, shared expert 512 + sigmoid gate, bf16 weights, fp32 activations; "
                               "1000 tokens, 1 token per call",
                   "global_batch": 1, "seq_len": 1, "tokens_per_step": tokens,
                   "dense_weight_instances": args.rotate, "timing": "HIP graph replay of 1000 calls"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(cfg.name),
                     "bytes_per_call": bytes_call, "us_per_call": round(per_call_s * 1e6, 3)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
