#!/usr/bin/env python3
"""Benchmark of the fused RoPE attention core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
    python bench.py --only CONFIG      # one configuration, one short line (for profiling)

One step = one call of the whole core (RoPE on Q/K, QK^T, FP32 online softmax, P.V)
over one batch of synthetic input already resident in HBM: at the long latent that is
two kernels, the pre-pass (RoPE of K, fp16 V^T tiles into a workspace allocated once
before timing) and the attention kernel. The headline workload
is the DiT long latent: B=2 (a CFG cond + uncond pair), H=24, L=4096, D=64, bf16 with
1% of K rows scaled by 8, full attention, FP32 output. Rank 0 prints ONE JSON line with
the metric (TFLOP/s of algorithmic work, 4*D FLOPs per query-key pair), the roofline of
the kernel against the MI355X dense bf16 MFMA peak, the CPU oracle timed on the host
cores as a baseline, and ms/call + TFLOP/s of every other synthetic configuration.

Timing: W untimed warmups (and at least 0.3 s of calls, so the clocks settle), then K
back-to-back calls bracketed by synchronisation and timed with one pair of HIP events
recorded on the stream the library launches on (torch's current stream, which the
binding passes to the C-ABI): ms_per_step is their mean. A second pass gives each call
its own event pair; its median, min and max are reported as the spread. In that pass a
call with the pre-pass is issued as its two kernels (policies "only" then "reuse") with
an event between them: the roofline uses the attention kernel's own mean duration.

After the timed region, 0.5 s more of headline calls run while a thread reads the
shader clock (pp_dpm_sclk of the one card) every 10 ms: its median gives the peak at the
clock the kernel actually ran at, next to the 2400 MHz figure.

Short latents: per-call time inside one captured graph of 96 and of 40 calls (the
number of fused attention calls in a medium / small DiT forward) at L = 1, 16, 64, 256,
next to the same figure for a trivial one-element kernel (the launch floor).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense FP16/BF16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
WARM_S = 0.3                 # minimum warmup time per timed configuration
HEAD_CONFIG = "dit_long"
OTHER_CONFIGS = ["tiny", "dit_short", "dit_2min", "dit_2min_prime", "samel_swa", "samel_w17", "dit_medium_diff",
                 "dit_long_d128"]
COLD_CONFIGS = {"tiny", "dit_short", "samel_swa", "samel_w17"}   # HBM/latency-bound: also timed cold
FLUSH_MB = 512                     # larger than the 256 MB MALL plus the L2s
GRAPH_LENGTHS = [1, 16, 64, 256]   # short-latent sequences captured as one graph of N calls
GRAPH_CALLS = [96, 40]             # fused attention calls per forward: medium and small DiT
KERNEL_SOURCES = [os.path.join(ROOT, "rope_attention_core_amd", "csrc", f) for f in ("attn_fwd.hip", "attn_common.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dit_long.json")


def pairs(cfg):
    """In-window (query, key) pairs per branch."""
    L, w = cfg.L, cfg.window
    per_head = L * L if (w < 0 or w >= L - 1) else L * (2 * w + 1) - w * (w + 1)
    return cfg.B * cfg.H * per_head


def flops(cfg):
    return 4 * cfg.D * pairs(cfg) * (2 if cfg.diff else 1)


def compulsory_bytes(cfg):
    n = cfg.B * cfg.H * cfg.L * cfg.D
    qk = 2 * n * 2 * (2 if cfg.diff else 1)
    v = 2 * n
    out = n * (4 if cfg.out_dtype == "f32" else 2)
    table = 2 * cfg.L * (cfg.D // 2) * 4
    return qk + v + out + table


def exps(cfg):
    """Softmax exponentials of the definition: one per in-window pair and branch."""
    return pairs(cfg) * (2 if cfg.diff else 1)


def sclk_file():
    """The shader-clock file of the one visible card (None unless exactly one exists)."""
    import glob
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    return files[0] if len(files) == 1 else None


def read_sclk_mhz(path):
    """Current shader clock: the line of pp_dpm_sclk marked with '*'."""
    with open(path) as f:
        for ln in f:
            if "*" in ln:
                tok = ln.split(":", 1)[1].strip().split()[0].lower()
                return float(tok.replace("mhz", ""))
    return None


def sample_clock(torch, bench, seconds=0.5):
    """Median shader clock while the headline call runs back to back for `seconds`
    (after the timed region, so the sampling thread does not touch it)."""
    import statistics
    import threading
    path = sclk_file()
    if path is None:
        return None
    vals, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                v = read_sclk_mhz(path)
            except OSError:
                v = None
            if v is not None:
                vals.append(v)
            stop.wait(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(8):
            bench.call()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return None
    return {"sclk_mhz_median": statistics.median(vals), "sclk_mhz_min": min(vals), "sclk_mhz_max": max(vals),
            "samples": len(vals), "source": os.path.basename(os.path.dirname(os.path.dirname(path))) +
            "/device/pp_dpm_sclk, sampled every 10 ms during 0.5 s of headline calls after the timed region"}


def kernel_source_sha():
    """sha256 over the attention kernel's sources (the counters hold while they are unchanged)."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic():
    """HBM bytes per launch from rocprofv3 counters, if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


class Bench:
    def __init__(self, torch, sa3, synth, cfg):
        import numpy as np
        self.torch, self.sa3, self.cfg = torch, sa3, cfg
        inp = synth.make_inputs(cfg)

        def dev(a):
            if cfg.io == "f16":
                return torch.from_numpy(np.ascontiguousarray(a)).cuda()
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

        self.q, self.k, self.v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
        c, s = sa3.rope_table(cfg.L, cfg.D, cfg.base)
        self.cos, self.sin = c.cuda(), s.cuda()
        dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[cfg.out_dtype]
        self.out = torch.empty((cfg.B, cfg.H, cfg.L, cfg.D), dtype=dt, device="cuda")
        self.inputs_host = inp
        # the pre-pass workspace (allocated once, outside every timed region), when the
        # library runs the pre-pass for this shape
        nb = sa3.workspace_bytes(cfg.B, cfg.H, cfg.L, cfg.D, window=cfg.window, differential=cfg.diff,
                                 dtype=sa3.BF16 if cfg.io == "bf16" else sa3.F16)
        self.ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None

    def call(self, prep="auto"):
        c = self.cfg
        self.sa3.forward(self.q, self.k, self.v, self.cos, self.sin, window=c.window, lam=c.lam,
                         scale=c.scale, out=self.out, differential=c.diff, prep=prep, workspace=self.ws)

    def run(self, steps, warmup):
        """Time `steps` back-to-back calls between two HIP events on the launch stream,
        bracketed by device synchronisation (the headline ms/call), then the same number
        of calls again, each between its own pair of events, for the spread. With the
        pre-pass, each call of the second pass is split into its two kernels (the
        pre-pass alone, then the attention kernel alone on its workspace) with an event
        between them, which gives each kernel's own average duration."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        # W warmup calls, and calls for at least WARM_S seconds, so the clocks have
        # settled under this load before the timed region starts
        n, t_end = 0, time.perf_counter() + WARM_S
        while n < warmup or time.perf_counter() < t_end:
            for _ in range(max(1, warmup)):
                self.call()
            torch.cuda.synchronize()
            n += max(1, warmup)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t0.record(stream)
        for _ in range(steps):
            self.call()
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total = t0.elapsed_time(t1)
        split = self.ws is not None
        ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
        for a, m, b in ev:
            a.record(stream)
            if split:
                self.call(prep="only")
                m.record(stream)
                self.call(prep="reuse")
            else:
                self.call()
                m.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) for a, m, b in ev)
        attn = sum(m.elapsed_time(b) for a, m, b in ev) / steps if split else None
        prep = sum(a.elapsed_time(m) for a, m, b in ev) / steps if split else None
        return {"ms_total": total, "ms_mean": total / steps, "ms_median": per[len(per) // 2],
                "ms_min": per[0], "ms_max": per[-1], "wall_s": wall,
                "ms_attn_kernel": attn if split else sum(per) / steps, "ms_prep_kernel": prep}


def cold_ms(torch, b, reps=7):
    """Median ms of single calls, each after writing a FLUSH_MB buffer so that no input
    is left in the L2s or the MALL (the flush is outside the timed event pair)."""
    flush = torch.empty(FLUSH_MB * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    return sorted(times)[len(times) // 2]


def graph_per_call_us(torch, fn, n_calls, replays=20):
    """Capture n_calls of fn() into one graph; time replays back to back; us per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_calls):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (replays * n_calls)


def prepared_loop_us(torch, sa3, b, calls=200):
    """us per call of back-to-back eager calls through a PreparedCall (sa3.prepare), whose
    host cost is one C-ABI call: between two HIP events, after 20 warmup calls."""
    c = b.cfg
    call = sa3.prepare(b.q, b.k, b.v, b.cos, b.sin, window=c.window, lam=c.lam, scale=c.scale, out=b.out,
                       differential=c.diff, workspace=b.ws)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        call()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / calls


def short_graphs(torch, sa3, synth):
    """Short-latent regime: per-call time of the fused core in a loop of 100 eager calls
    (through forward(), and through a PreparedCall) and inside one captured graph of
    96 / 40 calls, next to the per-launch floor of a trivial kernel (a one-element add)
    captured the same way."""
    x = torch.zeros(1, device="cuda")
    res = {"launch_floor_graph_us": round(graph_per_call_us(torch, lambda: x.add_(1.0), 96), 3)}
    for L in GRAPH_LENGTHS:
        cfg = synth.config("dit_short", L=L)
        b = Bench(torch, sa3, synth, cfg)
        r = b.run(100, 5)
        ent = {"shape": f"B{cfg.B} H{cfg.H} L{L} D{cfg.D} {cfg.io}",
               "eager_loop_us_per_call": round(r["ms_mean"] * 1e3, 3),
               "eager_prepared_us_per_call": round(prepared_loop_us(torch, sa3, b), 3)}
        for n in GRAPH_CALLS:
            ent[f"graph{n}_us_per_call"] = round(graph_per_call_us(torch, b.call, n), 3)
        ent["gbs_compulsory_graph96"] = round(compulsory_bytes(cfg) / (ent["graph96_us_per_call"] * 1e-6) / 1e9, 1)
        res[f"L{L}"] = ent
        del b
    return res


def cpu_baseline(cfg, inputs, budget_s=12.0):
    """Time the fp64 oracle (method mode) on whole heads of the same workload."""
    import numpy as np

    import oracle
    from threadpoolctl import threadpool_info

    q = oracle.widen_io(inputs["q"], cfg.io)
    k = oracle.widen_io(inputs["k"], cfg.io)
    v = oracle.widen_io(inputs["v"], cfg.io)
    c32, s32 = oracle.rope_table_f32(cfg.L, cfg.D, cfg.base)
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    # whole heads in order, over the heads again while the budget lasts (one pass over
    # every head of a call can take only a few seconds)
    done, t_used = 0, 0.0
    for i in range(len(heads) * 64):
        b, h = heads[i % len(heads)]
        sl = (slice(b, b + 1), slice(h, h + 1))
        t = time.perf_counter()
        if cfg.diff:
            oracle.attn_method(q[0][sl], k[0][sl], v[sl], c32, s32, cfg.io, cfg.scale, window=cfg.window,
                               lam=cfg.lam, q2=q[1][sl], k2=k[1][sl])
        else:
            oracle.attn_method(q[sl], k[sl], v[sl], c32, s32, cfg.io, cfg.scale, window=cfg.window)
        t_used += time.perf_counter() - t
        done += 1
        if t_used >= budget_s:
            break
    per_head_flops = flops(cfg) / (cfg.B * cfg.H)
    info = threadpool_info()
    threads = max((p.get("num_threads", 1) for p in info), default=1)
    blas = ",".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in info})) or "none"
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(per_head_flops * done / t_used / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} head calls over the {len(heads)} (b,h) heads of {cfg.name} "
                  f"({done / len(heads):.2g} passes), full output, numpy fp64 method mode; "
                  f"{t_used:.1f} s; ms/call extrapolated {t_used / done * len(heads) * 1e3:.0f}",
        "cpu": cpu_model,
        "blas": blas,
    }


def copy_reference(torch, mb):
    """Three plain device copies of mb MiB: a known-size reference for the HBM counters."""
    if mb <= 0:
        return
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_read": n * 4, "copy_reference_bytes_written": n * 4,
                      "copies": 3}), file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config lines")
    ap.add_argument("--only", metavar="CONFIG", default=None,
                    help="time just this synthetic configuration and print one short JSON line "
                         "(for profiling the kernel another configuration runs)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after the benchmark, run 3 plain device copies of this many MiB "
                         "(a known-size reference for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the fused core shards by "
                                   "(batch, head) with no exchange, so a multi-GPU figure adds "
                                   "nothing here; run with --gpus 1"}))
        sys.exit(2)

    import torch

    import rope_attention_core_amd as sa3
    from rope_attention_core_amd import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    sa3.load_library()
    torch.cuda.set_device(0)

    if args.only:
        c = synth.config(args.only)
        r = Bench(torch, sa3, synth, c).run(args.steps, args.warmup)
        f = flops(c)
        print(json.dumps({"config": args.only, "ms_per_call": round(r["ms_mean"], 5),
                          "ms_attn_kernel": round(r["ms_attn_kernel"], 5),
                          "ms_prep_kernel": None if r["ms_prep_kernel"] is None else round(r["ms_prep_kernel"], 5),
                          "tflops": round(f / (r["ms_mean"] * 1e-3) / 1e12, 2),
                          "gbs_compulsory": round(compulsory_bytes(c) / (r["ms_mean"] * 1e-3) / 1e9, 1)}),
              flush=True)
        copy_reference(torch, args.copy_mb)
        return

    cfg = synth.config(HEAD_CONFIG)
    bench = Bench(torch, sa3, synth, cfg)
    t = bench.run(args.steps, args.warmup)
    fl = flops(cfg)
    ms = t["ms_mean"]
    tflops = fl / (ms * 1e-3) / 1e12
    k_tflops = fl / (t["ms_attn_kernel"] * 1e-3) / 1e12   # the attention kernel alone
    traffic = load_traffic()
    clock = sample_clock(torch, bench)
    if clock is not None:
        # the peak scales with the clock: 2516.6 TFLOP/s is quoted at 2400 MHz
        at_clk = PEAK_BF16_TFLOPS * clock["sclk_mhz_median"] / 2400.0
        clock["peak_tflops_at_clock"] = round(at_clk, 1)
        clock["attn_kernel_frac_at_clock"] = round(k_tflops / at_clk, 4) if at_clk > 0 else None

    per_config = {}
    if not args.no_configs:
        for name in OTHER_CONFIGS:
            c = synth.config(name)
            b = Bench(torch, sa3, synth, c)
            r = b.run(max(10, args.steps), 3)
            f = flops(c)
            per_config[name] = {
                "shape": f"B{c.B} H{c.H} L{c.L} D{c.D} {c.io}" + (f" w={c.window}" if c.window >= 0 else "")
                         + (f" diff lam={c.lam}" if c.diff else "") + f" out={c.out_dtype}",
                "ms_per_call": round(r["ms_mean"], 5),
                "ms_median": round(r["ms_median"], 5),
                "prep": r["ms_prep_kernel"] is not None,
                "tflops": round(f / (r["ms_mean"] * 1e-3) / 1e12, 2),
                "frac_mfma_peak": round(f / (r["ms_mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "gbs_compulsory": round(compulsory_bytes(c) / (r["ms_mean"] * 1e-3) / 1e9, 1),
                "gexp_per_s": round(exps(c) / (r["ms_mean"] * 1e-3) / 1e9, 1),
            }
            if name in COLD_CONFIGS:
                cm = cold_ms(torch, b)
                per_config[name]["ms_cold_median"] = round(cm, 5)
                per_config[name]["gbs_compulsory_cold"] = round(compulsory_bytes(c) / (cm * 1e-3) / 1e9, 1)
            del b
        torch.cuda.empty_cache()
    graphs = None if args.no_configs else short_graphs(torch, sa3, synth)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, bench.inputs_host)
        # the whole GPU step's rate over the oracle's, on the same workload
        cpu["gpu_over_oracle"] = round(tflops / cpu["value"], 1) if cpu["value"] > 0 else None

    line = {
        "metric": "attention-core TFLOP/s at L=4096 (DiT long latent, fused RoPE attention)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.io,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} L={cfg.L} D={cfg.D} bf16 q/k/v ~ N(0,1), "
                        f"1% of K rows x8, RoPE base 10000 (fp32 table), full attention, scale 1/8, fp32 out",
            "B": cfg.B, "H": cfg.H, "L": cfg.L, "D": cfg.D, "window": cfg.window, "out_dtype": cfg.out_dtype,
            "gflop_per_call": round(fl / 1e9, 3),
            "parallelism": "single GPU",
        },
        "ms_median": round(t["ms_median"], 5),
        "ms_min": round(t["ms_min"], 5),
        "ms_max": round(t["ms_max"], 5),
        "frac_of_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "gexp_per_s": round(exps(cfg) / (ms * 1e-3) / 1e9, 1),
        "clock": clock,
        "kernels_per_step": {
            "attn_prep_kernel_ms": None if t["ms_prep_kernel"] is None else round(t["ms_prep_kernel"], 5),
            "attn_fwd_kernel_ms": round(t["ms_attn_kernel"], 5),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel",
            "achieved": round(k_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(k_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "per_config": per_config,
        "short_graphs": graphs,
    }
    print(json.dumps(line), flush=True)

    copy_reference(torch, args.copy_mb)

if __name__ == "__main__":
    main()
