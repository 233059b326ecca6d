"""Benchmark of the 2:4 sparse GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload all|up|down|prefill|layers|slide|palette]

Default (--workload all): the whole metric, decode and prefill, in one JSON line.
  * The headline step (value, ms_per_step, roofline, cpu_baseline) is the
    decode-shaped FP8 FFN up-projection (K=4096, N=14336) at M = 1, 16 and 64
    tokens: one step = sp24_gemm_qx for each M (dynamic per-tensor E4M3
    quantisation of X and the sparse GEMM, including any split-K reduction) on
    weights pruned, compressed and quantised once at load.
  * "configs" holds every configuration of the metric, each with its own
    roofline fraction, dense-MFMA baseline and per-call p50/p99:
      up      -- the same up-projection per M (sparse GEMM, quantise + GEMM, dense
                 MFMA, hipBLASLt's dense FP8 as a reference);
      down    -- the down-projection (K=14336, N=4096) per M, which splits K;
      prefill -- M=8192, K=8192, N=28672 (bound: matrix cores), with the CPU
                 oracle timed on a slice;
      layers  -- 32 layers x (QKV, O, gate+up, down) at M=256, 128 sequential
                 sparse GEMMs per step, and the same sweep on dense MFMA.
--workload up|down|prefill|layers prints the line of that configuration alone
(the form the profiles are taken with); slide and palette measure the
SlideSparse 6:8 and exponent-palette variants.
--dtype int8: up, down or prefill with symmetric per-tensor INT8 codes (the
cookbook's INT8 W8A8 recipe); bf16: BF16 operands (no scales).

Inputs are seeded synthetic tensors (workloads/) resident in HBM before the
timed region.  At decode each call reads a different one of R weight copies
(> 2x the 256 MB last-level cache), so weight bytes come from HBM.  Steps are
captured once per weight copy in HIP graphs and replayed; the graphs' outputs
are checked bitwise against an eager run.  Kernel times are HIP events on the
stream the library launches on (torch's current stream); p50/p99 come from an
event pair around each of many calls.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse GEMM TFLOP/s + GB/s and % of roofline vs dense MFMA, decode & prefill"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
# MFMA peaks of MI355X from its unit counts and clock: 256 CUs x 2.4 GHz x dense flop per
# clock per CU (FP8 and INT8 8192, BF16 4096).  SMFMAC performs as many nonzero
# multiply-adds per clock as dense MFMA, so a 2:4 kernel is priced in nonzero MACs x 2 per
# second against these, which equals dense-equivalent flops against twice these (the
# sparse FP8 peak 10,066 TFLOP/s).
N_CU, CLOCK_HZ = 256, 2.4e9
FP8_DENSE_PEAK_TFLOPS = N_CU * 8192 * CLOCK_HZ / 1e12   # 5033.2 (INT8: the same in TOP/s)
BF16_DENSE_PEAK_TFLOPS = N_CU * 4096 * CLOCK_HZ / 1e12  # 2516.6
PEAK_SOURCE = "256 CUs x 2.4 GHz x 8192 (FP8/INT8) or 4096 (BF16) dense flop/clk/CU"
LLC_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all",
                    choices=["all", "up", "down", "prefill", "layers", "slide", "palette", "groups"])
    ap.add_argument("--dtype", default="fp8", choices=["fp8", "int8", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-percentiles", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=0,
                    help="GEMM launches per M for the per-kernel timing (0: automatic)")
    return ap.parse_args()


_CSRC = "bf16_gemm_linear_amd/csrc/"
KERNEL_NAMES = {0: "gemm_skinny_kernel", 1: "gemm_tiled_kernel", 2: "gemm_stream_kernel"}
KERNEL_SOURCES = {  # the dominant kernel's sources and the plan that picks its configuration
    "hbm": [_CSRC + f for f in ("sp24_gemm_stream.hip", "sp24_dma.hpp", "sp24_common.hpp",
                                "sp24_internal.hpp", "sp24_api.hip")],
    "mfma": [_CSRC + f for f in ("sp24_gemm_tiled.hip", "sp24_dma.hpp", "sp24_common.hpp",
                                 "sp24_internal.hpp", "sp24_api.hip")],
    # the layer sweep: stream and tiled kernels (both tile shapes) and the split-K reduction
    "sweep": [_CSRC + f for f in ("sp24_gemm_stream.hip", "sp24_gemm_tiled.hip", "sp24_gemm_tiled128.hip",
                                  "sp24_reduce.hip", "sp24_dma.hpp", "sp24_common.hpp", "sp24_internal.hpp",
                                  "sp24_api.hip")],
}


def counted_traffic(workload, bound):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summaries (profiles/*.md, FETCH_SIZE and WRITE_SIZE scaled by a copy of known size),
    or None when no summary matches the current kernel source."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[bound]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    digest = h.hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("workload") == workload and rec.get("kernel_source_sha256") == digest:
                        return rec["traffic_bytes_per_launch"]
    return None


def gemm_bytes(m, n, k, fp8):
    """Algorithmic bytes of one sparse GEMM: compressed values + metadata + X + Y."""
    es = 1 if fp8 else 2
    return n * (k // 2) * es + n * (k // 32) * 4 + m * k * es + m * n * 2


def dense_bytes(m, n, k, fp8):
    es = 1 if fp8 else 2
    return n * k * es + m * k * es + m * n * 2


def quant_bytes(m, k):
    return m * k * 2 + m * k + 4


def n_copies(nbytes):
    """Weight copies a decode call rotates over so that its weight comes from HBM."""
    import math
    return max(2, min(16, int(math.ceil(2.2 * LLC_BYTES / nbytes))))


class Events:
    """HIP events on the current (torch) stream, which is the stream libsp24 launches on."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, reps):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        s.record()
        for i in range(reps):
            fn(i)
        e.record()
        e.synchronize()
        return s.elapsed_time(e) / 1e3  # seconds

    def graph(self, fn, reps, replays=3):
        """Mean seconds per call of fn(0) .. fn(reps - 1), captured once in a HIP graph and
        replayed (launch-free back-to-back calls)."""
        t = self.torch
        fn(0)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        t.cuda.synchronize()
        sec = self.time(lambda i: g.replay(), replays) / replays / reps
        del g
        return sec

    def percentiles(self, fn, calls, warm=3):
        """Per-call duration (us) from an event pair around each of `calls` calls: p50, p99,
        mean.  A spin kernel first keeps the GPU busy so that the host enqueues every call
        ahead of it and no launch gap falls inside a pair."""
        t = self.torch
        for i in range(warm):
            fn(i)
        t.cuda.synchronize()
        pairs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(calls)]
        t.cuda._sleep(20_000_000)
        for i, (a, b) in enumerate(pairs):
            a.record()
            fn(i)
            b.record()
        t.cuda.synchronize()
        d = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)

        def pct(q):
            return d[min(len(d) - 1, int(round(q * (len(d) - 1))))]
        return {"p50_us": pct(0.50), "p90_us": pct(0.90), "p99_us": pct(0.99), "mean_us": sum(d) / len(d),
                "calls": calls}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on a single MI355X and has no "
              "multi-GPU path (asked for --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import bf16_gemm_linear_amd as sp
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kind = args.dtype
    if kind == "int8" and args.workload in ("layers", "palette", "all"):
        print("--dtype int8 is measured on the up, down, prefill and slide workloads", file=sys.stderr)
        sys.exit(2)
    if kind == "bf16" and args.workload == "slide":
        print("the slide workload multiplies one-byte codes: --dtype fp8 or int8", file=sys.stderr)
        sys.exit(2)
    ev = Events(torch)
    ctx = (args, torch, np, sp, W, ev, dev)

    if args.workload == "slide":
        print(json.dumps(run_slide(*ctx)))
        return
    if args.workload == "palette":
        print(json.dumps(run_palette(*ctx)))
        return
    if args.workload == "groups":
        print(json.dumps({"metric": "FP8 sparse GEMM with group scales: time against per-tensor scales",
                          "n_gpus": 1, "data": "synthetic (seeded, workloads/)", **run_groups(*ctx)}))
        return
    if args.workload == "layers":
        print(json.dumps(layers_line(args, run_layers(*ctx))))
        return
    if args.workload == "prefill":
        print(json.dumps(prefill_line(args, run_prefill(*ctx))))
        return
    if args.workload in ("up", "down"):
        print(json.dumps(decode_line(args, run_decode(*ctx, args.workload))))
        return

    # --workload all: the headline step, then every configuration of the metric
    t_all = time.perf_counter()
    up = run_decode(*ctx, "up")
    out = decode_line(args, up)
    torch.cuda.empty_cache()
    down = run_decode(*ctx, "down", headline=False)
    torch.cuda.empty_cache()
    pre = run_prefill(*ctx)
    torch.cuda.empty_cache()
    lay = run_layers(*ctx)
    torch.cuda.empty_cache()
    grp = run_groups(*ctx)
    out["config"]["workload"] = ("decode FFN up-projection, 2:4 sparse %s, M=1/16/64 tokens, K=4096, N=14336 "
                                 "(headline step); every configuration of the metric under configs"
                                 % up["label"])
    out["configs"] = {
        "up": config_summary_decode(up),
        "down": config_summary_decode(down),
        "prefill": config_summary_prefill(pre),
        "layers": config_summary_layers(lay),
        "groups": {"workload": "FP8 with one scale per 128-K group and per output channel (sp24_gemm_groups) "
                               "against per-tensor scales, decode up/down M=1/16/64 and prefill", **grp},
    }
    out["bench_wall_s"] = time.perf_counter() - t_all
    print(json.dumps(out))


# --------------------------------------------------------------------------- decode
def run_decode(args, torch, np, sp, W, ev, dev, which, headline=True):
    """The decode-shaped projection `which` ("up": K=4096, N=14336; "down": K=14336,
    N=4096) at M = 1, 16, 64: load path, the per-call step in HIP graphs, every GEMM
    alone, per-call percentiles, the dense-MFMA baseline and hipBLASLt's dense FP8."""
    kind = args.dtype
    fp8 = kind != "bf16"  # one-byte codes with per-tensor scales: E4M3 or INT8
    dt = {"fp8": sp.FP8, "int8": sp.INT8, "bf16": sp.BF16}[kind]
    quant = sp.quant_int8 if kind == "int8" else sp.quant_fp8
    code_t = torch.int8 if kind == "int8" else torch.uint8
    label = {"fp8": "FP8-E4M3 (per-tensor scales)", "int8": "INT8 W8A8 (per-tensor scales)", "bf16": "BF16"}[kind]
    spec = W.UP if which == "up" else W.DOWN
    K, N, Ms = spec["K"], spec["N"], list(spec["Ms"])
    w_cpu = W.up_weight() if which == "up" else W.down_weight()
    xs_cpu = {m: (W.up_x(m) if which == "up" else W.down_x(m)) for m in Ms}
    desc = ("decode FFN %s-projection, 2:4 sparse %s, M=%s tokens, K=%d, N=%d"
            % (which, label, "/".join(map(str, Ms)), K, N))

    # ---------------------------------------------------------------- load path
    w = w_cpu.to(dev)
    xs = {m: xs_cpu[m].to(dev) for m in Ms}
    values = torch.empty(N, K // 2, dtype=torch.bfloat16, device=dev)
    meta = torch.empty(N * (K // 32), dtype=torch.int32, device=dev)
    sp.prune_compress(w, values, meta)  # first launch loads the code object: not timed
    t_prune = ev.time(lambda i: sp.prune_compress(w, values, meta), 5) / 5
    qv, sw = (quant(values) if fp8 else (values, None))
    if fp8:
        qbuf = torch.empty_like(qv)
        quant(values, scale=sw, out=qbuf, mode=sp.SCALE_DYNAMIC)
        t_wq = ev.time(lambda i: quant(values, scale=sw, out=qbuf, mode=sp.SCALE_DYNAMIC), 5) / 5
        del qbuf
    else:
        t_wq = 0.0
    torch.cuda.synchronize()
    load_path = {
        "prune_compress_us": t_prune * 1e6,
        "prune_compress_GBs": (N * K * 2 + N * K + N * (K // 32) * 4) / t_prune / 1e9,
        "quant_weight_us": t_wq * 1e6 if fp8 else None,
        "quant_weight_GBs": (N * K // 2 * 2 + N * K // 2) / t_wq / 1e9 if fp8 else None,
    }
    del w

    # weight copies, so that each call reads its weight from HBM
    R = n_copies(qv.numel() * qv.element_size() + meta.numel() * 4)
    wq_copies = [qv] + [qv.clone() for _ in range(R - 1)]
    meta_copies = [meta] + [meta.clone() for _ in range(R - 1)]

    # per-M buffers (allocated once: graphs and timed loops allocate nothing)
    bufs = {}
    for m in Ms:
        b = {"y": torch.empty(m, N, dtype=torch.bfloat16, device=dev)}
        if fp8:
            b["xq"] = torch.empty(m, K, dtype=code_t, device=dev)
            b["sx"] = torch.empty(1, dtype=torch.float32, device=dev)
            nb = sp.workspace_size(sp.OP_QUANT, sp.BF16, m * K, 1, 1)
            b["qws"] = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        nb = sp.workspace_size(sp.OP_GEMM, dt, m, N, K)
        b["gws"] = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        if kind == "fp8":  # quantise + GEMM in one call (X quantised inside the kernel at M = 1)
            nb = sp.workspace_size(sp.OP_GEMM_QX, dt, m, N, K)
            b["qxws"] = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        b["plan"] = sp.plan(sp.OP_GEMM, dt, m, N, K)
        bufs[m] = b

    def call_quant(m):
        b = bufs[m]
        if fp8:
            quant(xs[m], scale=b["sx"], out=b["xq"], ws=b["qws"], mode=sp.SCALE_DYNAMIC)

    def call_gemm(m, r):
        b = bufs[m]
        if fp8:
            sp.gemm(b["xq"], wq_copies[r], meta_copies[r], x_scale=b["sx"], w_scale=sw, out=b["y"],
                    ws=b["gws"])
        else:
            sp.gemm(xs[m], wq_copies[r], meta_copies[r], out=b["y"], ws=b["gws"])

    def call_step(m, r):
        """One step's work for M tokens: quantise X (FP8, INT8) and the sparse GEMM."""
        b = bufs[m]
        if kind == "fp8":
            sp.gemm_qx(xs[m], wq_copies[r], meta_copies[r], sw, x_scale=b["sx"], out=b["y"], ws=b["qxws"])
        else:
            call_quant(m)
            call_gemm(m, r)

    def step(r):
        for j, m in enumerate(Ms):
            call_step(m, (r * len(Ms) + j) % R)

    # eager reference of every M's output for one rotation index
    step(0)
    torch.cuda.synchronize()
    eager = {m: bufs[m]["y"].clone() for m in Ms}

    # ---------------------------------------------------------------- graphs of the step
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    n_graphs = R  # one graph per rotation start
    for r in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()

    def replay(i):
        graphs[i % n_graphs].replay()

    steps = args.steps if headline else min(args.steps, 50)
    warmup = args.warmup if headline else min(args.warmup, 5)
    for i in range(warmup):
        replay(i)
    torch.cuda.synchronize()
    t_steps = ev.time(replay, steps)
    ms_per_step = t_steps / steps * 1e3

    # graphs replayed many times must reproduce the eager outputs bitwise
    graphs[0].replay()
    torch.cuda.synchronize()
    for m in Ms:
        if not torch.equal(bufs[m]["y"].view(torch.int16), eager[m].view(torch.int16)):
            raise SystemExit("graph replay output differs from the eager run for M=%d" % m)
    del graphs

    step_bytes = sum(gemm_bytes(m, N, K, fp8) + (quant_bytes(m, K) if fp8 else 0) for m in Ms)
    step_flops = sum(2 * m * N * K for m in Ms)          # dense-equivalent

    # ---------------------------------------------------------------- the sparse GEMM alone
    per_m = {}
    for m in Ms:
        reps = args.kernel_reps or R * 16
        t = ev.graph(lambda i: call_gemm(m, i % R), reps)
        gb = gemm_bytes(m, N, K, fp8)
        per_m[m] = {"gemm_us": t * 1e6, "GBs": gb / t / 1e9,
                    "hbm_frac": gb / t / 1e9 / HBM_PEAK_GBS,
                    "algorithmic_bytes": gb,
                    "tflops_dense_equiv": 2 * m * N * K / t / 1e12,
                    "tflops_effective": m * N * K / t / 1e12,
                    "plan": {k2: v for k2, v in bufs[m]["plan"].items()
                             if k2 in ("kernel", "config", "tile_n", "tile_m", "waves", "split_k")}}
        if not args.no_percentiles:
            per_m[m]["gemm_call"] = ev.percentiles(lambda i: call_gemm(m, i % R), 400)
    for m in Ms:  # quantiser alone
        if fp8:
            reps = 200
            t = ev.time(lambda i: call_quant(m), reps) / reps
            per_m[m]["quant_x_us_eager"] = t * 1e6
    if kind == "fp8":
        # quantise + GEMM in one call, per tensor (the step) and per token, graph-replayed
        for m in Ms:
            b = bufs[m]
            xsr = torch.empty(m, dtype=torch.float32, device=dev)
            wsr = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, N, K)), dtype=torch.uint8,
                              device=dev)
            calls = {"step_qx_us": lambda i: sp.gemm_qx(xs[m], wq_copies[i % R], meta_copies[i % R], sw,
                                                        x_scale=b["sx"], out=b["y"], ws=b["qxws"]),
                     "step_rows_qx_us": lambda i: sp.gemm_rows_qx(xs[m], wq_copies[i % R], meta_copies[i % R], sw,
                                                                  x_scales=xsr, out=b["y"], ws=wsr)}
            for key, fn in calls.items():
                per_m[m][key] = ev.graph(fn, R * 8) * 1e6
            per_m[m]["step_qx_over_gemm_us"] = per_m[m]["step_qx_us"] - per_m[m]["gemm_us"]
            if not args.no_percentiles:
                per_m[m]["step_qx_call"] = ev.percentiles(calls["step_qx_us"], 200)

    # ---------------------------------------------------------------- dense baseline
    if not args.no_dense:
        wd = sp.decompress(qv, meta, K)
        Rd = n_copies(wd.numel() * wd.element_size())
        wd_copies = [wd] + [wd.clone() for _ in range(Rd - 1)]
        for m in Ms:
            b = bufs[m]
            xin = b["xq"] if fp8 else xs[m]
            yd = torch.empty_like(b["y"])
            nb = sp.workspace_size(sp.OP_DENSE_GEMM, dt, m, N, K)
            dws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)

            def dcall(i, m=m, xin=xin, yd=yd, dws=dws):
                sp.dense_gemm(xin, wd_copies[i % Rd], x_scale=bufs[m].get("sx"), w_scale=sw, out=yd,
                              ws=dws)
            t = ev.graph(dcall, args.kernel_reps or Rd * 16)
            db = dense_bytes(m, N, K, fp8)
            per_m[m]["dense_gemm_us"] = t * 1e6
            per_m[m]["dense_GBs"] = db / t / 1e9
            per_m[m]["sparse_speedup_vs_dense"] = t / (per_m[m]["gemm_us"] / 1e6)
            if kind == "fp8":
                tv = vendor_dense_fp8(torch, ev, xin, wd_copies, bufs[m]["sx"], sw, m, "hbm")
                if tv is not None:
                    per_m[m]["vendor_dense_fp8_us"] = tv * 1e6
                    per_m[m]["sparse_speedup_vs_vendor_dense"] = tv / (per_m[m]["gemm_us"] / 1e6)
        del wd_copies, wd

    tot_b = sum(gemm_bytes(m, N, K, fp8) for m in Ms)
    tot_t = sum(per_m[m]["gemm_us"] for m in Ms) / 1e6
    achieved = tot_b / tot_t / 1e9
    kernels = "/".join(sorted({KERNEL_NAMES[bufs[m]["plan"]["kernel"]] for m in Ms}))
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": counted_traffic(which, "hbm") if kind == "fp8" else None,
                "kernel": "%s (sparse %s), mean over M=%s" % (kernels, kind, "/".join(map(str, Ms))),
                "per_unit": "values N*K/2*es + metadata N*K/8 + X M*K*es + Y 2*M*N bytes per launch"}
    cpu = None
    if not args.no_cpu_baseline and headline:
        cpu = cpu_baseline(w_cpu, xs_cpu, Ms, N, K, kind, step_bytes)
    del wq_copies, meta_copies
    return {"which": which, "kind": kind, "label": label, "desc": desc, "K": K, "N": N, "Ms": Ms, "R": R,
            "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step, "step_bytes": step_bytes,
            "step_flops": step_flops, "per_m": per_m, "roofline": roofline, "cpu": cpu,
            "load_path": load_path, "device": torch.cuda.get_device_name(dev)}


def decode_line(args, d):
    kind = d["kind"]
    return {
        "metric": METRIC,
        "value": d["step_bytes"] / (d["ms_per_step"] / 1e3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": d["steps"], "warmup": d["warmup"], "ms_per_step": d["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "int8": "int8", "bf16": "bf16"}[kind],
        "data": "synthetic (seeded, workloads/)",
        "config": {"workload": d["desc"], "M": d["Ms"], "K": d["K"], "N": d["N"], "weight_copies": d["R"],
                   "step": {"fp8": "per M: sp24_gemm_qx (quantise X + sparse GEMM; one launch at M=1)",
                            "int8": "per M: sp24_quant_int8 + sparse INT8 GEMM",
                            "bf16": "per M: sparse GEMM"}[kind]},
        "roofline": d["roofline"],
        "cpu_baseline": d["cpu"],
        "per_m": {str(m): d["per_m"][m] for m in d["Ms"]},
        "step_GB": d["step_bytes"] / 1e9,
        "step_tflops_dense_equiv": d["step_flops"] / (d["ms_per_step"] / 1e3) / 1e12,
        "load_path": d["load_path"],
        "device": d["device"],
    }


def config_summary_decode(d):
    return {"workload": d["desc"], "K": d["K"], "N": d["N"], "weight_copies": d["R"],
            "roofline": d["roofline"],
            "step_qx_GBs": d["step_bytes"] / (d["ms_per_step"] / 1e3) / 1e9 if d["kind"] == "fp8" else None,
            "per_m": {str(m): d["per_m"][m] for m in d["Ms"]}}


def vendor_dense_fp8(torch, ev, xq, w_copies, sx, sw, m, bound):
    """Reference only: the same dense FP8 product through torch._scaled_mm (hipBLASLt on
    ROCm), X padded to 16 rows, back-to-back launches without graphs.  None if unavailable."""
    try:
        f8 = torch.float8_e4m3fn
        mp = max(16, (m + 15) // 16 * 16)
        xp = torch.zeros(mp, xq.shape[1], dtype=f8, device=xq.device)
        xp[:m] = xq.view(f8)
        ws = [w.view(f8) for w in w_copies]
        fn = lambda i: torch._scaled_mm(xp, ws[i % len(ws)].t(), scale_a=sx.reshape(()), scale_b=sw.reshape(()),
                                        out_dtype=torch.bfloat16)
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        reps = 8 * len(ws) if bound == "hbm" else 5
        return ev.time(fn, reps) / reps
    except Exception:  # pragma: no cover - depends on the torch build
        return None


# --------------------------------------------------------------------------- prefill
def run_prefill(args, torch, np, sp, W, ev, dev):
    """The prefill-shaped GEMM M=8192, K=8192, N=28672 (bound: matrix cores): the sparse
    GEMM alone (mean and per-call percentiles), quantise + GEMM, the dense-MFMA baseline,
    hipBLASLt's dense FP8, and the CPU oracle on a slice."""
    kind = args.dtype
    fp8 = kind != "bf16"
    dt = {"fp8": sp.FP8, "int8": sp.INT8, "bf16": sp.BF16}[kind]
    quant = sp.quant_int8 if kind == "int8" else sp.quant_fp8
    label = {"fp8": "FP8-E4M3 (per-tensor scales)", "int8": "INT8 W8A8 (per-tensor scales)", "bf16": "BF16"}[kind]
    M, K, N = W.PREFILL["M"], W.PREFILL["K"], W.PREFILL["N"]
    w_cpu, x_cpu = W.prefill_weight(), W.prefill_x()
    w, x = w_cpu.to(dev), x_cpu.to(dev)
    values, meta = sp.prune_compress(w)
    del w
    if fp8:
        qv, sw = quant(values)
        xq, sx = quant(x)
    else:
        qv, sw, xq, sx = values, None, x, None
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    gws = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM, dt, M, N, K)), dtype=torch.uint8, device=dev)
    plan = sp.plan(sp.OP_GEMM, dt, M, N, K)

    def call(i):
        sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw, out=y, ws=gws)
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    reps = 20
    t = ev.time(call, reps) / reps
    flops = 2.0 * M * N * K
    peak = FP8_DENSE_PEAK_TFLOPS if fp8 else BF16_DENSE_PEAK_TFLOPS
    res = {"gemm_ms": t * 1e3, "tflops_dense_equiv": flops / t / 1e12, "tflops_effective": flops / 2 / t / 1e12,
           "frac_of_sparse_peak": flops / 2 / t / 1e12 / peak,
           "GBs": gemm_bytes(M, N, K, fp8) / t / 1e9,
           "plan": {k2: v for k2, v in plan.items() if k2 in ("kernel", "config", "tile_n", "tile_m", "waves",
                                                              "split_k")}}
    if not args.no_percentiles:
        res["gemm_call"] = ev.percentiles(call, 40)
    if kind == "fp8":  # the per-call step: quantise X (two launches at this size) + GEMM
        sxs = torch.empty(1, dtype=torch.float32, device=dev)
        qws = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM_QX, sp.FP8, M, N, K)), dtype=torch.uint8,
                          device=dev)
        fn = lambda i: sp.gemm_qx(x, qv, meta, sw, x_scale=sxs, out=y, ws=qws)
        fn(0)
        torch.cuda.synchronize()
        res["step_qx_ms"] = ev.time(fn, 10) / 10 * 1e3
        del qws
    if not args.no_dense:
        wd = sp.decompress(qv, meta, K)
        dws = torch.empty(max(16, sp.workspace_size(sp.OP_DENSE_GEMM, dt, M, N, K)), dtype=torch.uint8, device=dev)
        dcall = lambda i: sp.dense_gemm(xq, wd, x_scale=sx, w_scale=sw, out=y, ws=dws)
        for i in range(2):
            dcall(i)
        torch.cuda.synchronize()
        td = ev.time(dcall, 10) / 10
        res.update({"dense_gemm_ms": td * 1e3, "dense_tflops": flops / td / 1e12,
                    "dense_frac_of_dense_peak": flops / td / 1e12 / peak,
                    "sparse_speedup_vs_dense": td / t})
        if kind == "fp8":
            tv = vendor_dense_fp8(torch, ev, xq, [wd], sx, sw, M, "mfma")
            if tv is not None:
                res["vendor_dense_fp8_ms"] = tv * 1e3
                res["sparse_speedup_vs_vendor_dense"] = tv / t
        del wd, dws
    eff = res["tflops_effective"]
    roofline = {"bound": "mfma", "achieved": eff, "peak": peak,
                "unit": "TOP/s" if kind == "int8" else "TFLOP/s", "frac": eff / peak,
                "traffic": counted_traffic("prefill", "mfma") if kind == "fp8" else None,
                "kernel": "%s (sparse %s): nonzero MACs x 2 per second against the dense %s MFMA peak (%s); "
                          "equals dense-equivalent flops against twice that peak"
                          % (KERNEL_NAMES[plan["kernel"]], kind, kind.upper(), PEAK_SOURCE),
                "per_unit": "M*N*K nonzero multiply-adds (2*M*N*K dense-equivalent flops) per launch"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_prefill_baseline(w_cpu, x_cpu, kind)
    del qv, meta, xq, y, gws
    return {"kind": kind, "label": label, "M": M, "K": K, "N": N, "res": res, "roofline": roofline, "cpu": cpu,
            "desc": "prefill GEMM, 2:4 sparse %s, M=%d, K=%d, N=%d" % (label, M, K, N),
            "device": torch.cuda.get_device_name(dev)}


def prefill_line(args, p):
    kind, r = p["kind"], p["res"]
    return {
        "metric": METRIC,
        "value": r["tflops_effective"],
        "unit": ("TOP/s" if kind == "int8" else "TFLOP/s") + " (nonzero MACs x2)",
        "n_gpus": 1, "steps": 20, "warmup": 3, "ms_per_step": r["gemm_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "fp8_e4m3", "int8": "int8", "bf16": "bf16"}[kind],
        "data": "synthetic (seeded, workloads/)",
        "config": {"workload": p["desc"], "M": p["M"], "K": p["K"], "N": p["N"], "step": "sparse GEMM"},
        "roofline": p["roofline"], "cpu_baseline": p["cpu"], "prefill": r, "device": p["device"],
    }


def config_summary_prefill(p):
    return {"workload": p["desc"], "M": p["M"], "K": p["K"], "N": p["N"], "roofline": p["roofline"],
            "cpu_baseline": p["cpu"], **p["res"]}


def cpu_prefill_baseline(w_cpu, x_cpu, kind):
    """The CPU oracle's per-call path on a slice of the prefill GEMM: rows 0..255 of W
    (pruned, compressed and quantised at load, not timed) against tokens 0..511 of X
    (quantise X, decompress W, float64 product and magnitude sum), repeated for about 8 s;
    reported as dense-equivalent TFLOP/s of the slice."""
    import workloads as W
    from oracle import sp24_ref as O
    wb = W.bf16_bits(w_cpu[:256])
    xb = W.bf16_bits(x_cpu[:512])
    K = wb.shape[1]
    v, meta = O.prune_compress(wb)
    if kind == "fp8":
        vq, sw = O.quant_fp8(v)
    elif kind == "int8":
        vq, sw = O.quant_int8(v)
    reps, t0 = 0, time.perf_counter()
    while True:
        if kind == "fp8":
            xq, sx = O.quant_fp8(xb)
            O.gemm_ref(*O.sparse_operands_fp8(xq, sx, vq, meta, sw, K))
        elif kind == "int8":
            xq, sx = O.quant_int8(xb)
            O.gemm_ref(*O.sparse_operands_int8(xq, sx, vq, meta, sw, K))
        else:
            O.gemm_ref(*O.sparse_operands_bf16(xb, v, meta, K))
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 50:
            break
    flops = 2.0 * 512 * 256 * K
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": "%d call(s) of a 512-token x 256-row slice of the prefill GEMM (K=%d: quantise X, "
                      "decompress W, float64 product and magnitude sum), %.1f s wall" % (reps, K, el)}


def run_slide(args, torch, np, sp, W, ev, dev):
    """SlideSparse 6:8 (N = 4) on the 2:4 path against the dense GEMM and the 2:4 GEMM of
    the same shape and code type (FP8-E4M3, or INT8 W8A8 with --dtype int8): the decode up-projection (K=4096, N=14336, M=1/16/64) and the prefill
    GEMM (M=8192, K=8192, N=28672).  The 6:8 weight is expanded to K' = 1.5 K; its bound
    over dense is N/(N-1) = 4/3 in matrix work (the page's S_max), and the byte ratio at
    decode.  Weights: 0.02 N(0, 1) (prefill 0.01) drawn on the GPU (seeds 1 and 3); X from
    workloads/.  Decode rotates weight copies past the last-level cache."""
    n_pat = 4
    i8 = args.dtype == "int8"
    dt = sp.INT8 if i8 else sp.FP8
    quant = sp.quant_int8 if i8 else sp.quant_fp8
    quant_rows = sp.quant_int8_rows if i8 else sp.quant_fp8_rows
    slide_quant = sp.slide_quant_int8_rows if i8 else sp.slide_quant_fp8_rows
    tname = "INT8" if i8 else "FP8"
    shapes = [("up", m, 4096, 14336) for m in (1, 16, 64)] + [("prefill", 8192, 8192, 28672)]
    out = {}
    cache = {}
    for name, m, k, n in shapes:
        kp = k * (2 * n_pat - 2) // n_pat
        if (k, n) not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            g = torch.Generator(device=dev)
            g.manual_seed(1 if name == "up" else 3)
            w = (torch.randn(n, k, generator=g, device=dev) * (0.02 if name == "up" else 0.01)).to(torch.bfloat16)
            wp = sp.slide_prune_pack(w, n_pat)
            v68, m68 = sp.prune_compress(wp)
            del wp
            q68, s68 = quant(v68)
            v24, m24 = sp.prune_compress(w)
            q24, s24 = quant(v24)
            qd, sd = quant(w)
            del w, v68, v24
            b68 = q68.numel() + m68.numel() * 4
            b24 = q24.numel() + m24.numel() * 4
            bd = qd.numel()
            decode = name == "up"
            reps = lambda b: max(2, min(16, int(np.ceil(2.2 * LLC_BYTES / b)))) if decode else 1
            cache[(k, n)] = dict(
                w68=[(q68, m68)] + [(q68.clone(), m68.clone()) for _ in range(reps(b68) - 1)],
                w24=[(q24, m24)] + [(q24.clone(), m24.clone()) for _ in range(reps(b24) - 1)],
                wd=[qd] + [qd.clone() for _ in range(reps(bd) - 1)],
                s68=s68, s24=s24, sd=sd, b68=b68, b24=b24, bd=bd)
        c = cache[(k, n)]
        x = (W.up_x(m) if name == "up" else W.prefill_x()).to(dev)
        xq68, sx68 = slide_quant(x, n_pat)
        xq24, sx24 = quant_rows(x)
        y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        ws68 = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM, dt, m, n, kp)), dtype=torch.uint8, device=dev)
        wsq68 = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM_ROWS_QX, sp.FP8, m, n, kp)), dtype=torch.uint8,
                            device=dev)
        ws24 = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM, dt, m, n, k)), dtype=torch.uint8, device=dev)
        wsd = torch.empty(max(16, sp.workspace_size(sp.OP_DENSE_GEMM, dt, m, n, k)), dtype=torch.uint8,
                          device=dev)
        sxd = sx24[:1].contiguous()
        calls = {
            "slide_gemm": lambda i: sp.gemm_rows(xq68, c["w68"][i % len(c["w68"])][0], c["w68"][i % len(c["w68"])][1],
                                                 sx68, c["s68"], out=y, ws=ws68),
            "slide_step_fused": (lambda i: sp.slide_gemm_qx(x, c["w68"][i % len(c["w68"])][0],
                                                            c["w68"][i % len(c["w68"])][1], c["s68"], n_pat,
                                                            x_scales=sx68, out=y, ws=wsq68)) if not i8 else None,
            "slide_step": lambda i: (slide_quant(x, n_pat, out=xq68, scales=sx68),
                                     sp.gemm_rows(xq68, c["w68"][i % len(c["w68"])][0], c["w68"][i % len(c["w68"])][1],
                                                  sx68, c["s68"], out=y, ws=ws68)),
            "sparse24_gemm": lambda i: sp.gemm_rows(xq24, c["w24"][i % len(c["w24"])][0],
                                                    c["w24"][i % len(c["w24"])][1], sx24, c["s24"], out=y, ws=ws24),
            "dense_gemm": lambda i: sp.dense_gemm(xq24, c["wd"][i % len(c["wd"])], x_scale=sxd, w_scale=c["sd"],
                                                  out=y, ws=wsd),
        }
        res = {}
        for key, fn in calls.items():
            if fn is None:
                continue
            nrep = 48 if name == "up" else 5
            fn(0)
            torch.cuda.synchronize()
            if name == "up":
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(nrep):
                        fn(i)
                graph.replay()
                torch.cuda.synchronize()
                t = ev.time(lambda i: graph.replay(), 3) / 3 / nrep
                del graph
            else:
                for i in range(2):
                    fn(i)
                t = ev.time(fn, nrep) / nrep
            res[key + "_us"] = t * 1e6
        flops = 2.0 * m * n * k
        res.update({
            "K": k, "K_expanded": kp, "N": n,
            "speedup_vs_dense": res["dense_gemm_us"] / res["slide_gemm_us"],
            "speedup_2of4_vs_dense": res["dense_gemm_us"] / res["sparse24_gemm_us"],
            "bound_vs_dense": (c["bd"] + m * k + 2 * m * n) / (c["b68"] + m * kp + 2 * m * n) if name == "up"
            else n_pat / (n_pat - 1),
            "weight_bytes": {"slide_6of8": c["b68"], "sparse_2of4": c["b24"], "dense": c["bd"]},
            "tflops_dense_equiv": flops / res["slide_gemm_us"] / 1e6,
        })
        out["%s M=%d" % (name, m)] = res
    pre = out["prefill M=8192"]
    return {"metric": "SlideSparse 6:8 %s GEMM (2:4 path over K' = 1.5 K): speedup over the dense %s GEMM"
                      % (tname, tname),
            "value": pre["speedup_vs_dense"], "unit": "x (prefill, dense time / SlideSparse time)",
            "n_gpus": 1, "steps": None, "warmup": None, "ms_per_step": pre["slide_gemm_us"] / 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8" if i8 else "fp8_e4m3",
            "data": "synthetic (seeded)",
            "config": {"workload": "SlideSparse 6:8 (N=4): decode up-projection M=1/16/64 (K=4096, N=14336) and "
                                   "prefill 8192x28672x8192; per-token X scales, per-tensor W scale"},
            "per_shape": out}


def run_palette(args, torch, np, sp, W, ev, dev):
    """Lossless BF16 exponent-palette weights against the dense BF16 GEMM of the same weight,
    M = 1/4/16: the decode up- and down-projections (weights from workloads/), and the
    up-projection weight with every magnitude raised to at least 0.02 * 2^-11 (sign kept),
    which leaves 15 exponents, so that every row fits the palette (the page's premise that
    the 16 most common exponents cover nearly all weights, here for every row).  A call
    reads one of R copies of the encoded weight, past the last-level cache."""
    def narrow(w):
        f = w.float()
        sign = torch.where(f >= 0, 1.0, -1.0)
        return (sign * f.abs().clamp(min=0.02 * 2.0 ** -11)).to(torch.bfloat16)
    cases = [("up", W.up_weight(), W.up_x), ("down", W.down_weight(), W.down_x),
             ("up, every row in the palette", narrow(W.up_weight()), W.up_x)]
    out = {}
    for name, w_cpu, xfn in cases:
        torch.cuda.empty_cache()
        w = w_cpu.to(dev)
        n, k = w.shape
        pw = sp.palette_encode(w)
        torch.cuda.synchronize()
        t_enc = ev.time(lambda i: sp.palette_encode(w), 3) / 3   # includes its one host read of the counts
        R = max(2, min(16, int(np.ceil(2.2 * LLC_BYTES / pw.nbytes))))
        pws = [pw] + [sp.PaletteWeight(pw.n, pw.k, pw.palette.clone(), pw.pal_rows.clone(), pw.sm.clone(),
                                       pw.ix.clone(), pw.verb_rows.clone(), pw.verb.clone()) for _ in range(R - 1)]
        wds = [w] + [w.clone() for _ in range(R - 1)]
        res = {"rows_in_palette": pw.n_pal, "rows_verbatim": pw.n_verb, "encoded_bytes": pw.nbytes,
               "bf16_bytes": n * k * 2, "byte_ratio": pw.nbytes / (n * k * 2), "encode_ms": t_enc * 1e3,
               "weight_copies": R}
        for m in (1, 4, 16):
            x = xfn(m).to(dev)
            y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            dws = torch.empty(max(16, sp.workspace_size(sp.OP_DENSE_GEMM, sp.BF16, m, n, k)), dtype=torch.uint8,
                              device=dev)
            times = {}
            for key, fn in (("palette", lambda i: sp.palette_gemm(x, pws[i % R], out=y)),
                            ("dense_bf16", lambda i: sp.dense_gemm(x, wds[i % R], out=y, ws=dws))):
                nrep = R * 8
                fn(0)
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(nrep):
                        fn(i)
                graph.replay()
                torch.cuda.synchronize()
                times[key] = ev.time(lambda i: graph.replay(), 3) / 3 / nrep
                del graph
            pb = pw.nbytes + m * k * 2 + m * n * 2
            db = n * k * 2 + m * k * 2 + m * n * 2
            res["M=%d" % m] = {"palette_us": times["palette"] * 1e6, "dense_bf16_us": times["dense_bf16"] * 1e6,
                               "speedup_vs_dense": times["dense_bf16"] / times["palette"],
                               "palette_GBs": pb / times["palette"] / 1e9,
                               "dense_GBs": db / times["dense_bf16"] / 1e9}
        out[name] = res
        del pws, wds, pw, w
    up1 = out["up"]["M=1"]
    return {"metric": "lossless BF16 exponent-palette GEMM at decode: GB/s of encoded weight, and speedup over "
                      "the dense BF16 GEMM",
            "value": up1["palette_GBs"], "unit": "GB/s (up-projection, M=1)",
            "n_gpus": 1, "steps": None, "warmup": None, "ms_per_step": up1["palette_us"] / 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded, workloads/)",
            "config": {"workload": "exponent-palette weights (16-entry palette, verbatim rows), decode "
                                   "up-projection K=4096 N=14336 and down-projection K=14336 N=4096, M=1/4/16"},
            "roofline": {"bound": "hbm", "achieved": up1["palette_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": up1["palette_GBs"] / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "pal_gemm_kernel, up-projection M=1"},
            "cpu_baseline": None if args.no_cpu_baseline else cpu_palette_baseline(W),
            "per_weight": out}


def cpu_palette_baseline(W):
    """The CPU oracle's per-call path for palette weights -- rebuild W from its encoded form
    and the float64 product -- on the first 1024 rows of the up-projection weight at M=1
    (encoding, a load-time step, is not timed), repeated for about 10 s."""
    import numpy as np

    from oracle import palette_ref as P
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    wb = W.bf16_bits(W.up_weight()[:1024])
    xb = W.bf16_bits(W.up_x(1))
    enc = P.palette_encode(wb)
    nbytes = P.encoded_bytes(enc) + xb.size * 2 + 1024 * 2
    reps, t0 = 0, time.perf_counter()
    while True:
        P.gemm_ref(xb, P.palette_decode(enc))
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 200:
            break
    return {"value": nbytes * reps / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d call(s) on rows 0..1023 of the up-projection weight at M=1 (rebuild W from the "
                      "palette form, float64 product and magnitude sum), %.1f s wall" % (reps, el)}




# --------------------------------------------------------------------------- group scales
def run_groups(args, torch, np, sp, W, ev, dev):
    """FP8 with finer scales (sp24_gemm_groups) against the per-tensor sparse GEMM of the
    same shape: 128-K groups and one group per row (per-token X, per-output-channel W), at
    the decode up- and down-projection (M = 1/16/64, weight copies rotated past the
    last-level cache, HIP graphs) and at prefill (M=8192, K=8192, N=28672).  The codes and
    scales come from sp24_quant_fp8_groups (X in groups along K, the compressed weight in
    groups of group/2 kept values)."""
    out = {}
    cases = [("up", W.up_weight, W.up_x, W.UP), ("down", W.down_weight, W.down_x, W.DOWN)]
    for name, wf, xf, spec in cases:
        K, N = spec["K"], spec["N"]
        w = wf().to(dev)
        values, meta = sp.prune_compress(w)
        del w
        qv, sw = sp.quant_fp8(values)
        forms = {g: sp.quant_fp8_groups(values, g // 2) for g in (128, K)}
        del values
        R = n_copies(qv.numel() + meta.numel() * 4)
        metas = [meta] + [meta.clone() for _ in range(R - 1)]
        qvs = [qv] + [qv.clone() for _ in range(R - 1)]
        gq = {g: [f] + [(f[0].clone(), f[1].clone()) for _ in range(R - 1)] for g, f in forms.items()}
        res = {}
        for m in spec["Ms"]:
            x = xf(m).to(dev)
            xq, sx = sp.quant_fp8(x)
            y = torch.empty(m, N, dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM_GROUPS, sp.FP8, m, N, K)), dtype=torch.uint8,
                             device=dev)
            r = {"per_tensor_us": ev.graph(lambda i: sp.gemm(xq, qvs[i % R], metas[i % R], x_scale=sx, w_scale=sw,
                                                             out=y, ws=ws), R * 8) * 1e6}
            for g, label in ((128, "group128_us"), (K, "per_channel_us")):
                gx, gs = sp.quant_fp8_groups(x, g)
                r[label] = ev.graph(lambda i: sp.gemm_groups(gx, gs, gq[g][i % R][0], metas[i % R], gq[g][i % R][1], g,
                                                             out=y, ws=ws), R * 8) * 1e6
            gb = gemm_bytes(m, N, K, True)
            r["group128_GBs"] = (gb + N * K // 128 * 4 + m * K // 128 * 4) / r["group128_us"] / 1e3
            r["group128_over_per_tensor"] = r["group128_us"] / r["per_tensor_us"]
            res[str(m)] = r
        out[name] = res
        del qvs, metas, gq, forms, qv, meta
        torch.cuda.empty_cache()
    # prefill: one call each, eager
    M, K, N = W.PREFILL["M"], W.PREFILL["K"], W.PREFILL["N"]
    w = W.prefill_weight().to(dev)
    values, meta = sp.prune_compress(w)
    del w
    x = W.prefill_x().to(dev)
    qv, sw = sp.quant_fp8(values)
    xq, sx = sp.quant_fp8(x)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, sp.workspace_size(sp.OP_GEMM_GROUPS, sp.FP8, M, N, K)), dtype=torch.uint8, device=dev)
    pre = {}
    fn = lambda i: sp.gemm(xq, qv, meta, x_scale=sx, w_scale=sw, out=y, ws=ws)
    fn(0)
    torch.cuda.synchronize()
    pre["per_tensor_ms"] = ev.time(fn, 5) / 5 * 1e3
    for g, label in ((K, "per_channel_ms"), (128, "group128_ms")):
        gw, gws = sp.quant_fp8_groups(values, g // 2)
        gx, gxs = sp.quant_fp8_groups(x, g)
        fn = lambda i: sp.gemm_groups(gx, gxs, gw, meta, gws, g, out=y, ws=ws)
        fn(0)
        torch.cuda.synchronize()
        reps = 5 if g == K else 2
        pre[label] = ev.time(fn, reps) / reps * 1e3
        pre[label.replace("_ms", "_tflops_dense_equiv")] = 2.0 * M * N * K / (pre[label] / 1e3) / 1e12
        del gw, gws, gx, gxs
    out["prefill"] = pre
    del qv, meta, values, x, xq, y, ws
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- layer sweep
def run_layers(args, torch, np, sp, W, ev, dev):
    """Layer sweep: 32 layers x (QKV, O, gate+up, down) of a Llama-3-8B-sized block at 256
    tokens, 128 sequential sparse GEMMs per step on weights pruned, compressed and (FP8)
    quantised once at load, and the same 128 products on dense MFMA over the decompressed
    pruned weights.  Weights are drawn on the GPU from seeded generators (seed
    5000 + 4*layer + projection, 0.02 * N(0, 1)); the two inputs X [256, 4096] ~ N(0, 1) and
    [256, 14336] ~ SiLU(N(0, 1)) come from workloads/ and are quantised once.  The whole
    sweep (4.4 GB of FP8 weights) exceeds the last-level cache, so no weight copies."""
    kind = "fp8" if args.dtype == "fp8" or args.workload == "all" else args.dtype
    fp8 = kind == "fp8"
    dt = sp.FP8 if fp8 else sp.BF16
    M, L = W.LAYER_M, W.N_LAYERS
    projs = W.LAYER_PROJS
    xs, xq, sx = {}, {}, {}
    for _, k, _ in projs:
        if k not in xs:
            xs[k] = W.layer_x(k).to(dev)
            if fp8:
                xq[k], sx[k] = sp.quant_fp8(xs[k])
            else:
                xq[k], sx[k] = xs[k], None
    t0 = time.perf_counter()
    wts = []
    for layer in range(L):
        row = []
        for p, (name, k, n) in enumerate(projs):
            g = torch.Generator(device=dev)
            g.manual_seed(5000 + 4 * layer + p)
            w = (torch.randn(n, k, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            values, meta = sp.prune_compress(w)
            del w
            qv, sw = sp.quant_fp8(values) if fp8 else (values, None)
            row.append((qv, meta, sw))
            del values
        wts.append(row)
    torch.cuda.synchronize()
    load_s = time.perf_counter() - t0
    ys = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for _, _, n in projs]
    wss = [torch.empty(max(16, sp.workspace_size(sp.OP_GEMM, dt, M, n, k)), dtype=torch.uint8,
                       device=dev) for _, k, n in projs]
    plans = [sp.plan(sp.OP_GEMM, dt, M, n, k) for _, k, n in projs]

    def call(layer, p):
        _, k, _ = projs[p]
        qv, meta, sw = wts[layer][p]
        sp.gemm(xq[k], qv, meta, x_scale=sx[k], w_scale=sw, out=ys[p], ws=wss[p])

    def sweep():
        for layer in range(L):
            for p in range(len(projs)):
                call(layer, p)

    sweep()
    torch.cuda.synchronize()
    eager = [y.clone() for y in ys]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sweep()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sweep()
    torch.cuda.synchronize()
    warmup = min(args.warmup, 10)
    for _ in range(warmup):
        graph.replay()
    steps = max(1, min(args.steps, 30))
    t = ev.time(lambda i: graph.replay(), steps) / steps
    graph.replay()
    torch.cuda.synchronize()
    for p in range(len(projs)):
        if not torch.equal(ys[p].view(torch.int16), eager[p].view(torch.int16)):
            raise SystemExit("graph replay output differs from the eager run for %s" % projs[p][0])
    del graph

    per_proj, tot_b, tot_t = {}, 0, 0.0
    for p, (name, k, n) in enumerate(projs):
        tp = ev.graph(lambda i: call(i % L, p), L, replays=5)
        b = gemm_bytes(M, n, k, fp8)
        tot_b += b * L
        tot_t += tp * L
        per_proj[name] = {"K": k, "N": n, "gemm_us": tp * 1e6, "GBs": b / tp / 1e9,
                          "hbm_frac": b / tp / 1e9 / HBM_PEAK_GBS,
                          "tflops_dense_equiv": 2 * M * n * k / tp / 1e12,
                          "plan": {k2: v for k2, v in plans[p].items()
                                   if k2 in ("kernel", "config", "tile_n", "tile_m", "waves", "split_k")}}
    sweep_bytes = sum(gemm_bytes(M, n, k, fp8) for _, k, n in projs) * L

    dense = None
    if not args.no_dense:
        # the same products on dense MFMA over the decompressed pruned weights
        wd = [[sp.decompress(wts[layer][p][0], wts[layer][p][1], projs[p][1]) for p in range(len(projs))]
              for layer in range(L)]
        dws = [torch.empty(max(16, sp.workspace_size(sp.OP_DENSE_GEMM, dt, M, n, k)), dtype=torch.uint8,
                           device=dev) for _, k, n in projs]

        def dcall(layer, p):
            _, k, _ = projs[p]
            sp.dense_gemm(xq[k], wd[layer][p], x_scale=sx[k], w_scale=wts[layer][p][2], out=ys[p], ws=dws[p])

        def dsweep():
            for layer in range(L):
                for p in range(len(projs)):
                    dcall(layer, p)
        dt_sweep = ev.graph(lambda i: dsweep(), 1, replays=max(3, min(args.steps, 20)))
        dense = {"sweep_ms": dt_sweep * 1e3, "sparse_speedup_vs_dense": dt_sweep / t,
                 "GBs": sum(dense_bytes(M, n, k, fp8) for _, k, n in projs) * L / dt_sweep / 1e9}
        for p, (name, k, n) in enumerate(projs):
            tp = ev.graph(lambda i: dcall(i % L, p), L, replays=5)
            per_proj[name]["dense_gemm_us"] = tp * 1e6
            per_proj[name]["sparse_speedup_vs_dense"] = tp / (per_proj[name]["gemm_us"] / 1e6)
        del wd, dws
    achieved = tot_b / tot_t / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_layer_baseline(W, fp8, gemm_bytes(M, 4096, 4096, fp8))
    label = "FP8-E4M3 (per-tensor scales)" if fp8 else "BF16"
    return {"kind": kind, "M": M, "L": L, "projs": projs, "steps": steps, "warmup": warmup, "t": t,
            "sweep_bytes": sweep_bytes, "per_proj": per_proj, "dense": dense, "cpu": cpu, "load_s": load_s,
            "desc": "layer sweep: %d layers x QKV/O/gate+up/down, M=%d tokens, 2:4 sparse %s" % (L, M, label),
            "flops": sum(2 * M * n * k for _, k, n in projs) * L,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "traffic": counted_traffic("layers", "sweep") if kind == "fp8" else None,
                         "kernel": "%s (sparse %s), all 128 calls" % (
                             "/".join(sorted({KERNEL_NAMES[pl["kernel"]] for pl in plans})), kind),
                         "per_unit": "values N*K/2*es + metadata N*K/8 + X M*K*es + Y 2*M*N bytes per launch"},
            "device": torch.cuda.get_device_name(dev)}


def layers_line(args, d):
    return {
        "metric": METRIC,
        "value": d["sweep_bytes"] / d["t"] / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": d["steps"], "warmup": d["warmup"], "ms_per_step": d["t"] * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if d["kind"] == "fp8" else "bf16",
        "data": "synthetic (seeded; weights drawn on the GPU, inputs from workloads/)",
        "config": {"workload": d["desc"], "M": d["M"], "layers": d["L"], "projections": [list(pr) for pr in d["projs"]],
                   "step": "128 sequential sparse GEMMs (X quantised once)"},
        "roofline": d["roofline"], "cpu_baseline": d["cpu"], "per_projection": d["per_proj"],
        "dense_sweep": d["dense"], "sweep_GB": d["sweep_bytes"] / 1e9,
        "sweep_tflops_dense_equiv": d["flops"] / d["t"] / 1e12,
        "load_path": {"generate_prune_compress_quantise_s": d["load_s"]}, "device": d["device"],
    }


def config_summary_layers(d):
    return {"workload": d["desc"], "sweep_ms": d["t"] * 1e3, "sweep_GBs": d["sweep_bytes"] / d["t"] / 1e9,
            "roofline": d["roofline"], "dense_sweep": d["dense"], "cpu_baseline": d["cpu"],
            "sweep_tflops_dense_equiv": d["flops"] / d["t"] / 1e12, "per_projection": d["per_proj"]}


def cpu_layer_baseline(W, fp8, call_bytes):
    """The CPU oracle on one call of the sweep (layer 0's O projection, 256 x 4096 x 4096),
    repeated for about 5 s."""
    from oracle import sp24_ref as O
    wb = W.bf16_bits(W.layer_weight(0, 1))
    xb = W.bf16_bits(W.layer_x(4096))
    v, meta = O.prune_compress(wb)
    if fp8:
        vq, sw = O.quant_fp8(v)
    reps, t0 = 0, time.perf_counter()
    while True:
        if fp8:
            xq, sx = O.quant_fp8(xb)
            O.gemm_ref(*O.sparse_operands_fp8(xq, sx, vq, meta, sw, 4096))
        else:
            O.gemm_ref(*O.sparse_operands_bf16(xb, v, meta, 4096))
        reps += 1
        el = time.perf_counter() - t0
        if el > 5.0 or reps >= 20:
            break
    return {"value": call_bytes * reps / el / 1e9, "unit": "GB/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": "%d call(s) of layer 0's O projection (256 x 4096 x 4096: quantise X, "
                      "decompress W, float64 product and magnitude sum), %.1f s wall" % (reps, el)}


def cpu_baseline(w_cpu, xs_cpu, Ms, N, K, kind, step_bytes):
    """The CPU oracle's per-call path on the same inputs: quantise X and the float64
    product over the decompressed weight, one full step (all M) per repetition, for
    about 8 s."""
    import workloads as W
    from oracle import sp24_ref as O
    wb = W.bf16_bits(w_cpu)
    v, meta = O.prune_compress(wb)            # load path, not timed
    if kind == "fp8":
        vq, sw = O.quant_fp8(v)
    elif kind == "int8":
        vq, sw = O.quant_int8(v)
    xb = {m: W.bf16_bits(xs_cpu[m]) for m in Ms}
    reps, t0 = 0, time.perf_counter()
    while True:
        for m in Ms:
            if kind == "fp8":
                xq, sx = O.quant_fp8(xb[m])
                O.gemm_ref(*O.sparse_operands_fp8(xq, sx, vq, meta, sw, K))
            elif kind == "int8":
                xq, sx = O.quant_int8(xb[m])
                O.gemm_ref(*O.sparse_operands_int8(xq, sx, vq, meta, sw, K))
            else:
                O.gemm_ref(*O.sparse_operands_bf16(xb[m], v, meta, K))
        reps += 1
        el = time.perf_counter() - t0
        if el > 8.0 or reps >= 20:
            break
    return {"value": step_bytes * reps / el / 1e9, "unit": "GB/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": "%d full step(s) of the same workload (quantise X, decompress W, float64 "
                      "product and magnitude sum for M=%s), %.1f s wall" % (
                          reps, "/".join(map(str, Ms)), el)}


if __name__ == "__main__":
    main()
