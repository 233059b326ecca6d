"""Summaries of rocprofv3 runs of bench.py for profiles/ (markdown on stdout).

    python -m bf16_gemm_linear_amd.profile_summary trace DIR
        kernel table of a `rocprofv3 --kernel-trace --stats --output-format csv` run:
        calls, mean / min / max duration, share of GPU time, per-launch p50 and p99,
        and each stream-kernel configuration spelled out
    python -m bf16_gemm_linear_amd.profile_summary traffic WORKLOAD FETCH_DIR WRITE_DIR COPY_FETCH_DIR \
            COPY_WRITE_DIR COPY_BYTES KERNEL_SUBSTRING [KERNEL_SUBSTRING ...]
        HBM bytes per launch of the kernels whose names contain every one of the substrings, from
        a FETCH_SIZE run and a WRITE_SIZE run, each scaled by what the counter reads for a
        copy of COPY_BYTES bytes (FETCH_SIZE and WRITE_SIZE are in KiB per dispatch), and
        the machine-readable traffic record bench.py reads (tied to the hash of the
        sources of the kernel family: the stream kernel for up/down, the tiled one for
        prefill, both with the split-K reduction for the layer sweep)
    python -m bf16_gemm_linear_amd.profile_summary counters DIR [KERNEL_SUBSTRING ...]
        mean, min and max per dispatch of every counter of a `--pmc` run, per kernel

rocprofv3 writes its CSV files below the -d directory (host and process folders); every
file of the wanted kind below DIR is read.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "bf16_gemm_linear_amd/csrc/"
SOURCES = {
    "hbm": [CSRC + f for f in ("sp24_gemm_stream.hip", "sp24_dma.hpp", "sp24_common.hpp", "sp24_internal.hpp",
                               "sp24_api.hip")],
    "mfma": [CSRC + f for f in ("sp24_gemm_tiled.hip", "sp24_dma.hpp", "sp24_common.hpp", "sp24_internal.hpp",
                                "sp24_api.hip")],
    "sweep": [CSRC + f for f in ("sp24_gemm_stream.hip", "sp24_gemm_tiled.hip", "sp24_gemm_tiled128.hip",
                                 "sp24_reduce.hip", "sp24_dma.hpp", "sp24_common.hpp", "sp24_internal.hpp",
                                 "sp24_api.hip")],
}
BOUND = {"prefill": "mfma", "layers": "sweep"}  # the source set of each workload's record (else "hbm")
DT_NAMES = {"0": "BF16", "1": "FP8", "2": "INT8"}


def source_hash(bound):
    h = hashlib.sha256()
    for f in SOURCES[bound]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(pattern, d):
    out = []
    for path in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(path, newline="") as fh:
            out += list(csv.DictReader(fh))
    if not out:
        raise SystemExit("no %s below %s" % (pattern, d))
    return out


def short_name(name):
    """Kernel name without the return type, the namespaces and the argument list."""
    name = name.replace("sp24::(anonymous namespace)::", "").replace("sp24::", "")
    name = re.sub(r"\([^()]*\)\s*$", "", name.strip())
    return re.sub(r"^void\s+", "", name).strip()


def describe_tiled(name):
    """Words for gemm_tiled_kernel<DT, SPARSE, PARTIAL, ROWS>."""
    m = re.search(r"gemm_tiled_kernel<(\d+), (true|false), (true|false), (\d+)>", name)
    if not m:
        return None
    dt, sparse, partial, rows = m.groups()
    return ("%s %s; %s W rows x 256 tokens per workgroup, 8 waves of %s x 64 outputs, 32 x 32 instructions%s"
            % (DT_NAMES.get(dt, dt), "sparse" if sparse == "true" else "dense", rows, int(rows) // 2,
               "; K split over the grid (fp32 partial tiles)" if partial == "true" else ""))


def describe_stream(name):
    """Words for StreamCfg<DT, SPARSE, RBW, RB, MW, KW, MB, U, SMAX[, BUDGET]> (or a tiled kernel)."""
    m = re.search(r"StreamCfg<(\d+), (true|false), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)", name)
    if not m:
        return describe_tiled(name)
    dt, sparse, rbw, rb, mw, kw, mb, u, smax = m.groups()
    rbw, rb, mw, kw, mb, u, smax = map(int, (rbw, rb, mw, kw, mb, u, smax))
    return ("%s %s; %d waves = %d along the rows x %d along the tokens x %d along K; each wave %d row "
            "block(s) of 16 x %d token block(s) of 16 over %d unit(s) of 128 K per step; %d rows and %d tokens "
            "per workgroup; at most %d LDS buffers"
            % (DT_NAMES.get(dt, dt), "sparse" if sparse == "true" else "dense", rbw * mw * kw, rbw, mw, kw, rb, mb,
               u, 16 * rbw * rb, 16 * mw * mb, smax))


def _durations(rows):
    per = {}
    for r in rows:
        k = short_name(r.get("Kernel_Name") or r.get("KernelName") or r["Kernel-Name"])
        t0, t1 = int(r.get("Start_Timestamp") or r["Start-Timestamp"]), int(r.get("End_Timestamp") or
                                                                           r["End-Timestamp"])
        per.setdefault(k, []).append((t1 - t0) / 1e3)
    return per


def pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def trace(d):
    per = _durations(_rows("*kernel_trace.csv", d))
    total = sum(sum(v) for v in per.values())
    print("| kernel | calls | avg us | min us | max us | p50 us | p99 us | % of GPU time |")
    print("|---|---|---|---|---|---|---|---|")
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print("| `%s` | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.1f |"
              % (k, len(v), statistics.mean(v), min(v), max(v), pct(v, 0.5), pct(v, 0.99), 100 * sum(v) / total))
    seen = [k for k in per if describe_stream(k)]
    if seen:
        print()
        for k in seen:
            print("- `%s`: %s" % (k, describe_stream(k)))


def _counter(d, counter, subs, every=False):
    rows = _rows("*counter_collection.csv", d)
    per = {}
    for r in rows:
        name = r.get("Counter_Name") or r["Counter-Name"]
        if name != counter:
            continue
        k = short_name(r.get("Kernel_Name") or r["Kernel-Name"])
        if subs and not (all if every else any)(s in k for s in subs):
            continue
        disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or r.get("Correlation_Id")
        per.setdefault(k, {}).setdefault(disp, 0.0)
        per[k][disp] += float(r.get("Counter_Value") or r["Counter-Value"])
    return {k: list(v.values()) for k, v in per.items()}


def counters(d, subs):
    rows = _rows("*counter_collection.csv", d)
    names = sorted({r.get("Counter_Name") or r["Counter-Name"] for r in rows})
    print("| kernel | counter | dispatches | mean | min | max |")
    print("|---|---|---|---|---|---|")
    for c in names:
        for k, v in sorted(_counter(d, c, subs).items()):
            print("| `%s` | %s | %d | %.10g | %.10g | %.10g |" % (k, c, len(v), statistics.mean(v), min(v), max(v)))


def traffic(workload, fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes, subs):
    copy_kib = copy_bytes / 1024.0
    cf = _counter(cfetch_dir, "FETCH_SIZE", ["copy"])
    cw = _counter(cwrite_dir, "WRITE_SIZE", ["copy"])
    fscale = copy_kib / statistics.mean(next(iter(cf.values())))
    wscale = copy_kib / statistics.mean(next(iter(cw.values())))
    f = _counter(fetch_dir, "FETCH_SIZE", subs, every=True)
    w = _counter(write_dir, "WRITE_SIZE", subs, every=True)
    print("Copy of %d bytes: FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f." % (copy_bytes, fscale, wscale))
    print()
    print("| kernel | launches | fetched MB / launch | written MB / launch |")
    print("|---|---|---|---|")
    tot, n = 0.0, 0
    for k in sorted(set(f) | set(w)):
        fb = statistics.mean(f.get(k, [0.0])) * 1024 * fscale
        wb = statistics.mean(w.get(k, [0.0])) * 1024 * wscale
        print("| `%s` | %d | %.2f | %.3f |" % (k, len(f.get(k, [])), fb / 1e6, wb / 1e6))
        nk = len(f.get(k, []))
        tot += (fb + wb) * nk
        n += nk
    bound = BOUND.get(workload, "hbm")
    rec = {"workload": workload, "kernel_source_sha256": source_hash(bound), "traffic_bytes_per_launch": tot / n,
           "fetch_scale": fscale, "write_scale": wscale}
    print()
    print("Mean over the launches above: %.2f MB of HBM traffic per launch." % (tot / n / 1e6))
    print()
    print("traffic-record: " + json.dumps(rec))


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        trace(argv[1])
    elif len(argv) >= 8 and argv[0] == "traffic":
        traffic(argv[1], argv[2], argv[3], argv[4], argv[5], int(argv[6]), argv[7:])
    elif len(argv) >= 2 and argv[0] == "counters":
        counters(argv[1], argv[2:])
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
