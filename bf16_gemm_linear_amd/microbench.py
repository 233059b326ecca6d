"""Measured ceilings of the device: HBM stream rates and matrix-instruction rates.

    python -m bf16_gemm_linear_amd.microbench

Prints one JSON object:
  * hbm_read_GBs[size]: sp24_probe_read over `size` bytes, rotating over enough
    buffers that every read misses the 256 MB last-level cache;
  * hbm_copy_GBs: sp24_probe_copy of 512 MiB (bytes read + bytes written);
  * mfma_tflops[variant]: sp24_probe_mfma_rate with every SIMD busy, in
    dense-equivalent flops per second (sparse variants count the full K), and
    the implied clock assuming the instruction's nominal cycle count.

    python -m bf16_gemm_linear_amd.microbench --ring

Prints one JSON object with the load path of the LDS-ring GEMM kernels
(sp24_probe_ring, one workgroup of 8 waves per CU, 128 steps): per shape (KB of
W and of X per step, buffers, barrier) the time of one launch (best of 5) and
the KB per microsecond per CU, W streamed from HBM (1 GB in all, a fresh part
per launch), X from L2.
"""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import bf16_gemm_linear_amd as sp  # noqa: E402

LLC = 256 << 20

# variant -> (name, dense-equivalent flops per instruction per wave, nominal cycles per instruction)
VARIANTS = {
    0: ("smfmac_f32_16x16x128_fp8", 2 * 16 * 16 * 128, 16),
    1: ("smfmac_f32_16x16x64_bf16", 2 * 16 * 16 * 64, 16),
    3: ("smfmac_f32_32x32x64_fp8", 2 * 32 * 32 * 64, 32),
    4: ("smfmac_f32_32x32x32_bf16", 2 * 32 * 32 * 32, 32),
    6: ("mfma_f32_16x16x128_f8f6f4(fp8)", 2 * 16 * 16 * 128, 32),
    7: ("mfma_f32_16x16x32_bf16", 2 * 16 * 16 * 32, 16),
    8: ("smfmac_i32_16x16x128_i8", 2 * 16 * 16 * 128, 16),
    9: ("smfmac_i32_32x32x64_i8", 2 * 32 * 32 * 64, 32),
    10: ("mfma_i32_16x16x64_i8", 2 * 16 * 16 * 64, 16),
    11: ("mfma_i32_32x32x32_i8", 2 * 32 * 32 * 32, 32),
}


def _time(fn, reps):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(reps):
        fn(i)
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / 1e3


def hbm_read(size):
    n = max(1, -(-int(2.2 * LLC) // size))
    bufs = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(n)]
    out = torch.empty(sp.lib.sp24_probe_read_blocks(), dtype=torch.int32, device="cuda")
    for b in bufs:
        sp.probe_read(b, out)
    reps = max(n * 4, 40)
    t = _time(lambda i: sp.probe_read(bufs[i % n], out), reps) / reps
    return size / t / 1e9, t


def hbm_copy(size=512 << 20):
    a = torch.empty(size, dtype=torch.uint8, device="cuda")
    b = torch.empty(size, dtype=torch.uint8, device="cuda")
    sp.probe_copy(a, b)
    t = _time(lambda i: sp.probe_copy(a, b), 10) / 10
    return 2 * size / t / 1e9, t


def mfma_rate(variant, cus):
    name, flops, cycles = VARIANTS[variant]
    blocks, waves, iters = cus * 4, 4, 4096
    out = torch.empty(blocks * waves * 64, dtype=torch.float32, device="cuda")
    sp.probe_mfma_rate(variant, 16, blocks, waves, out)
    t = _time(lambda i: sp.probe_mfma_rate(variant, iters, blocks, waves, out), 3) / 3
    instr = blocks * waves * iters * 4
    tflops = instr * flops / t / 1e12
    # each SIMD runs blocks*waves/(4*cus) waves back to back
    per_simd = instr / (cus * 4)
    clock_ghz = per_simd * cycles / t / 1e9
    return name, tflops, clock_ghz


RING_SHAPES = [(8, 16, 4, True), (8, 16, 4, False), (8, 16, 6, True), (8, 0, 4, True), (24, 0, 4, True),
               (0, 16, 4, True), (0, 24, 4, True)]


def ring(cus):
    steps, w_stride = 128, 4 << 20
    w = torch.empty(cus * w_stride, dtype=torch.uint8, device="cuda")
    x = torch.empty(8 * (256 << 10), dtype=torch.uint8, device="cuda")
    w.fill_(1)
    x.fill_(1)
    out = torch.empty(cus, dtype=torch.int32, device="cuda")
    res = {}
    for w_kb, x_kb, stages, bar in RING_SHAPES:
        per = steps * max(w_kb, 1) << 10  # W bytes of one launch per workgroup
        parts = w_stride // per            # each launch reads a fresh part of every region

        def launch(i):
            wv = w[(i % parts) * per:]
            sp.probe_ring(w_kb, x_kb, stages, bar, wv, w_stride, x, cus, steps, out)
        launch(0)
        t = min(_time(launch, 1) for _ in range(5))
        per_cu = steps * (w_kb + x_kb) / (t * 1e6)  # KB per microsecond per CU
        key = "W%d_X%d_S%d_%s" % (w_kb, x_kb, stages, "bar" if bar else "nobar")
        res[key] = {"us": t * 1e6, "KB_per_us_per_CU": per_cu,
                    "W_TBs": cus * steps * w_kb * 1024 / t / 1e12}
    return res


def main():
    if "--ring" in sys.argv:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        print(json.dumps({"ring": ring(cus), "compute_units": cus}))
        return
    if "--copy-only" in sys.argv:  # reference kernel of known traffic, for counter scaling
        gbs, t = hbm_copy(256 << 20)
        print(json.dumps({"copy_bytes_read": 256 << 20, "copy_bytes_written": 256 << 20,
                          "copy_GBs": gbs, "launches": 11}))
        return
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    res = {"device": props.name, "compute_units": cus, "hbm_read_GBs": {}, "mfma_tflops": {},
           "implied_clock_GHz": {}}
    for size in (36 << 20, 128 << 20, 1 << 30):
        gbs, t = hbm_read(size)
        res["hbm_read_GBs"][str(size)] = gbs
    res["hbm_copy_GBs"], _ = hbm_copy()
    for v in VARIANTS:
        name, tf, clk = mfma_rate(v, cus)
        res["mfma_tflops"][name] = tf
        res["implied_clock_GHz"][name] = clk
    print(json.dumps(res))


if __name__ == "__main__":
    main()
