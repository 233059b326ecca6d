"""Write tests/golden/tiny_oracle.txt: digests of the oracle's outputs on the
tiny workload (X[8,256], W[256,256], seed 0).

Calls only the oracle and the seeded input generators.  The stored digests pin
the oracle against unintended changes; a deliberate change of its arithmetic
must regenerate this file in the same commit and say why.
Run: python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as W  # noqa: E402
from oracle import sp24_ref as O  # noqa: E402


def digest(a):
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.tobytes()).hexdigest()


def tiny_records():
    x, w = W.tiny()
    xb, wb = W.bf16_bits(x), W.bf16_bits(w)
    mask = O.prune_mask(wb)
    values, meta = O.compress(wb, mask)
    xq, sx = O.quant_fp8(xb)
    vq, sw = O.quant_fp8(values)
    ref_bf16, mag_bf16 = O.gemm_ref(*O.sparse_operands_bf16(xb, values, meta, 256))
    ref_fp8, _ = O.gemm_ref(*O.sparse_operands_fp8(xq, sx, vq, meta, sw, 256))
    rec = {
        "x_bits": digest(xb), "w_bits": digest(wb),
        "mask": digest(mask.astype(np.uint8)), "values": digest(values), "meta": digest(meta),
        "meta_row0": " ".join("%08x" % int(v) for v in meta[0]),
        "xq": digest(xq), "x_scale": "%08x" % int(np.float32(sx).view(np.uint32)),
        "vq": digest(vq), "w_scale": "%08x" % int(np.float32(sw).view(np.uint32)),
        "ref_bf16_00": repr(float(ref_bf16[0, 0])), "ref_bf16_sum": repr(float(ref_bf16.sum())),
        "mag_bf16_sum": repr(float(mag_bf16.sum())),
        "ref_fp8_00": repr(float(ref_fp8[0, 0])), "ref_fp8_sum": repr(float(ref_fp8.sum())),
    }
    return rec


if __name__ == "__main__":
    rec = tiny_records()
    with open(os.path.join(HERE, "tiny_oracle.txt"), "w") as f:
        f.write("# oracle outputs on the tiny workload; written by tests/golden/make_golden.py\n")
        for k, v in rec.items():
            f.write("%s %s\n" % (k, v))
    print("wrote", len(rec), "records")
