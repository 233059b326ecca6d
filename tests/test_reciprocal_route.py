"""Host proof that the quantisers' reciprocal route codes exactly as the IEEE division.

The GPU quantisers take the per-tensor, per-token and per-group E4M3 / INT8 quotient
v / s of a dynamic scale (s from the data's own largest magnitude) as v * fp32(1/s)
plus one correction by the exact residual, when amax >= 2^-63 (bf16 key 0x2000).
`reciprocal_route.c` compares the resulting codes with those of the correctly rounded
quotient, which the oracle uses, over every (amax, v) pair with |v| <= amax: there must
be no difference from key 0x2000 up.  Below that key the route does differ, which is why
the kernels divide there.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("recip") / "reciprocal_route")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe,
                    os.path.join(HERE, "reciprocal_route.c"), "-lm"], check=True)
    return exe


def _run(exe, kind, kmin):
    out = subprocess.run([exe, kind, kmin], check=True, capture_output=True, text=True,
                         env=dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))).stdout
    m = re.search(r"(\d+) pairs, (\d+) codes differ, (\d+) keys", out)
    assert m, out
    return int(m.group(1)), int(m.group(2)), int(m.group(3))


@pytest.mark.parametrize("kind", ["e4m3", "int8"])
def test_reciprocal_route_codes_equal_division_codes_from_key_0x2000(checker, kind):
    pairs, differ, abnormal = _run(checker, kind, "2000")
    assert pairs > 900_000_000 and abnormal == 0
    assert differ == 0


def test_reciprocal_route_differs_for_tiny_maxima(checker):
    # the threshold is needed: with amax of 2^-100 and below, some codes differ (a
    # subnormal residual is not exact)
    _, differ, _ = _run(checker, "e4m3", "0001")
    assert differ > 0
