"""CPU oracle for the 2:4 sparse GEMM path and the BF16 exponent-palette weight
format -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The HIP library never imports, links or calls it.
"""
from .sp24_ref import *  # noqa: F401,F403
from . import sp24_ref  # noqa: F401
from . import palette_ref  # noqa: F401
