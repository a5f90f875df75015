"""CPU reference GEMM in float64.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library (``oracle.c`` is
built by the host C compiler on its own); the product path never calls it.

Parity pins: every function here is pinned by ``tests/test_oracle.py`` against
closed forms, exact rational arithmetic, identity/permutation products, the
worked 4x6 . 6x4 block decomposition and planted mistakes.  Values of large
random products have no printed counterpart on the source pages; for those the
oracle's own fp64 result is the reference (no further pin exists).

``oracle.softmax`` is the float64 row softmax (numpy only), pinned by
``tests/test_softmax_oracle.py`` against closed forms, the logistic function,
scipy's softmax, degenerate rows and planted mistakes.
"""
from .oracle import (  # noqa: F401
    EPI_NONE, EPI_LEAKY_RELU, gemm_full, gemm_points, to_f64, scaled, tolerance, check,
    plant_fault, load, default_threads,
)
from . import softmax  # noqa: F401,E402
