"""Oracle for the fused multi-head attention backward (test infrastructure only).

This package is a plain, slow, fp64 CPU statement of what the GPU path computes: the
forward of softmax attention (O and its log-sum-exp) and the exact gradient of O with
respect to Q, K and V for a given upstream gradient dO.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product library never
does, and it shares no code with the HIP path.

Every function is pinned by the CPU tests in ``tests/test_oracle.py`` against finite
differences, an independent library implementation (torch fp64 SDPA + autograd) on the
cases where it applies, closed forms and exact identities.  The dropout generator (Philox,
written once for any word size) is pinned bit-exactly at 64-bit words against numpy's
Philox4x64-10; the 32-bit variant the dropout uses differs only in its published constants.
Nothing here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    MASK_NONE,
    MASK_CAUSAL_TOP_LEFT,
    MASK_CAUSAL_BOTTOM_RIGHT,
    MASK_WINDOW,
    mask_geometry,
    allowed,
    forward,
    backward,
    row_statistics,
    dq_rows,
    dkdv_rows,
    dq_split_reduce,
    rowsum_product,
)
