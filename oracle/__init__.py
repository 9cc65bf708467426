"""fp64 CPU oracle for the max-shifted log-sum-exp family.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the HIP path in ``log_softmax_reductions_amd`` and
neither imports the other.  See ``oracle.c`` for the definitions and the
passages of the pages each one follows.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    lse_axis0,
    log_softmax_rows,
    softmax_rows,
    lse_axis,
    log_softmax_axis,
    lse_chunk_partials,
    lse_merge,
    hardswish,
    conv2d,
    fused_chain,
    max_threads,
)
