"""CPU fp64 oracle for exact attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The HIP path never imports or calls it, and the two share
no code; only the seeded input generators in ``workloads`` serve both.

Every function follows the plain definition of attention written out in float64
(see ``oracle.attention`` for the page citations of each step).  Every function here
is pinned by the CPU tests in ``tests/test_oracle_*.py`` against closed forms,
invariants, an independent library routine or brute force; none is "parity unpinned".
``oracle.fp8`` (the E4M3 format, block quantisation and attention on dequantised
tensors) is imported by name; it is pinned by ``tests/test_oracle_fp8.py``.
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_rows,
    backward_cols_dkdv,
    backward_rows_dq,
    block_state,
    blockwise_forward,
    finalize_state,
    initial_state,
    merge_lse_partials,
    merge_states,
    streaming_rows,
)
