"""CPU reference (the oracle) for attention forward -- TEST INFRASTRUCTURE.

Only the test suite, the package entry file's smoke check and the benchmark's
CPU-baseline leg may import this package.  The HIP library never imports it,
links it or calls it, and the two share no code.

* :mod:`oracle.sdpa`       -- NumPy float64: materialised-score definition,
  online (tiled) recurrence, split partial + log-sum-exp merge, paged decode,
  varlen paged prefill, per-row log-sum-exp and the backward pass.
* :mod:`oracle.bruteforce` -- pure-Python 50-digit decimal statement of the same
  definition, for tiny inputs.
"""
from .sdpa import (  # noqa: F401
    admissible,
    admissible_pair_count,
    attention_partial_f64,
    kv_head_of,
    lse_merge_f64,
    paged_decode_f64,
    paged_prefill_varlen_f64,
    paged_gather,
    query_positions,
    sdpa_naive_f64,
    sdpa_online_f64,
    sdpa_lse_f64,
    sdpa_backward_f64,
    transform_scores,
)
