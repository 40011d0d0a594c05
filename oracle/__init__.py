"""CPU oracle for fused multi-head attention forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The GPU product path never calls it, links it or falls
back to it.  It shares no code with the HIP implementation; the only module both
sides use is ``mha_inputs`` (seeded random draws, no attention arithmetic).

Contents:
  * :mod:`oracle.attention` -- the plain two-pass definition of softmax attention
    in float64 (what the fused kernel must reproduce up to rounding);
  * :mod:`oracle.online` -- the tiled online-softmax recurrence in float64, step for
    step as the FlashAttention-2 algorithm states it, used to check readings of the
    algorithm (deferred normalisation, masked tiles) on the CPU;
  * :mod:`oracle.paged` -- attention over a paged key/value cache (keys reached
    through a block table), the plain definition applied to the gathered keys;
  * :mod:`oracle.matmul` -- the dense matrix product and the error bound of a float32
    accumulated, once-rounded result.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force in
40-digit decimal arithmetic, a library attention routine in float64, closed forms
and invariants.
"""
from .attention import (  # noqa: F401
    decode,
    attention_forward,
    attention_rows,
)
from .online import attention_forward_tiled  # noqa: F401
from .paged import gather_keys, paged_attention_forward  # noqa: F401
from .matmul import gemm, gemm_error_bound  # noqa: F401
