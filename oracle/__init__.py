"""fp64 CPU oracle for decode attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the bench's CPU-baseline leg
import this package; the HIP library and its Python binding never do.
"""

from .fp64 import (  # noqa: F401
    attention,
    attention_fp8kv,
    bifurcated_attention,
    bifurcated_paged_attention,
    default_scale,
    fp8_e4m3_value,
    lse_combine,
    paged_attention,
    prefill_attention,
    split_partials,
)
