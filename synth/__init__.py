"""Seeded synthetic workloads for certified sparse attention.

This package only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path (through
its Python binding) consume the same arrays produced here.
"""

from .workloads import (  # noqa: F401
    Workload,
    HASH_SEED,
    config1,
    config2,
    peaked_head,
    config3_layer,
    config4_request,
    config5_base,
    config5_step_query,
    recipe_layer,
)
