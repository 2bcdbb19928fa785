"""Seeded synthetic inputs for one paged-attention step.

This package only *describes* workloads: sequence lengths, the initial order
of the free-block queue, the order in which requests ask the allocator for
blocks, and the Q/K/V element values.  It holds none of the method's
arithmetic: no block allocation, no cache scatter, no attention.  Both the
HIP path (through its Python binding) and the fp64 oracle consume it, each
running the allocation script against its own block pool.
"""
from .configs import (  # noqa: F401
    PREFIX_KEY,
    Request,
    StepSpec,
    CONFIG_NAMES,
    make_config,
    random_spec,
    allocation_script,
)
from .values import (  # noqa: F401
    value_table,
    kv_rows,
    q_rows,
    kv_values,
    q_values,
    kv_key_for,
    poison_bits,
)
from .step import StepMeta, run_allocation_script, step_rows  # noqa: F401
from .engine import EngineConfig, EngineLoop, EngineRequest, EngineStep  # noqa: F401
