"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This package only draws random numbers and lays bytes out in the paged cache format; it holds none
of the attention arithmetic. Both the CPU oracle (through the logical, unpaged rows) and the HIP
path (through the paged cache and block table) are fed from here.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    SUPPLEMENTARY,
    Spec,
    Workload,
    cache_layout,
    make,
    make_on_device,
)
