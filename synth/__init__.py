"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds shapes, random draws and block-table structure only --
none of the attention, addressing or quantization arithmetic.  Both the HIP
library and the CPU oracle consume what it produces.
"""

from .workloads import (  # noqa: F401
    Config,
    CONFIGS,
    Structure,
    structure,
    layer_structures,
    host_normal,
    device_normal_,
    decode_positions,
    prefill_tokens,
)
