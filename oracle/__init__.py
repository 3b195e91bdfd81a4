"""CPU oracle of the segment-routed multi-adapter LoRA delta.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never does, and
this package never imports the GPU library.
"""

from .oracle import (  # noqa: F401
    OracleError,
    bf16_round,
    bf16_to_f64,
    build,
    delta,
    library_path,
    pack_adapter,
    pack_family,
    pack_bias,
    reference_family,
    route,
    scaling,
    stack_to_f64,
)
from .slot_cache import OracleSlotCache, SlotCacheError  # noqa: F401,E402
