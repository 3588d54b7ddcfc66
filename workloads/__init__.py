"""Seeded synthetic shared-prefix decode batches.

This package only draws inputs: block tables, sequence lengths, the paged K/V
pool and the decode queries, plus the prefix forest that each batch was built
from.  It holds none of the attention or grouping arithmetic; both the CPU
oracle and the HIP path consume what it produces.
"""

from .forest import (  # noqa: F401
    CONFIGS,
    AttnShape,
    Batch,
    build_batch,
    config_by_name,
)
from .values import (  # noqa: F401
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    fill_values_numpy,
    BF16_NAN,
)
