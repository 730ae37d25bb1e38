"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds workload shapes and random-number generation only. It
contains none of the attention arithmetic: no scores, no softmax, no masks.
"""

from .inputs import (  # noqa: F401
    CONFIGS,
    PrefillConfig,
    DecodeConfig,
    prefill_inputs,
    decode_inputs,
    gen_normal,
    seed_key,
)
