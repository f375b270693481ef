"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark."""
from .gen import (  # noqa: F401
    CONFIGS,
    dense_case,
    varlen_lengths,
    varlen_case,
    decode_lengths,
    decode_case,
    append_case,
    rotary_tables,
    hadamard_signs,
    config_case,
)
