"""Seeded synthetic workloads for the DSA hot path (shared by the tests, the smoke check and the bench).

This package holds random draws, dtype casts and tensor layouts only -- none of the method's arithmetic.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    CHUNK,
    Workload,
    make,
    make_prefill_batch,
    regen_rows,
    stratified_rows,
    fp8_encode_rows,
    bits_u16,
    bits_u8,
)
