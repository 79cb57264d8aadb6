"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package builds inputs only: request lengths, shuffled page pools, page tables and
random bf16 / FP8 tensors, plus poison values in every slot no query may see.  It holds
none of the attention arithmetic, and neither the oracle nor the HIP library is imported
here.
"""

from .workloads import (
    DecodeCase,
    PrefillCase,
    WORKLOADS,
    make_decode_case,
    make_prefill_case,
    decode_workload,
    prefill_workload,
    extract_requests,
)

__all__ = [
    "DecodeCase",
    "PrefillCase",
    "WORKLOADS",
    "make_decode_case",
    "make_prefill_case",
    "decode_workload",
    "prefill_workload",
    "extract_requests",
]
