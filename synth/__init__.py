"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This package holds no attention arithmetic: it draws random numbers, rounds
them to the stored formats (bf16, OCP fp8 E4M3FN with a per-tensor scale, fp32)
and lays out varlen offsets, page pools and block tables. Both the oracle and
the HIP path consume the exact bytes produced here.
"""

from .gen import (  # noqa: F401
    Case,
    FP8_NAN_BYTE,
    dense_case,
    poison_,
    paged_case,
    varlen_case,
    varlen_paged_case,
    workload,
    WORKLOADS,
)
