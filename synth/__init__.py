"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package draws random numbers and lays them out in the storage formats the
library reads (float32, bfloat16 bits, OCP E4M3 codes with per-head scales, a
shuffled block table).  It holds none of the attention arithmetic: it neither
imports the oracle nor the HIP binding.
"""
from .workloads import (Workload, make_workload, named_workload, NAMED,
                        to_bf16_bits, quantize_e4m3)

__all__ = ["Workload", "make_workload", "named_workload", "NAMED",
           "to_bf16_bits", "quantize_e4m3"]
