"""Seeded synthetic inputs for the paged-KV decode workloads.

This package only draws random numbers and lays out tables: it holds none of the
attention, merge or address arithmetic, so both the oracle side and the HIP side can
consume its output without sharing any of the method's code.
"""

from .workloads import Case, WORKLOADS, bf16_round_bits, make_case, gqa_case, mla_case

__all__ = ["Case", "WORKLOADS", "bf16_round_bits", "make_case", "gqa_case", "mla_case"]
