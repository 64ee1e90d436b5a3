"""Seeded synthetic workloads shared by the oracle tests, GPU tests and bench."""
from .generate import (DTYPES, DecodeInputs, GatherInputs, alibi_slopes_geometric,
                       decode_inputs, gather_inputs, prefill_inputs, raw_bits, raw_u16)
from .catalog import HEADLINE, WORKLOADS, algorithmic_bytes, algorithmic_flops, workload_args

__all__ = [
    "DTYPES", "DecodeInputs", "GatherInputs", "alibi_slopes_geometric", "decode_inputs",
    "gather_inputs", "prefill_inputs", "raw_bits", "raw_u16", "HEADLINE", "WORKLOADS", "algorithmic_bytes",
    "algorithmic_flops", "workload_args",
]
