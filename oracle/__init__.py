"""fp64 CPU oracle for Multi-Segment Attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of bench.py, never by the product library or its binding.
"""
from .msa_oracle import (SEG_FIELDS, plan_ref, to_f64, alive_tokens_ref, attention_ref,
                         decode_ref, prefill_ref, partial_ref, merge_ref)

__all__ = ["SEG_FIELDS", "plan_ref", "to_f64", "alive_tokens_ref", "attention_ref",
           "decode_ref", "prefill_ref", "partial_ref", "merge_ref"]
