"""CPU fp64 oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check in __graft_entry__ and the
benchmark's cpu_baseline leg may import it.  The HIP library never does, and
this package imports nothing from the library (numpy only).
"""
from .attention import attention_ref, attention_ref_bhnd, merge_ref
from .backward import attention_bwd_ref
from .fp8 import attention_fp8_ref, e4m3_value, e8m0_value, mx_dequantize
from .tiled import tiled_ref

__all__ = ["attention_ref", "attention_ref_bhnd", "attention_bwd_ref", "merge_ref", "tiled_ref",
           "attention_fp8_ref", "e4m3_value", "e8m0_value", "mx_dequantize"]
