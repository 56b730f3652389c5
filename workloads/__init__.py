"""Seeded synthetic inputs for the Interdomain Attention token mixer.

This package only draws random numbers and rounds them to the storage dtype.
It holds none of the mixer's arithmetic, so the fp64 oracle and the HIP path
can both consume it without sharing any part of the method.
"""
from .configs import (CONFIGS, Case, bf16_bits, bf16_from_bits, bf16_round,
                      make_case, make_decode_state, make_decode_token,
                      make_params, make_rff_omega, make_rows, spec)

__all__ = ["CONFIGS", "Case", "bf16_bits", "bf16_from_bits", "bf16_round",
           "make_case", "make_decode_state", "make_decode_token",
           "make_params", "make_rff_omega", "make_rows", "spec"]
