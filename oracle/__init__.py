"""fp64 CPU oracle of the Interdomain Attention token mixer (test infrastructure).

This package is the checker, not the product.  Only the tests, the smoke
check of the package entry file and the CPU-baseline leg of the benchmark may
import it.  It shares no code with the HIP library: it does not import the
product package and the product never imports it.

Parity status of every function is listed in idattn_oracle's module header;
idattn_backward (gradients by autograd of a literal torch float64 forward)
lists its own pins.
"""
from .idattn_oracle import (decode_step, feature_map, feature_map_rff,
                            feature_map_unit, forward, forward_normalized, forward_varlen, rms_norm,
                            short_conv, silu, ssm_step, zoh)

__all__ = ["decode_step", "feature_map", "feature_map_rff", "feature_map_unit",
           "forward", "forward_normalized", "forward_varlen", "rms_norm", "short_conv", "silu",
           "ssm_step", "zoh"]
