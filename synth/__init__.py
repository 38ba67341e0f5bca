"""Seeded synthetic inputs for one EAGLE-2 draft round (no arithmetic of the method)."""
from .inputs import (CONFIGS, TreeConfig, make_inputs, bf16_bits, bf16_bits_to_f32,
                     config_by_name)

__all__ = ["CONFIGS", "TreeConfig", "make_inputs", "bf16_bits", "bf16_bits_to_f32",
           "config_by_name"]
