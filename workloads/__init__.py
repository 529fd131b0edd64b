"""Seeded synthetic inputs for the hybrid-mask attention path.

This package is shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, bench, smoke). It holds only input construction: configuration tables,
seeded random draws, rounding of draws to the storage format, segment tables and
per-token position ids. It contains none of the method's arithmetic (no mask,
no normalisation, no rotary embedding, no attention).
"""
from .configs import (SEG_CAUSAL, SEG_FULL, SEG_GCA, SEG_GEN, Segment, Workload, CONFIGS,
                      get_config, page_shape_configs)
from .generate import (Inputs, generate, positions_for, segment_table, f32_to_bf16_bits,
                       bf16_bits_to_f32, ProjectionInputs, generate_projection)

__all__ = ["SEG_CAUSAL", "SEG_FULL", "SEG_GCA", "SEG_GEN", "Segment", "Workload", "CONFIGS",
           "get_config", "page_shape_configs", "Inputs", "generate", "positions_for",
           "segment_table", "f32_to_bf16_bits", "bf16_bits_to_f32", "ProjectionInputs",
           "generate_projection"]
