"""Seeded synthetic workloads for the VideoMLA latent-KV chunk step.

This module only draws random numbers and describes shapes; it holds none of
the method's arithmetic.  Both the HIP path (through the Python binding) and
the CPU oracle receive exactly the arrays produced here.
"""
from .shapes import MLAShape, SHAPES, shape_by_name, attended_pairs
from .gen import (draw_weights, draw_frames, draw_rope_freq, round_to_bf16_bits,
                  bf16_bits_to_f32, FrameTokens, WEIGHT_NAMES)

__all__ = ["MLAShape", "SHAPES", "shape_by_name", "attended_pairs", "draw_weights", "draw_frames", "draw_rope_freq",
           "FrameTokens",
           "round_to_bf16_bits", "bf16_bits_to_f32", "WEIGHT_NAMES"]
