"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This package holds parameter-group shapes and seeded value generators only. It
contains none of the method's arithmetic (no layout, no summation, no
placement): both sides draw their inputs from here and compute independently.
"""
from .configs import CONFIGS, config_shapes, Config  # noqa: F401
from .values import (  # noqa: F401
    fp32_to_bf16_bits,
    host_grads,
    host_special_grads,
    host_rank_major_bits,
    device_grads,
    device_rank_major_bits,
)
