"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package only draws random tensors with fixed seeds and lays them out;
it performs none of the sparse-attention arithmetic.
"""
from .inputs import (  # noqa: F401
    HeadShape,
    MODEL_SHAPE,
    TINY_SHAPE,
    gen_prefill,
    gen_decode_paged,
    gen_planted_prefill,
    gen_long_context,
    bf16_round,
)
