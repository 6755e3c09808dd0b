"""Seeded synthetic inputs for the attention forward and backward passes.

This module only draws and encodes inputs (random normals, lengths, fp8 per-tensor
quantisation, padding and sentinels). It holds none of the attention arithmetic,
so both the HIP path's tests and the CPU oracle can take their inputs from it.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    DenseInputs,
    VarlenInputs,
    config_seed,
    draw_normal,
    make_grad,
    make_grad_on_device,
    make_new_rows,
    make_paged,
    PagedInputs,
    make_dense,
    make_dense_sink,
    make_dense_on_device,
    make_varlen,
    make_config,
    quantize_e4m3,
    to_bits,
)
