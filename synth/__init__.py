"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This package only draws and stores inputs: it holds the workload table, the
seeded generator and the storage-format encoders (fp32 -> bf16 bits, fp32 ->
OCP e4m3 codes with a per-token scale).  It computes nothing of the attention
itself, and both the CPU oracle tests and the GPU path take their inputs from
here.
"""
from .workloads import (WORKLOADS, Workload, workload, make_inputs, chunk_count_hint,  # noqa: F401
                        make_projection_inputs, PROJ_D_NOPE, PROJ_D_V)
from .formats import (f32_to_bf16_bits, bf16_bits_to_f32, f32_to_e4m3_codes,  # noqa: F401
                      quantize_rows_e4m3, BF16_NAN_BITS, E4M3_NAN_CODE)
