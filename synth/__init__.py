"""Seeded synthetic inputs and workload shapes (no attention arithmetic here)."""
from .workloads import WORKLOADS, Prefill, PagedDecode, MLADecode, ChunkedPrefill, DSADecode, LocalGlobalPrefill  # noqa: F401
from .generate import (  # noqa: F401
    f32_to_bf16_bits, normal, prefill_inputs, sampled_rows, paged_decode_inputs, mla_inputs,
    chunked_prefill_inputs, dsa_inputs, f32_to_e4m3_bits, f32_to_int8_bits, kv_scales,
)
