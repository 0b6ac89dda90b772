"""Seeded synthetic inputs for sparse MLA decode.

This package only *makes inputs*: query vectors, quantised latent KV rows laid
out in the cache byte format, top-k index lists and sequence lengths.  It holds
none of the decode arithmetic (no dequantisation, no attention, no softmax), so
both the CPU oracle and the HIP library can be fed from it without sharing any
of the method's code.
"""

from .generate import (  # noqa: F401
    CONFIGS,
    LATENT,
    NOPE,
    ROPE,
    ROW_BYTES,
    ROW_BYTES_OF_FORMAT,
    ROW_FMT_FP32,
    ROW_FMT_UE8M0,
    PagedLayout,
    Workload,
    bf16_bits_from_f32,
    build_host_cache,
    build_host_pool,
    config_workload,
    encode_e4m3fn,
    make_paged_layout,
    make_workload,
    physical_rows,
    quantise_rows,
    ue8m0_exponents,
)
