"""Seeded synthetic inputs for the CSA2 global-attention hot path.

This package draws random tensors and encodes them into the cache formats the
path consumes (FP8 E4M3 rows with fp32 scales, FP4 E2M1 records with fp32
scales, FP4 E2M1 rows with E4M3 scales per 16, bf16).  It holds no step of the scoring, selection or attention
arithmetic: both the HIP path and the CPU oracle consume the bytes it writes,
and the oracle decodes them with its own tables.
"""
from .formats import (  # noqa: F401
    encode_e4m3_rows, encode_fp4_records, encode_fp4s16_rows, encode_fp4s16_records,
    encode_swa_records, encode_bf16, FP4S16_RECORD_BYTES,
    E4M3_MAX, E2M1_MAX,
    FP4_RECORD_BYTES, SWA_RECORD_BYTES,
)
from .workloads import (  # noqa: F401
    Workload, make_workload, mini_workload, CONFIG_NAMES, EXTRA_WORKLOADS,
    CacheWriteInputs, cache_write_inputs, rope_table, PagedLayout, paged_layout,
)
