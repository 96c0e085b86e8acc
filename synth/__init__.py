"""Seeded synthetic inputs for the LoopVQ encoder and decode-attention path.

This package only draws inputs (keys, values, calibration codebooks, queries,
page tables, ragged lengths).  It holds none of the method's arithmetic, and it
is shared by the oracle side and the GPU side of every test and by the bench.
"""
from .workloads import (  # noqa: F401
    CONFIGS, Config, config_by_name, round_to_bf16, round_to_f16,
    loop_correlated, channel_scales, make_kv, make_codebooks, make_queries,
    make_seq_lens, make_block_table, slot_mapping_for, random_index_cache, make_kv_torch,
    make_window, window_positions, fill_window_pages, make_codebooks_per_group,
    make_tasq, make_sigma, codebooks_from_vectors,
)
