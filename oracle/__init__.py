"""CPU oracle of the SemKV hot path -- test infrastructure only.

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg;
never by the product path.
"""
from .semkv_oracle import *  # noqa: F401,F403
from .semkv_oracle import (GenerationCache, Pools, attention, decode_attention,  # noqa: F401
                           dequantize_pool, dequantize_rows, format_bits, fp16_bits,
                           group_params, nominal_bits, pack_rows, quantize_pack_cache,
                           quantize_rows, rank_order, rank_topr, rank_topr_batch,
                           row_bytes, scale_fp16_ceil, topr_count, unpack_rows,
                           hadamard128, rotate_rows_f32, fp16_floor, quantize_rows_rotated,
                           score_keynorm, RaggedGeneration, score_hidden_delta)
