"""Selective token cache (Dynamic Cache Updating + Frechet-profile commit) for MI355X.

The compute path is libdcu.so (hand-written HIP for gfx950, C ABI in include/dcu.h); this package
is its thin Python binding. See _lib for the entry points.
"""
from ._lib import (BF16, F32, DcuError, Layer, dcu_budget, dcu_distance, dcu_distance_rows,  # noqa: F401
                   dcu_attention_context, dcu_pack_gate_up, dcu_pack_qkv, dcu_pack_weights, dcu_select, dcu_v_features, dllm_apd, dllm_commit, dllm_commit_positions, dcu_selective_layer, dllm_confidence,
                   frechet_commit, lib_path, load, status_string, version)
