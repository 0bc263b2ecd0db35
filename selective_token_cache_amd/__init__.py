"""Selective token cache (Dynamic Cache Updating + Frechet-profile commit) for MI355X.

The compute path is libdcu.so (hand-written HIP for gfx950, C ABI in include/dcu.h); this package
is its thin Python binding (shape and dtype checks, device pointers, the current stream). Every
call only enqueues kernels, so a whole step can be captured in a HIP graph.

One denoising step over L layers of a batch of B sequences of N tokens (bf16 tensors on the GPU):

    layers = [Layer(d, H, dh, F, eps, w_qkv, w_o, w_gate, w_up, w_down, g_attn, g_ffn,
                    rope_theta=5e5) for ...]          # weights packed once into the blocked layout
    budgets = dcu_budget(s_prev, B, L, b_layer)       # [B, L] from the previous step's means
    for l in range(L):
        dist, _ = dcu_distance(x_cur[l], x_prev[l], want_mean=False)
        sel, cnt = dcu_select(dist, budgets, l, key_pos, b_window, mean=s_cur[l])
        dcu_selective_layer(layers[l], x_cur[l], sel, cnt, k_cache[l], v_cache[l], y[l],
                            workspace=ws)             # recomputes only the selected rows
        x_prev[l], x_cur[l] = x_cur[l], x_prev[l]     # the cache roll is a swap
    conf, tok = dllm_confidence(logits, V)            # end of step
    n_commit, order = frechet_commit(conf.view(B, m), delta)

Closed loop: feed y[l] to layer l+1 and use dcu_distance_rows for the layers after the first;
dllm_commit_positions turns the commits into the next step's key positions. Other pieces:
dllm_commit (factor / threshold / per-position threshold rules), dllm_apd (adaptive parallel
decoding), dcu_v_features and dcu_attention_context (other distance features).
dcu_selective_layer_noalloc is the layer call for callers that cannot allocate (its scratch is a
device array of the library, shared by all calls on a GPU).
"""
from ._lib import (BF16, F32, DcuError, Layer, dcu_attention_context, dcu_budget,  # noqa: F401
                   dcu_distance, dcu_distance_rows, dcu_pack_gate_up, dcu_pack_qkv,
                   dcu_pack_weights, dcu_select, dcu_selective_layer,
                   dcu_selective_layer_noalloc, dcu_v_features, dllm_apd,
                   dllm_commit, dllm_commit_positions, dllm_confidence, frechet_commit, lib_path,
                   load, status_string, version)
from ._lib import dcu_measure_mfma_loop, dcu_measure_stream_read  # noqa: F401
