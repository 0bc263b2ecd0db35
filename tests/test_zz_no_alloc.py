"""The allocation-free layer call (dcu_selective_layer_noalloc, scratch in the library's own device
array) against dcu_selective_layer with a caller workspace: the same kernels, so the same bits, on
two calls in a row, the second with a smaller input (the scratch keeps the first call's contents).
Sizes beyond the array are rejected on the host."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from selective_token_cache_amd import _lib
from tests.util import dev, dev_bf16, host_bf16
from workloads import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setup(shape, B, N, counts, seed, theta):
    g = synth.rng(995, seed)
    w = synth.layer_weights(g, shape, gain_jitter=0.2)
    t = {k: dev_bf16(v) for k, v in w.items()}
    lay = stc.Layer(shape.d, shape.n_heads, shape.head_dim, shape.ffn, shape.eps, t["w_qkv"],
                    t["w_o"], t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"],
                    rope_theta=theta)
    lay._keep = t
    x = synth.normal_bf16(g, (B, N, shape.d))
    kv_std = 0.02 * np.sqrt(shape.d)
    kc = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
    vc = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
    y = synth.normal_bf16(g, (B, N, shape.d))
    sel = np.full((B, N), -1, np.int32)
    for b, c in enumerate(counts):
        sel[b, :c] = np.sort(g.choice(N, size=c, replace=False))
    return lay, x, kc, vc, y, sel, np.asarray(counts, np.int32)


def _run(fn, lay, x, kc, vc, y, sel, cnt, max_rows):
    B = x.shape[0]
    k, v, yy = dev_bf16(kc), dev_bf16(vc), dev_bf16(y)
    done = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    fn(lay, dev_bf16(x), dev(sel), dev(cnt), k, v, yy, max_rows, done)
    torch.cuda.synchronize()
    return host_bf16(k), host_bf16(v), host_bf16(yy), done.cpu().numpy()


def _with_workspace(lay, x, sel, cnt, k, v, y, max_rows, done):
    stc.dcu_selective_layer(lay, x, sel, cnt, k, v, y, max_rows=max_rows, rows_done=done)


def _noalloc(lay, x, sel, cnt, k, v, y, max_rows, done):
    stc.dcu_selective_layer_noalloc(lay, x, sel, cnt, k, v, y, max_rows, rows_done=done)


@pytest.mark.parametrize("shape,calls,theta", [
    # LLaDA-8B layer at batch 1: 64 rows of a 1024-token sequence, then 40 rows of 512 tokens
    (synth.LLADA8B, [(1, 1024, [64], 64), (1, 512, [40], 40)], 5e5),
    # a small layer: three sequences, then two shorter ones with fewer rows
    (synth.LayerShape(d=256, n_heads=4, head_dim=64, ffn=512),
     [(3, 300, [30, 7, 20], 64), (2, 100, [30, 0], 40)], 0.0),
])
def test_noalloc_matches_the_workspace_call(shape, calls, theta):
    for i, (B, N, counts, max_rows) in enumerate(calls):
        _log(f"noalloc d={shape.d} call {i}: B={B} N={N} rows={counts} max_rows={max_rows}")
        args = _setup(shape, B, N, counts, seed=shape.d + i, theta=theta)
        assert args[0].workspace_bytes(B, N, max_rows) <= _lib.NOALLOC_SCRATCH_BYTES
        ref = _run(_with_workspace, *args, max_rows)
        got = _run(_noalloc, *args, max_rows)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        assert got[3].tolist() == list(counts)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    shape = synth.LLADA8B
    lay, x, kc, vc, y, sel, cnt = _setup(shape, 1, 1024, [64], seed=9, theta=0.0)
    assert lay.workspace_bytes(1, 1024, 0) > _lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(stc.DcuError) as e:
        stc.dcu_selective_layer_noalloc(lay, dev_bf16(x), dev(sel), dev(cnt), dev_bf16(kc),
                                        dev_bf16(vc), dev_bf16(y), 0)
    assert e.value.status == _lib.EWORKSPACE
