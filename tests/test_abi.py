"""The C ABI library loads, exports every function include/dcu.h declares, and rejects invalid
arguments on the host before any launch (these calls never reach a GPU)."""
import ctypes
import os
import re

import pytest

import selective_token_cache_amd as stc
from selective_token_cache_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.lib_path()),
                                reason="libdcu.so not built (run the build first)")


def _declared():
    txt = "\n".join(open(h).read() for h in HEADERS)
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)) -
                  {"if", "sizeof", "defined", "extern"})


def test_every_declared_function_is_exported():
    names = _declared()
    assert {"dcu_distance", "dcu_budget", "dcu_select", "dcu_selective_layer", "dllm_confidence",
            "frechet_commit"} <= set(names)
    L = ctypes.CDLL(_lib.lib_path())
    for n in names:
        assert hasattr(L, n), n
    assert set(_lib.EXPORTS) == set(names)


def test_status_strings_and_version():
    assert stc.status_string(0) == "ok"
    assert "invalid" in stc.status_string(1)
    assert stc.status_string(99) == "unknown status"
    assert stc.version() >= 100


FAKE = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first


def test_budget_validation():
    L = stc.load()
    assert L.dcu_budget(None, 2, 4, 8, None, None) == _lib.EINVAL           # budget NULL
    assert L.dcu_budget(None, 0, 4, 8, FAKE, None) == _lib.EINVAL           # B <= 0
    assert L.dcu_budget(None, 2, 0, 8, FAKE, None) == _lib.EINVAL           # L <= 0
    assert L.dcu_budget(None, 2, 4, -1, FAKE, None) == _lib.EINVAL          # b_layer < 0
    assert L.dcu_budget(None, 2, 4, 2**30, FAKE, None) == _lib.EINVAL       # T overflows
    assert L.dcu_budget(None, 2, 2000, 1, FAKE, None) == _lib.EUNSUPPORTED  # L > 1024


def test_distance_validation():
    L = stc.load()
    assert L.dcu_distance(None, FAKE, 1, 1, 1, 8, FAKE, None, None) == _lib.EINVAL
    assert L.dcu_distance(FAKE, FAKE, 1, 0, 1, 8, FAKE, None, None) == _lib.EINVAL
    assert L.dcu_distance(FAKE, FAKE, 7, 1, 1, 8, FAKE, None, None) == _lib.EINVAL
    assert L.dcu_distance(FAKE, FAKE, 1, 1, 1, 12, FAKE, None, None) == _lib.EUNSUPPORTED
    assert L.dcu_distance(FAKE, FAKE, 0, 1, 1, 6, FAKE, None, None) == _lib.EUNSUPPORTED
    odd = ctypes.c_void_p(256 + 4)
    assert L.dcu_distance(odd, FAKE, 1, 1, 1, 8, FAKE, None, None) == _lib.EUNSUPPORTED


def test_distance_rows_validation():
    L = stc.load()
    assert L.dcu_distance_rows(None, FAKE, 1, 1, 4, 8, FAKE, FAKE, FAKE, 1, None) == _lib.EINVAL
    assert L.dcu_distance_rows(FAKE, FAKE, 1, 1, 4, 8, None, FAKE, FAKE, 1, None) == _lib.EINVAL
    assert L.dcu_distance_rows(FAKE, FAKE, 7, 1, 4, 8, FAKE, FAKE, FAKE, 1, None) == _lib.EINVAL
    assert L.dcu_distance_rows(FAKE, FAKE, 1, 0, 4, 8, FAKE, FAKE, FAKE, 1, None) == _lib.EINVAL
    assert L.dcu_distance_rows(FAKE, FAKE, 1, 1, 4, 12, FAKE, FAKE, FAKE, 1, None) == _lib.EUNSUPPORTED
    assert L.dcu_distance_rows(FAKE, FAKE, 1, 70000, 4, 8, FAKE, FAKE, FAKE, 1, None) == _lib.EUNSUPPORTED


def test_select_validation():
    L = stc.load()
    args = dict(dist=FAKE, budgets=FAKE, L=4, layer=0, key_pos=FAKE, P=1, B=2, N=64, bw=8,
                sel=FAKE, cnt=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return L.dcu_select(a["dist"], a["budgets"], a["L"], a["layer"], a["key_pos"], a["P"],
                            a["B"], a["N"], a["bw"], a["sel"], a["cnt"], None, None)

    assert call(layer=4) == _lib.EINVAL
    assert call(layer=-1) == _lib.EINVAL
    assert call(bw=-1) == _lib.EINVAL
    assert call(P=-1) == _lib.EINVAL
    assert call(key_pos=None) == _lib.EINVAL
    assert call(sel=None) == _lib.EINVAL
    assert call(N=0) == _lib.EINVAL
    assert call(N=8193) == _lib.EUNSUPPORTED


def test_confidence_and_commit_validation():
    L = stc.load()
    assert L.dllm_confidence(FAKE, 1, 4, 10, 8, FAKE, FAKE, None) == _lib.EINVAL      # ld < V
    assert L.dllm_confidence(FAKE, 1, 0, 8, 8, FAKE, FAKE, None) == _lib.EINVAL
    assert L.dllm_confidence(FAKE, 3, 4, 8, 8, FAKE, FAKE, None) == _lib.EINVAL
    assert L.dllm_confidence(FAKE, 1, 4, 10, 12, FAKE, FAKE, None) == _lib.EUNSUPPORTED
    assert L.frechet_commit(FAKE, None, 2, 16, -0.1, FAKE, FAKE, None) == _lib.EINVAL
    assert L.frechet_commit(FAKE, None, 2, 16, float("nan"), FAKE, FAKE, None) == _lib.EINVAL
    assert L.frechet_commit(FAKE, None, 0, 16, 0.1, FAKE, FAKE, None) == _lib.EINVAL
    assert L.frechet_commit(FAKE, None, 2, 8193, 0.1, FAKE, FAKE, None) == _lib.EUNSUPPORTED
    assert L.dllm_commit(FAKE, None, 2, 16, 4, 0.5, None, FAKE, FAKE, None) == _lib.EINVAL  # rule
    assert L.dllm_commit(FAKE, None, 2, 16, 1, float("inf"), None, FAKE, FAKE, None) == _lib.EINVAL
    assert L.dllm_commit(FAKE, None, 2, 16, 2, float("nan"), None, FAKE, FAKE, None) == _lib.EINVAL
    assert L.dllm_commit(FAKE, None, 2, 16, 0, -0.1, None, FAKE, FAKE, None) == _lib.EINVAL  # delta
    assert L.dllm_commit(FAKE, None, 2, 16, 3, 0.0, None, FAKE, FAKE, None) == _lib.EINVAL   # no tau
    assert L.dllm_commit(FAKE, None, 2, 8193, 1, 0.9, None, FAKE, FAKE, None) == _lib.EUNSUPPORTED
    assert L.dllm_commit(None, None, 2, 16, 1, 0.9, None, FAKE, FAKE, None) == _lib.EINVAL


def test_apd_validation():
    L = stc.load()

    def call(logits=FAKE, R=4, V=10, ld=16, alpha=0.1, beta=0.1, tau=FAKE, dtype=1):
        return L.dllm_apd(logits, None, dtype, R, V, ld, alpha, beta, tau, FAKE, FAKE, FAKE, None,
                          None, None)

    assert call(logits=None) == _lib.EINVAL
    assert call(tau=None) == _lib.EINVAL
    assert call(R=0) == _lib.EINVAL
    assert call(ld=8) == _lib.EINVAL                 # ld < V
    assert call(alpha=-0.1) == _lib.EINVAL
    assert call(beta=float("nan")) == _lib.EINVAL
    assert call(dtype=5) == _lib.EINVAL
    assert call(ld=12) == _lib.EUNSUPPORTED           # bf16 rows not a whole number of 16-B chunks
    odd = ctypes.c_void_p(256 + 4)
    assert call(logits=odd) == _lib.EUNSUPPORTED


def test_pack_weights_validation():
    L = stc.load()
    assert L.dcu_pack_weights(None, 16, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_weights(FAKE, 16, 64, None, None) == _lib.EINVAL
    assert L.dcu_pack_weights(FAKE, 0, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_weights(FAKE, 24, 64, FAKE, None) == _lib.EUNSUPPORTED   # rows % 16
    assert L.dcu_pack_weights(FAKE, 16, 96, FAKE, None) == _lib.EUNSUPPORTED   # cols % 64
    odd = ctypes.c_void_p(256 + 8)
    assert L.dcu_pack_weights(odd, 16, 64, FAKE, None) == _lib.EUNSUPPORTED


def test_pack_gate_up_validation():
    L = stc.load()
    assert L.dcu_pack_gate_up(FAKE, None, 16, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_gate_up(FAKE, FAKE, 0, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_gate_up(FAKE, FAKE, 8, 64, FAKE, None) == _lib.EUNSUPPORTED    # F % 16
    assert L.dcu_pack_gate_up(FAKE, FAKE, 16, 32, FAKE, None) == _lib.EUNSUPPORTED   # d % 64


def test_pack_qkv_validation():
    L = stc.load()
    assert L.dcu_pack_qkv(None, 256, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_qkv(FAKE, 256, 64, None, None) == _lib.EINVAL
    assert L.dcu_pack_qkv(FAKE, 0, 64, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_qkv(FAKE, 256, 0, FAKE, None) == _lib.EINVAL
    assert L.dcu_pack_qkv(FAKE, 320, 128, FAKE, None) == _lib.EINVAL          # d % head_dim
    assert L.dcu_pack_qkv(FAKE, 192, 96, FAKE, None) == _lib.EUNSUPPORTED     # head_dim 96
    assert L.dcu_pack_qkv(FAKE, 96, 32, FAKE, None) == _lib.EUNSUPPORTED      # d % 64
    odd = ctypes.c_void_p(256 + 8)
    assert L.dcu_pack_qkv(FAKE, 256, 64, odd, None) == _lib.EUNSUPPORTED


def _desc(**kw):
    a = dict(d=256, n_heads=4, head_dim=64, ffn=512, eps=1e-5, layout=_lib.WEIGHTS_BLOCKED,
             theta=0.0)
    a.update(kw)
    return _lib.LayerDesc(a["d"], a["n_heads"], a["head_dim"], a["ffn"], a["eps"],
                          *([FAKE] * 6), a["layout"], a["theta"])


def test_layer_validation():
    L = stc.load()
    ws = L.dcu_selective_layer_workspace

    def call(desc, B=2, N=64, sel=None, cnt=None):
        return L.dcu_selective_layer(ctypes.byref(desc), FAKE, sel, cnt, B, N, 0, FAKE, FAKE, FAKE,
                                     FAKE, 1 << 40, None, None)

    assert ws(ctypes.byref(_desc()), 2, 64, 0) > 0
    assert ws(ctypes.byref(_desc(layout=0)), 2, 64, 0) == 0
    assert call(_desc(layout=0)) == _lib.EUNSUPPORTED              # row-major weights claimed
    assert call(_desc(d=250)) == _lib.EINVAL                       # d != n_heads * head_dim
    assert call(_desc(d=192, n_heads=2, head_dim=96)) == _lib.EUNSUPPORTED   # head_dim 96
    assert call(_desc(ffn=500)) == _lib.EUNSUPPORTED              # ffn % 64
    assert call(_desc(eps=-1.0)) == _lib.EINVAL
    assert call(_desc(layout=3)) == _lib.EUNSUPPORTED
    assert call(_desc(theta=1e4)) == _lib.EINVAL                   # rotary base without its layout
    rope = _lib.WEIGHTS_BLOCKED_ROPE
    assert ws(ctypes.byref(_desc(layout=rope, theta=5e5)), 2, 64, 0) > 0
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert call(_desc(layout=rope, theta=bad)) == _lib.EINVAL
    assert call(_desc(), B=0) == _lib.EINVAL
    assert call(_desc(), N=70000) == _lib.EUNSUPPORTED
    assert call(_desc(), sel=FAKE) == _lib.EINVAL                  # only one of sel_idx / sel_count
    # workspace smaller than the query says
    assert L.dcu_selective_layer(ctypes.byref(_desc()), FAKE, None, None, 2, 64, 0, FAKE, FAKE, FAKE,
                                 FAKE, 16, None, None) == _lib.EWORKSPACE


def test_attention_context_validation():
    L = stc.load()

    def call(desc=None, x=FAKE, k=FAKE, v=FAKE, out=FAKE, B=2, N=64, wsb=1 << 40):
        return L.dcu_attention_context(ctypes.byref(desc or _desc()), x, B, N, k, v, out, FAKE, wsb,
                                       None)

    assert call(x=None) == _lib.EINVAL
    assert call(k=None) == _lib.EINVAL
    assert call(out=None) == _lib.EINVAL
    assert call(B=0) == _lib.EINVAL
    assert call(desc=_desc(layout=0)) == _lib.EUNSUPPORTED
    assert call(v=ctypes.c_void_p(256 + 8)) == _lib.EUNSUPPORTED
    assert call(wsb=16) == _lib.EWORKSPACE


def test_commit_positions_validation():
    L = stc.load()
    assert L.dllm_commit_positions(None, FAKE, FAKE, 2, 16, 4, FAKE, None) == _lib.EINVAL
    assert L.dllm_commit_positions(FAKE, FAKE, FAKE, 2, 16, 0, FAKE, None) == _lib.EINVAL
    assert L.dllm_commit_positions(FAKE, FAKE, None, 2, 16, 4, FAKE, None) == _lib.EINVAL


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more exits with a message before touching a GPU."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_m0_check_of_the_dma_kernels():
    """The build's scan of the DMA kernels' assembly: the built listing passes, and a compiler-style
    use of M0 (a write not followed by the DMA, an implicit reader) inserted into it is caught."""
    from selective_token_cache_amd import build as b
    path = os.path.join(ROOT, "_build", "layer.hip.gfx950.s")
    if not os.path.exists(path):
        pytest.skip("assembly listing not built")
    asm = open(path).read()
    assert b.check_m0(asm) == []
    i = asm.index("k_attnILi128E")
    j = asm.index("s_endpgm", i)
    bad = asm[:j] + "s_mov_b32 m0, -1\n\tv_movrels_b32 v1, v2\n\t" + asm[j:]
    problems = b.check_m0(bad)
    assert any("M0 used by the compiler" in p for p in problems)
    assert any("reading M0" in p for p in problems)


def test_stage_wait_check_of_the_dma_kernels():
    """The build's scan for full memory waits inside the staged DMA loops: the built listing has
    none, and one inserted after a stage barrier of the QKV projection is caught."""
    from selective_token_cache_amd import build as b
    path = os.path.join(ROOT, "_build", "layer.hip.gfx950.s")
    if not os.path.exists(path):
        pytest.skip("assembly listing not built")
    asm = open(path).read()
    assert b.check_stage_waits(asm) == []
    i = asm.index("k_gemmILi5E")
    j = asm.index("s_barrier", i) + len("s_barrier")
    bad = asm[:j] + "\n\ts_waitcnt vmcnt(0)" + asm[j:]
    problems = b.check_stage_waits(bad)
    assert len(problems) == 1 and "k_gemmILi5E" in problems[0]
