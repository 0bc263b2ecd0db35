"""ctypes binding of libdcu.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks shape / dtype / layout,
passes raw device pointers and the current HIP stream to the C ABI, and raises DcuError on a
non-zero status. No step of the computation happens here. If the library has not been built the
first call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdcu.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class DcuError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


class LayerDesc(ctypes.Structure):
    """Mirror of dcu_layer in include/dcu.h."""
    _fields_ = [("d", _i32), ("n_heads", _i32), ("head_dim", _i32), ("ffn", _i32),
                ("rms_eps", ctypes.c_float), ("w_qkv", _vp), ("w_o", _vp), ("w_gate_up", _vp),
                ("w_down", _vp), ("g_attn", _vp), ("g_ffn", _vp), ("weight_layout", _i32),
                ("rope_theta", ctypes.c_float)]


WEIGHTS_BLOCKED = 1       # DCU_WEIGHTS_BLOCKED
WEIGHTS_BLOCKED_ROPE = 2  # DCU_WEIGHTS_BLOCKED_ROPE


_lib = None

EXPORTS = {
    "dcu_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dcu_version": (ctypes.c_int, []),
    "dcu_budget": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "dcu_distance": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp]),
    "dcu_distance_rows": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _i32,
                                         _vp]),
    "dcu_select": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                  _vp, _vp]),
    "dcu_pack_weights": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "dcu_pack_gate_up": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "dcu_pack_qkv": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "dcu_selective_layer_workspace": (ctypes.c_size_t,
                                      [ctypes.POINTER(LayerDesc), _i32, _i32, _i32]),
    "dcu_selective_layer": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _vp, _vp, _vp, _i32, _i32,
                                           _i32, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp]),
    "dcu_selective_layer_noalloc": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _vp, _vp, _vp, _i32,
                                                   _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "dcu_v_features": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _vp, _i32, _i32, _vp, _vp,
                                      ctypes.c_size_t, _vp]),
    "dcu_attention_context": (ctypes.c_int, [ctypes.POINTER(LayerDesc), _vp, _i32, _i32, _vp, _vp,
                                             _vp, _vp, ctypes.c_size_t, _vp]),
    "dcu_selective_layer_staged": (ctypes.c_int,
                                   [ctypes.POINTER(LayerDesc), _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                    _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp,
                                    ctypes.POINTER(_vp), _i32]),
    "dllm_confidence": (ctypes.c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp]),
    "frechet_commit": (ctypes.c_int, [_vp, _vp, _i32, _i32, ctypes.c_double, _vp, _vp, _vp]),
    "dllm_commit": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, ctypes.c_double, _vp, _vp, _vp,
                                   _vp]),
    "dllm_commit_positions": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "dllm_apd": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i64, _i64, ctypes.c_float, ctypes.c_float,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    # include/dcu_measure.h
    "dcu_measure_stream_read": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "dcu_measure_mfma_loop": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
}


def lib_path() -> str:
    return _PATH


def load():
    """Load libdcu.so (torch is imported first so that one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_PATH):
        raise RuntimeError(f"{_PATH} is not built; run `python -m selective_token_cache_amd.build`")
    L = ctypes.CDLL(_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().dcu_status_string(int(status)).decode()


def version() -> int:
    return load().dcu_version()


# ----------------------------------------------------------------------------- helpers
def _p(t: torch.Tensor | None):
    # ctypes takes the integer address for a c_void_p argument
    return None if t is None else t.data_ptr()


# The current stream's raw handle without building a torch.cuda.Stream object per call (the
# public torch.cuda.current_stream() costs ~3 us of host time, more than a launch): torch's own
# accessors when present, else the public path.
if hasattr(torch._C, "_cuda_getCurrentRawStream") and hasattr(torch._C, "_cuda_getDevice"):
    def _current_raw_stream():
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
else:  # pragma: no cover - older torch
    def _current_raw_stream():
        return torch.cuda.current_stream().cuda_stream


def _stream(stream):
    return _current_raw_stream() if stream is None else stream.cuda_stream


def _new(shape, dtype, device, stream):
    """A tensor the binding allocates (an output the caller did not pass, or a workspace). It comes
    from the caching allocator on the current stream; when the work is enqueued on another stream
    the block is marked as used there, so it is not handed out again before that work is done."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check(fn: str, status: int):
    if status != OK:
        raise DcuError(fn, status)


# ----------------------------------------------------------------------------- entry points
def dcu_budget(s_prev: torch.Tensor | None, B: int, L: int, b_layer: int, out=None, stream=None):
    """s_prev [L, B] fp32 (layer-major previous-step means) or None -> budget [B, L] int32."""
    if s_prev is not None:
        _need(s_prev, "s_prev", torch.float32, (L, B))
        dev = s_prev.device
    else:
        dev = torch.device("cuda", torch.cuda.current_device())
    out = _new((B, L), torch.int32, dev, stream) if out is None else out
    _need(out, "budget", torch.int32, (B, L))
    _check("dcu_budget", load().dcu_budget(_p(s_prev), B, L, b_layer, _p(out), _stream(stream)))
    return out


def dcu_distance(x_cur: torch.Tensor, x_prev: torch.Tensor, dist=None, mean=None, want_mean=True,
                 stream=None):
    """x_cur, x_prev [G, N, d] (bf16 or fp32) -> dist [G, N] fp32, mean [G] fp32 (or None)."""
    _need(x_cur, "x_cur")
    _need(x_prev, "x_prev", x_cur.dtype, x_cur.shape)
    if x_cur.dim() != 3 or x_cur.dtype not in _DT:
        raise ValueError("x_cur must be [G, N, d] bf16 or fp32")
    G, N, d = x_cur.shape
    dist = _new((G, N), torch.float32, x_cur.device, stream) if dist is None else dist
    _need(dist, "dist", torch.float32, (G, N))
    if want_mean and mean is None:
        mean = _new((G,), torch.float32, x_cur.device, stream)
    if mean is not None:
        _need(mean, "mean", torch.float32, (G,))
    st = load().dcu_distance(_p(x_cur), _p(x_prev), _DT[x_cur.dtype], G, N, d, _p(dist), _p(mean),
                             _stream(stream))
    _check("dcu_distance", st)
    return dist, mean


def dcu_distance_rows(x_cur: torch.Tensor, x_prev: torch.Tensor, sel_idx: torch.Tensor,
                      sel_count: torch.Tensor, dist=None, roll: bool = True, stream=None):
    """x_cur, x_prev [G, N, d]; only the listed rows (sel_idx [G, N], sel_count [G]) may differ ->
    dist [G, N] fp32 (0 on the other rows); roll copies the listed rows of x_cur into x_prev."""
    _need(x_cur, "x_cur")
    _need(x_prev, "x_prev", x_cur.dtype, x_cur.shape)
    if x_cur.dim() != 3 or x_cur.dtype not in _DT:
        raise ValueError("x_cur must be [G, N, d] bf16 or fp32")
    G, N, d = x_cur.shape
    _need(sel_idx, "sel_idx", torch.int32, (G, N))
    _need(sel_count, "sel_count", torch.int32, (G,))
    dist = _new((G, N), torch.float32, x_cur.device, stream) if dist is None else dist
    _need(dist, "dist", torch.float32, (G, N))
    st = load().dcu_distance_rows(_p(x_cur), _p(x_prev), _DT[x_cur.dtype], G, N, d, _p(sel_idx),
                                  _p(sel_count), _p(dist), int(bool(roll)), _stream(stream))
    _check("dcu_distance_rows", st)
    return dist


def dcu_select(dist: torch.Tensor, budgets: torch.Tensor, layer: int, key_pos: torch.Tensor | None,
               b_window: int, sel_idx=None, sel_count=None, mean=None, stream=None):
    """dist [B, N] fp32, budgets [B, L] int32, key_pos [B, P] int32 -> (sel_idx [B, N], sel_count [B]).
    mean: optional [B] fp32 out, the layer mean of dist per sequence (as dcu_distance's)."""
    _need(dist, "dist", torch.float32)
    B, N = dist.shape
    _need(budgets, "budgets", torch.int32)
    if budgets.dim() != 2 or budgets.shape[0] != B:
        raise ValueError("budgets must be [B, L]")
    L = budgets.shape[1]
    P = 0
    if key_pos is not None:
        _need(key_pos, "key_pos", torch.int32)
        if key_pos.dim() != 2 or key_pos.shape[0] != B:
            raise ValueError("key_pos must be [B, P]")
        P = key_pos.shape[1]
    sel_idx = _new((B, N), torch.int32, dist.device, stream) if sel_idx is None else sel_idx
    sel_count = _new((B,), torch.int32, dist.device, stream) if sel_count is None else sel_count
    _need(sel_idx, "sel_idx", torch.int32, (B, N))
    _need(sel_count, "sel_count", torch.int32, (B,))
    if mean is not None:
        _need(mean, "mean", torch.float32, (B,))
    st = load().dcu_select(_p(dist), _p(budgets), L, layer, _p(key_pos) if P else None, P, B, N,
                           b_window, _p(sel_idx), _p(sel_count), _p(mean), _stream(stream))
    _check("dcu_select", st)
    return sel_idx, sel_count


def dcu_pack_weights(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The blocked layout of a row-major [rows, cols] bf16 projection matrix (a new tensor of the
    same shape unless `out` is given), written by the library's permutation kernel."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be a 2-D [rows, cols] matrix")
    if out is None:
        out = _new(tuple(w.shape), w.dtype, w.device, stream)
    _need(out, "out", torch.bfloat16, tuple(w.shape))
    _check("dcu_pack_weights",
           load().dcu_pack_weights(_p(w), w.shape[0], w.shape[1], _p(out), _stream(stream)))
    return out


def dcu_pack_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """The fused blocked gate/up matrix [2F, d] of two row-major [F, d] bf16 matrices."""
    _need(w_gate, "w_gate", torch.bfloat16)
    if w_gate.dim() != 2:
        raise ValueError("w_gate must be a 2-D [F, d] matrix")
    _need(w_up, "w_up", torch.bfloat16, tuple(w_gate.shape))
    F, d = w_gate.shape
    if out is None:
        out = _new((2 * F, d), torch.bfloat16, w_gate.device, stream)
    _need(out, "out", torch.bfloat16, (2 * F, d))
    _check("dcu_pack_gate_up", load().dcu_pack_gate_up(_p(w_gate), _p(w_up), F, d, _p(out),
                                                       _stream(stream)))
    return out


def dcu_pack_qkv(w_qkv: torch.Tensor, head_dim: int, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """The blocked [3d, d] W_qkv of a layer with rotary embedding (Q and K rows pair-interleaved
    inside each head, see include/dcu.h)."""
    _need(w_qkv, "w_qkv", torch.bfloat16)
    if w_qkv.dim() != 2 or w_qkv.shape[0] != 3 * w_qkv.shape[1]:
        raise ValueError("w_qkv must be a [3d, d] matrix")
    if out is None:
        out = _new(tuple(w_qkv.shape), w_qkv.dtype, w_qkv.device, stream)
    _need(out, "out", torch.bfloat16, tuple(w_qkv.shape))
    _check("dcu_pack_qkv", load().dcu_pack_qkv(_p(w_qkv), w_qkv.shape[1], head_dim, _p(out),
                                               _stream(stream)))
    return out


class Layer:
    """Holds the device weights of one layer and the matching dcu_layer descriptor. The five
    projection matrices are given row-major ([out, in]) and copied once into the library's blocked
    layout (dcu_pack_weights, or dcu_pack_qkv for W_qkv when rope_theta > 0; gate and up fused by
    dcu_pack_gate_up; on the current stream); the caller's tensors are not kept. rope_theta > 0
    turns on rotary position embedding with that base."""

    def __init__(self, d, n_heads, head_dim, ffn, eps, w_qkv, w_o, w_gate, w_up, w_down, g_attn,
                 g_ffn, rope_theta: float = 0.0):
        for name, t, shape in [("w_qkv", w_qkv, (3 * d, d)), ("w_o", w_o, (d, d)),
                               ("w_gate", w_gate, (ffn, d)), ("w_up", w_up, (ffn, d)),
                               ("w_down", w_down, (d, ffn)), ("g_attn", g_attn, (d,)),
                               ("g_ffn", g_ffn, (d,))]:
            _need(t, name, torch.bfloat16, shape)
        rope = float(rope_theta) > 0
        qkv = dcu_pack_qkv(w_qkv, head_dim) if rope else dcu_pack_weights(w_qkv)
        packed = [qkv, dcu_pack_weights(w_o), dcu_pack_gate_up(w_gate, w_up),
                  dcu_pack_weights(w_down)]
        self.tensors = (*packed, g_attn, g_ffn)
        self.d, self.n_heads, self.head_dim, self.ffn, self.eps = d, n_heads, head_dim, ffn, eps
        self.rope_theta = float(rope_theta)
        self.desc = LayerDesc(d, n_heads, head_dim, ffn, float(eps), *[_p(t) for t in self.tensors],
                              WEIGHTS_BLOCKED_ROPE if rope else WEIGHTS_BLOCKED, self.rope_theta)

    def workspace_bytes(self, B: int, N: int, max_rows: int = 0) -> int:
        return int(load().dcu_selective_layer_workspace(ctypes.byref(self.desc), B, N, max_rows))


LAYER_STAGES = ("gather_rmsnorm", "qkv_scatter", "qkv_fixup", "attention",
                "o_proj_residual", "o_proj_fixup", "rmsnorm", "gate_up_swiglu", "gate_up_fixup",
                "down_residual_scatter", "down_fixup")


def dcu_selective_layer(layer: Layer, x_in: torch.Tensor, sel_idx, sel_count, k_cache, v_cache,
                        y_out, max_rows: int = 0, workspace: torch.Tensor | None = None,
                        stream=None, events=None, rows_done: torch.Tensor | None = None):
    """Recompute the selected rows in place (k_cache, v_cache, y_out are in/out).

    rows_done: optional [B] int32 out, the rows of each sequence actually recomputed (listed
    positions inside [0, N) that fit in max_rows).
    events: optional sequence of len(LAYER_STAGES) + 1 torch.cuda.Event(enable_timing=True) or
    None; event 0 is recorded before the first kernel and event i after stage i, on the library's
    stream (dcu_selective_layer_staged); a None entry skips that mark."""
    _need(x_in, "x_in", torch.bfloat16)
    B, N, d = x_in.shape
    if d != layer.d:
        raise ValueError("x_in width does not match the layer")
    _need(k_cache, "k_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    _need(v_cache, "v_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    _need(y_out, "y_out", torch.bfloat16, (B, N, d))
    if (sel_idx is None) != (sel_count is None):
        raise ValueError("sel_idx and sel_count go together")
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, (B, N))
        _need(sel_count, "sel_count", torch.int32, (B,))
    if rows_done is not None:
        _need(rows_done, "rows_done", torch.int32, (B,))
    need = layer.workspace_bytes(B, N, max_rows)
    if workspace is None:
        workspace = _new((max(need, 1),), torch.uint8, x_in.device, stream)
    _need(workspace, "workspace", torch.uint8)
    if events is None:
        st = load().dcu_selective_layer(ctypes.byref(layer.desc), _p(x_in), _p(sel_idx),
                                        _p(sel_count), B, N, max_rows, _p(k_cache), _p(v_cache),
                                        _p(y_out), _p(workspace), workspace.numel(),
                                        _p(rows_done), _stream(stream))
        _check("dcu_selective_layer", st)
    else:
        if len(events) < len(LAYER_STAGES) + 1:
            raise ValueError(f"need {len(LAYER_STAGES) + 1} events")
        arr = (_vp * len(events))(*[_vp(e.cuda_event if e is not None else None) for e in events])
        st = load().dcu_selective_layer_staged(ctypes.byref(layer.desc), _p(x_in), _p(sel_idx),
                                               _p(sel_count), B, N, max_rows, _p(k_cache),
                                               _p(v_cache), _p(y_out), _p(workspace),
                                               workspace.numel(), _p(rows_done), _stream(stream),
                                               arr, len(events))
        _check("dcu_selective_layer_staged", st)
    return k_cache, v_cache, y_out


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # DCU_NOALLOC_SCRATCH_BYTES


def dcu_selective_layer_noalloc(layer: Layer, x_in: torch.Tensor, sel_idx, sel_count, k_cache,
                                v_cache, y_out, max_rows: int, rows_done: torch.Tensor | None = None,
                                stream=None):
    """dcu_selective_layer with the library's own device scratch (no workspace, nothing allocated):
    for callers that cannot allocate. Calls on one GPU share that scratch and must not overlap."""
    _need(x_in, "x_in", torch.bfloat16)
    B, N, d = x_in.shape
    if d != layer.d:
        raise ValueError("x_in width does not match the layer")
    _need(k_cache, "k_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    _need(v_cache, "v_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    _need(y_out, "y_out", torch.bfloat16, (B, N, d))
    if (sel_idx is None) != (sel_count is None):
        raise ValueError("sel_idx and sel_count go together")
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", torch.int32, (B, N))
        _need(sel_count, "sel_count", torch.int32, (B,))
    if rows_done is not None:
        _need(rows_done, "rows_done", torch.int32, (B,))
    st = load().dcu_selective_layer_noalloc(ctypes.byref(layer.desc), _p(x_in), _p(sel_idx),
                                            _p(sel_count), B, N, max_rows, _p(k_cache),
                                            _p(v_cache), _p(y_out), _p(rows_done),
                                            _stream(stream))
    _check("dcu_selective_layer_noalloc", st)
    return k_cache, v_cache, y_out


def dllm_confidence(logits: torch.Tensor, V: int | None = None, conf=None, token=None, stream=None):
    """logits [R, ld] (bf16 or fp32) -> conf [R] fp32, token [R] int32 over the first V columns."""
    _need(logits, "logits")
    if logits.dim() != 2 or logits.dtype not in _DT:
        raise ValueError("logits must be [R, ld] bf16 or fp32")
    R, ld = logits.shape
    V = ld if V is None else V
    conf = _new((R,), torch.float32, logits.device, stream) if conf is None else conf
    token = _new((R,), torch.int32, logits.device, stream) if token is None else token
    _need(conf, "conf", torch.float32, (R,))
    _need(token, "token", torch.int32, (R,))
    st = load().dllm_confidence(_p(logits), _DT[logits.dtype], R, V, ld, _p(conf), _p(token),
                                _stream(stream))
    _check("dllm_confidence", st)
    return conf, token


def frechet_commit(conf: torch.Tensor, delta: float, m_valid: torch.Tensor | None = None,
                   n_commit=None, order=None, stream=None):
    """conf [B, m] fp32 -> n_commit [B] int32, order [B, m] int32."""
    _need(conf, "conf", torch.float32)
    B, m = conf.shape
    if m_valid is not None:
        _need(m_valid, "m_valid", torch.int32, (B,))
    n_commit = _new((B,), torch.int32, conf.device, stream) if n_commit is None else n_commit
    order = _new((B, m), torch.int32, conf.device, stream) if order is None else order
    _need(n_commit, "n_commit", torch.int32, (B,))
    _need(order, "order", torch.int32, (B, m))
    st = load().frechet_commit(_p(conf), _p(m_valid), B, m, float(delta), _p(n_commit), _p(order),
                               _stream(stream))
    _check("frechet_commit", st)
    return n_commit, order


COMMIT_RULES = {"frechet": 0, "factor": 1, "threshold": 2, "tau": 3}  # DCU_COMMIT_*


def dllm_commit(conf: torch.Tensor, rule: str, param: float = 0.0, m_valid: torch.Tensor | None = None,
                tau: torch.Tensor | None = None, n_commit=None, order=None, stream=None):
    """conf [B, m] fp32 -> n_commit [B] int32, order [B, m] int32 under rule 'frechet' (param =
    delta), 'factor' (param = f), 'threshold' (param = tau) or 'tau' (per-candidate thresholds
    tau [B, m] fp32)."""
    if rule not in COMMIT_RULES:
        raise ValueError(f"rule must be one of {sorted(COMMIT_RULES)}")
    _need(conf, "conf", torch.float32)
    B, m = conf.shape
    if rule == "tau":
        _need(tau, "tau", torch.float32, (B, m))
    else:
        tau = None
    if m_valid is not None:
        _need(m_valid, "m_valid", torch.int32, (B,))
    n_commit = _new((B,), torch.int32, conf.device, stream) if n_commit is None else n_commit
    order = _new((B, m), torch.int32, conf.device, stream) if order is None else order
    _need(n_commit, "n_commit", torch.int32, (B,))
    _need(order, "order", torch.int32, (B, m))
    st = load().dllm_commit(_p(conf), _p(m_valid), B, m, COMMIT_RULES[rule], float(param), _p(tau),
                            _p(n_commit), _p(order), _stream(stream))
    _check("dllm_commit", st)
    return n_commit, order


def dllm_apd(logits: torch.Tensor, logits_prev: torch.Tensor | None, V: int, alpha: float,
             beta: float, tau: torch.Tensor, zmax: torch.Tensor, conf=None, token=None,
             c_conc=None, h_instab=None, stream=None):
    """logits [R, ld] (bf16 or fp32) of this step, logits_prev the previous step's or None; tau and
    zmax [R] fp32 state updated in place -> (conf [R], token [R], c [R] or None, H [R] or None)."""
    _need(logits, "logits")
    if logits.dim() != 2 or logits.dtype not in _DT:
        raise ValueError("logits must be [R, ld] bf16 or fp32")
    R, ld = logits.shape
    if logits_prev is not None:
        _need(logits_prev, "logits_prev", logits.dtype, (R, ld))
    _need(tau, "tau", torch.float32, (R,))
    _need(zmax, "zmax", torch.float32, (R,))
    dev_ = logits.device
    conf = _new((R,), torch.float32, dev_, stream) if conf is None else conf
    token = _new((R,), torch.int32, dev_, stream) if token is None else token
    _need(conf, "conf", torch.float32, (R,))
    _need(token, "token", torch.int32, (R,))
    for name, t in (("c_conc", c_conc), ("h_instab", h_instab)):
        if t is not None:
            _need(t, name, torch.float32, (R,))
    st = load().dllm_apd(_p(logits), _p(logits_prev), _DT[logits.dtype], R, V, ld, float(alpha),
                         float(beta), _p(tau), _p(zmax), _p(conf), _p(token), _p(c_conc),
                         _p(h_instab), _stream(stream))
    _check("dllm_apd", st)
    return conf, token, c_conc, h_instab


def dcu_v_features(layer: Layer, x_in: torch.Tensor, v_out=None, workspace=None, stream=None):
    """Value vectors of every row: x_in [B, N, d] bf16 -> v_out [B, N, d] bf16 (the V-cache row
    layout), RMSNorm(x; g_attn) W_v^T."""
    _need(x_in, "x_in", torch.bfloat16)
    B, N, d = x_in.shape
    if d != layer.d:
        raise ValueError("x_in width does not match the layer")
    v_out = _new(tuple(x_in.shape), x_in.dtype, x_in.device, stream) if v_out is None else v_out
    _need(v_out, "v_out", torch.bfloat16, (B, N, d))
    need = layer.workspace_bytes(B, N, B * N)
    if workspace is None:
        workspace = _new((max(need, 1),), torch.uint8, x_in.device, stream)
    _need(workspace, "workspace", torch.uint8)
    st = load().dcu_v_features(ctypes.byref(layer.desc), _p(x_in), B, N, _p(v_out), _p(workspace),
                               workspace.numel(), _stream(stream))
    _check("dcu_v_features", st)
    return v_out


def dcu_attention_context(layer: Layer, x_in: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, ctx_out=None, workspace=None, stream=None):
    """Attention context of every row: x_in [B, N, d] bf16 and the caches [B, N, H, dh] bf16 (read
    only) -> ctx_out [B, N, d] bf16 = softmax(q K^T / sqrt(dh)) V per head, q = RMSNorm(x) W_q^T
    (rotated with the rotary layout)."""
    _need(x_in, "x_in", torch.bfloat16)
    B, N, d = x_in.shape
    if d != layer.d:
        raise ValueError("x_in width does not match the layer")
    _need(k_cache, "k_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    _need(v_cache, "v_cache", torch.bfloat16, (B, N, layer.n_heads, layer.head_dim))
    ctx_out = _new(tuple(x_in.shape), x_in.dtype, x_in.device, stream) if ctx_out is None else ctx_out
    _need(ctx_out, "ctx_out", torch.bfloat16, (B, N, d))
    need = layer.workspace_bytes(B, N, B * N)
    if workspace is None:
        workspace = _new((max(need, 1),), torch.uint8, x_in.device, stream)
    _need(workspace, "workspace", torch.uint8)
    st = load().dcu_attention_context(ctypes.byref(layer.desc), _p(x_in), B, N, _p(k_cache),
                                      _p(v_cache), _p(ctx_out), _p(workspace), workspace.numel(),
                                      _stream(stream))
    _check("dcu_attention_context", st)
    return ctx_out


def dllm_commit_positions(order: torch.Tensor, n_commit: torch.Tensor, slot_pos: torch.Tensor,
                          P: int, key_pos=None, stream=None) -> torch.Tensor:
    """order [B, m], n_commit [B], slot_pos [B, m] int32 -> key_pos [B, P] int32 (-1 padded)."""
    _need(order, "order", torch.int32)
    B, m = order.shape
    _need(n_commit, "n_commit", torch.int32, (B,))
    _need(slot_pos, "slot_pos", torch.int32, (B, m))
    key_pos = _new((B, P), torch.int32, order.device, stream) if key_pos is None else key_pos
    _need(key_pos, "key_pos", torch.int32, (B, P))
    st = load().dllm_commit_positions(_p(order), _p(n_commit), _p(slot_pos), B, m, P, _p(key_pos),
                                      _stream(stream))
    _check("dllm_commit_positions", st)
    return key_pos


def dcu_measure_stream_read(buf: torch.Tensor, grid: int, sink: torch.Tensor, stream=None):
    """One streaming read of every byte of buf (include/dcu_measure.h)."""
    _need(buf, "buf")
    _need(sink, "sink", torch.int32)
    _check("dcu_measure_stream_read",
           load().dcu_measure_stream_read(_p(buf), buf.numel() * buf.element_size(), int(grid),
                                          _p(sink), _stream(stream)))


def dcu_measure_mfma_loop(grid: int, iters: int, sink: torch.Tensor, stream=None) -> int:
    """grid x 4 waves x iters x 8 bf16 MFMAs of 32 x 32 x 16 (include/dcu_measure.h); returns the
    flop count."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < 256:
        raise ValueError("sink must hold 256 floats")
    _check("dcu_measure_mfma_loop",
           load().dcu_measure_mfma_loop(int(grid), int(iters), _p(sink), _stream(stream)))
    return int(grid) * 4 * int(iters) * 8 * 32 * 32 * 16 * 2
