"""GPU parity of dcu_selective_layer against the oracle's fp64 layer on the same bf16 inputs.

Bars: rel-L2 <= 1e-2 per tensor (K, V and output rows that were recomputed); rows outside the
selection bitwise untouched; bitwise-deterministic across runs. Caches start from synthetic bf16
contents (the state a previous step left behind), shared by both sides."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from oracle import layer as olayer
from tests.util import dev, dev_bf16, host_bf16, rel_l2, row_rel_l2
from workloads import synth

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _log(msg):
    print(msg, flush=True)


class Case:
    def __init__(self, shape, B, N, seed, std=0.02, theta=0.0):
        g = synth.rng(950, seed)
        self.shape, self.B, self.N, self.theta = shape, B, N, theta
        self.w = synth.layer_weights(g, shape, std=std, gain_jitter=0.2)
        self.x = synth.normal_bf16(g, (B, N, shape.d))
        # a previous step's cache contents, scaled like projections of unit-RMS rows
        kv_std = std * np.sqrt(shape.d)
        self.kc = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
        self.vc = synth.normal_bf16(g, (B, N, shape.n_heads, shape.head_dim), kv_std)
        self.y = synth.normal_bf16(g, (B, N, shape.d))
        self.g = g

    def layer(self):
        s = self.shape
        t = {k: dev_bf16(v) for k, v in self.w.items()}
        self._t = t
        return stc.Layer(s.d, s.n_heads, s.head_dim, s.ffn, s.eps, t["w_qkv"], t["w_o"],
                         t["w_gate"], t["w_up"], t["w_down"], t["g_attn"], t["g_ffn"],
                         rope_theta=self.theta)

    def run_gpu(self, sel, cnt, max_rows=0, reps=1, rows_done=None):
        L = self.layer()
        out = []
        for _ in range(reps):
            kc, vc, y = dev_bf16(self.kc), dev_bf16(self.vc), dev_bf16(self.y)
            rd = torch.full((self.B,), -7, dtype=torch.int32, device="cuda")
            stc.dcu_selective_layer(L, dev_bf16(self.x), None if sel is None else dev(sel),
                                    None if cnt is None else dev(cnt), kc, vc, y,
                                    max_rows=max_rows, rows_done=rd)
            torch.cuda.synchronize()
            out.append((host_bf16(kc), host_bf16(vc), host_bf16(y)))
            if rows_done is not None:
                rows_done.append(rd.cpu().numpy())
        return out

    def run_oracle(self, sel, cnt):
        s = self.shape
        return olayer.selective_layer(self.w, s.n_heads, s.head_dim, s.eps, self.x, sel, cnt,
                                      self.kc, self.vc, self.y, self.theta)


@pytest.mark.parametrize("rows,cols", [(16, 64), (48, 192), (3 * 4096, 4096)])
def test_pack_weights_layout(rows, cols):
    """dcu_pack_weights against the layout its header states, bit for bit: block (g, t) of rows
    16g.. and columns 64t.. at (g * cols/64 + t) * 1024, columns 64t+8c..+7 of row 16g+r at
    (16c + r) * 8 inside it."""
    _log(f"pack {rows} x {cols}")
    g = np.random.default_rng(rows + cols)
    w = g.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    got = host_bf16(stc.dcu_pack_weights(dev_bf16(w)))
    want = w.reshape(rows // 16, 16, cols // 64, 8, 8).transpose(0, 2, 3, 1, 4).reshape(rows, cols)
    assert np.array_equal(got.reshape(rows, cols), want)


@pytest.mark.parametrize("F,d", [(16, 64), (48, 128), (12288, 4096)])
def test_pack_gate_up_layout(F, d):
    """dcu_pack_gate_up against its header: the [2F, d] matrix with alternating 16-row groups of
    gate and up, in the blocked layout (checked through the same block formula as above)."""
    _log(f"pack gate/up {F} x {d}")
    g = np.random.default_rng(F + d)
    wg = g.integers(0, 1 << 16, size=(F, d), dtype=np.uint16)
    wu = g.integers(0, 1 << 16, size=(F, d), dtype=np.uint16)
    got = host_bf16(stc.dcu_pack_gate_up(dev_bf16(wg), dev_bf16(wu)))
    inter = np.stack([wg.reshape(F // 16, 16, d), wu.reshape(F // 16, 16, d)], axis=1).reshape(2 * F, d)
    want = inter.reshape(2 * F // 16, 16, d // 64, 8, 8).transpose(0, 2, 3, 1, 4).reshape(2 * F, d)
    assert np.array_equal(got.reshape(2 * F, d), want)


def _rows(sel, cnt, B, N):
    if sel is None:
        return [np.arange(N) for _ in range(B)]
    return [sel[b, :cnt[b]].astype(np.int64) for b in range(B)]


def _compare(case, got, ref, rows):
    kc, vc, y = got
    rk, rv, ry = ref
    f = synth.bf16_to_f32
    for b, r in enumerate(rows):
        keep = np.setdiff1d(np.arange(case.N), r)
        assert np.array_equal(kc[b, keep], case.kc[b, keep])
        assert np.array_equal(vc[b, keep], case.vc[b, keep])
        assert np.array_equal(y[b, keep], case.y[b, keep])
    allr = [(b, r) for b, r in enumerate(rows) if len(r)]
    if not allr:
        return
    gk = np.concatenate([f(kc[b, r]).reshape(len(r), -1) for b, r in allr])
    gv = np.concatenate([f(vc[b, r]).reshape(len(r), -1) for b, r in allr])
    gy = np.concatenate([f(y[b, r]) for b, r in allr])
    ok = np.concatenate([rk[b, r].reshape(len(r), -1) for b, r in allr])
    ov = np.concatenate([rv[b, r].reshape(len(r), -1) for b, r in allr])
    oy = np.concatenate([ry[b, r] for b, r in allr])
    ek, ev, ey = rel_l2(gk, ok), rel_l2(gv, ov), rel_l2(gy, oy)
    rk_, rv_, ry_ = row_rel_l2(gk, ok).max(), row_rel_l2(gv, ov).max(), row_rel_l2(gy, oy).max()
    _log(f"  rel-L2 K {ek:.2e} V {ev:.2e} Y {ey:.2e}; worst row K {rk_:.2e} V {rv_:.2e} Y {ry_:.2e}")
    assert ek <= TOL and ev <= TOL and ey <= TOL
    # the same bar on every recomputed row, so one bad row cannot hide in the pooled value
    assert rk_ <= TOL and rv_ <= TOL and ry_ <= TOL


def _random_selection(g, B, N, counts):
    sel = np.full((B, N), -1, np.int32)
    for b, c in enumerate(counts):
        sel[b, :c] = np.sort(g.choice(N, size=c, replace=False))
    return sel, np.asarray(counts, np.int32)


@pytest.mark.parametrize("shape,B,N,counts", [
    (synth.TINY, 1, 64, [20]),                                                   # tiny fp32 config shapes
    (synth.TINY, 2, 64, [20, 41]),                                               # one K-tile, 2 sequences
    (synth.LayerShape(d=256, n_heads=4, head_dim=64, ffn=512), 3, 200, [130, 1, 0]),
    (synth.LayerShape(d=512, n_heads=4, head_dim=128, ffn=768), 2, 300, [64, 257]),
    (synth.LayerShape(d=128, n_heads=4, head_dim=32, ffn=192), 4, 77, [77, 5, 33, 64]),
    # K long enough for the split-K path of the output (K = 1024) and down (K = 2048) projections
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 2, 256, [100, 37]),
    # 700 rows: gate/up has 6 x 64 = 384 tiles for 512 workgroups (at most two rounds), so it runs
    # the early-refill loop with the CU-paired tail (128 tiles cut in 2 K-segments, fixup); the
    # output projection's 48 tiles are all split, so the RMSNorm finishes them a workgroup per row
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=4096), 2, 512, [400, 300]),
])
def test_selective_layer_small_shapes(shape, B, N, counts):
    _log(f"layer d={shape.d} H={shape.n_heads} dh={shape.head_dim} F={shape.ffn} B={B} N={N}")
    case = Case(shape, B, N, seed=shape.d + N)
    sel, cnt = _random_selection(case.g, B, N, counts)
    (got, got2) = case.run_gpu(sel, cnt, reps=2)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, B, N))


@pytest.mark.parametrize("shape,B,N,counts,max_rows", [
    # ragged weight tiles (QKV 960, FFN 448, output 320 rows), no split
    (synth.LayerShape(d=320, n_heads=5, head_dim=64, ffn=448), 2, 100, [30, 23], 60),
    # split K on every projection, one row
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 1, 256, [1], 1),
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 3, 90, [17, 40, 7], 64),
])
def test_selective_layer_at_most_64_rows(shape, B, N, counts, max_rows):
    """A tight caller bound max_rows <= 64: workspace and launch grids sized for at most 64 rows,
    every projection in one 64-row tile, split along K where the weight tiles are few."""
    _log(f"layer <=64 rows d={shape.d} F={shape.ffn} B={B} N={N} max_rows={max_rows}")
    case = Case(shape, B, N, seed=shape.d + N + 1)
    sel, cnt = _random_selection(case.g, B, N, counts)
    (got, got2) = case.run_gpu(sel, cnt, max_rows=max_rows, reps=2)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, B, N))


@pytest.mark.parametrize("shape,B,N,counts,max_rows,theta", [
    # rows of 6144 and 8192 values under a row bound of 64: the fused QKV stream (gains of up to
    # 8192 values in LDS) and the workgroup-per-row fixup + RMSNorm with 3 and 4 groups per thread
    (synth.LayerShape(d=6144, n_heads=48, head_dim=128, ffn=256), 2, 40, [17, 30], 64, 5e5),
    (synth.LayerShape(d=8192, n_heads=64, head_dim=128, ffn=256), 1, 48, [33], 48, 0.0),
    # 8256 values: past both limits, so the gather kernel, the split fixup and the plain RMSNorm run
    (synth.LayerShape(d=8256, n_heads=129, head_dim=64, ffn=192), 1, 40, [21], 32, 1e4),
])
def test_wide_rows_at_most_64_rows(shape, B, N, counts, max_rows, theta):
    _log(f"layer wide rows d={shape.d} B={B} N={N} max_rows={max_rows}")
    case = Case(shape, B, N, seed=shape.d + N + 9, theta=theta)
    sel, cnt = _random_selection(case.g, B, N, counts)
    (got, got2) = case.run_gpu(sel, cnt, max_rows=max_rows, reps=2)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, B, N))


def test_dense_mode_small():
    shape = synth.LayerShape(d=256, n_heads=2, head_dim=128, ffn=320)
    case = Case(shape, 2, 150, seed=7)
    (got,) = case.run_gpu(None, None)
    _compare(case, got, case.run_oracle(None, None), _rows(None, None, 2, 150))


def test_empty_selection_and_max_rows_clamp():
    shape = synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=128)
    case = Case(shape, 3, 100, seed=8)
    sel, cnt = _random_selection(case.g, 3, 100, [0, 0, 0])
    done = []
    (got,) = case.run_gpu(sel, cnt, rows_done=done)
    assert np.array_equal(got[0], case.kc) and np.array_equal(got[2], case.y)
    assert done[0].tolist() == [0, 0, 0]
    # counts 40 + 50 + 30 with room for 70 rows: sequence 0 fully, sequence 1 its first 30 rows,
    # which rows_done reports
    sel, cnt = _random_selection(case.g, 3, 100, [40, 50, 30])
    done = []
    (got,) = case.run_gpu(sel, cnt, max_rows=70, rows_done=done)
    cl = np.array([40, 30, 0], np.int32)
    assert done[0].tolist() == cl.tolist()
    _compare(case, got, case.run_oracle(sel, cl), _rows(sel, cl, 3, 100))
    # counts past N are clamped to N (dense rows of that sequence)
    sel = np.tile(np.arange(100, dtype=np.int32), (3, 1))
    done = []
    (got,) = case.run_gpu(sel, np.array([500, 0, 3], np.int32), rows_done=done)
    assert done[0].tolist() == [100, 0, 3]
    _compare(case, got, case.run_oracle(sel, np.array([100, 0, 3], np.int32)),
             _rows(sel, np.array([100, 0, 3], np.int32), 3, 100))


@pytest.mark.parametrize("shape,B,N,theta,max_rows", [
    (synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=128), 3, 100, 0.0, 0),
    (synth.LayerShape(d=256, n_heads=4, head_dim=64, ffn=512), 2, 300, 1e4, 0),
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 2, 90, 5e5, 64),
])
def test_positions_outside_the_sequence_are_skipped(shape, B, N, theta, max_rows):
    """A selection list holding -1, N and other out-of-range entries among its counted positions:
    nothing is read or written for those entries (caches and output untouched there), every valid
    position is recomputed as the oracle recomputes the list without them, and rows_done counts
    the valid positions only."""
    _log(f"layer skipped positions d={shape.d} B={B} N={N} theta={theta}")
    case = Case(shape, B, N, seed=shape.d + N + 77, theta=theta)
    g = case.g
    sel = np.full((B, N), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    valid = []
    for b in range(B):
        k = min(N // 3, 25 if max_rows else N // 3)
        good = np.sort(g.choice(N, size=k, replace=False)).astype(np.int32)
        bad = np.array([-1, N, N + 5, -(2 ** 31), 2 ** 31 - 1][: 2 + b], np.int32)
        lst = np.concatenate([good, bad])
        g.shuffle(lst)
        sel[b, :len(lst)] = lst
        cnt[b] = len(lst)
        valid.append(good)
    done = []
    (got, got2) = case.run_gpu(sel, cnt, max_rows=max_rows, reps=2, rows_done=done)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    assert done[0].tolist() == [len(v) for v in valid]
    vsel = np.full((B, N), -1, np.int32)
    vcnt = np.array([len(v) for v in valid], np.int32)
    for b, v in enumerate(valid):
        vsel[b, :len(v)] = v
    _compare(case, got, case.run_oracle(vsel, vcnt), _rows(vsel, vcnt, B, N))


def test_layer_on_a_side_stream_keeps_its_workspace():
    """The binding's own workspace, allocated on the current stream for work enqueued on another
    stream, is not handed to a later allocation on the current stream while that work runs: a
    call on a side stream followed at once by allocations filled with garbage on the default
    stream gives the same bits as the same call on the default stream."""
    shape = synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048)
    B, N = 2, 512
    case = Case(shape, B, N, seed=91)
    sel, cnt = _random_selection(case.g, B, N, [300, 250])
    (ref,) = case.run_gpu(sel, cnt)
    L = case.layer()
    side = torch.cuda.Stream()
    x, ds, dc = dev_bf16(case.x), dev(sel), dev(cnt)
    n_junk = L.workspace_bytes(B, N) // 4
    for _ in range(3):
        kc, vc, y = dev_bf16(case.kc), dev_bf16(case.vc), dev_bf16(case.y)
        torch.cuda.synchronize()
        stc.dcu_selective_layer(L, x, ds, dc, kc, vc, y, stream=side)
        junk = [torch.full((n_junk,), float("nan"), device="cuda") for _ in range(4)]
        side.synchronize()
        torch.cuda.synchronize()
        assert np.array_equal(host_bf16(kc), ref[0]) and np.array_equal(host_bf16(vc), ref[1])
        assert np.array_equal(host_bf16(y), ref[2])
        del junk


def test_full_size_single_sequence_64_rows():
    """One LLaDA-8B-shaped layer (d=4096, 32 heads x 128, FFN 12288), batch 1, N=1024, 64 rows:
    a 32-wide window around one key in [512, 1024) plus 32 scattered rows."""
    _log("layer full size batch 1")
    case = Case(synth.LLADA8B, 1, 1024, seed=3)
    key = int(case.g.integers(512, 1024))
    lo = max(0, min(key - 16, 1024 - 32))
    win = set(range(lo, lo + 32))
    rest = np.setdiff1d(np.arange(1024), list(win))
    extra = set(case.g.choice(rest, size=32, replace=False).tolist())
    rows = np.array(sorted(win | extra), np.int32)
    sel = np.full((1, 1024), -1, np.int32)
    sel[0, :64] = rows
    cnt = np.array([64], np.int32)
    (got, got2) = case.run_gpu(sel, cnt, reps=2)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    ref = case.run_oracle(sel, cnt)
    _compare(case, got, ref, _rows(sel, cnt, 1, 1024))
    # the same call with the caller's tight bound max_rows = 64 (workspace and grids sized for it)
    (got64,) = case.run_gpu(sel, cnt, max_rows=64)
    _compare(case, got64, ref, _rows(sel, cnt, 1, 1024))


@pytest.mark.parametrize("counts,b,theta", [
    # 1041 rows: 9 row tiles, the output and down projections (288 tiles) run one whole tile per CU
    # plus 32 tiles in 8 K-segments
    ([150, 90, 200, 64, 128, 170, 99, 140], 2, 0.0),
    # 1250 rows (320 tiles: 64 tiles in 4 segments) and 1400 rows (352 tiles: 96 in 2)
    ([160, 170, 150, 180, 155, 140, 165, 130], 5, 0.0),
    ([180, 175, 170, 185, 176, 168, 172, 174], 7, 0.0),
    # rotary embedding with LLaDA's base, positions up to 1023
    ([160, 170, 150, 180, 155, 140, 165, 130], 3, 5e5),
])
def test_full_size_batched_sampled(counts, b, theta):
    """Batch 8, N=1024, LLaDA-8B shapes, ~130-200 rows per sequence; the oracle recomputes one
    sequence completely (its rows depend only on that sequence's cache)."""
    _log(f"layer full size batch 8, {sum(counts)} rows, rope theta {theta}")
    shape = synth.LLADA8B
    case = Case(shape, 8, 1024, seed=4 + b, theta=theta)
    sel, cnt = _random_selection(case.g, 8, 1024, counts)
    (got,) = case.run_gpu(sel, cnt)
    ref = olayer.selective_layer(case.w, shape.n_heads, shape.head_dim, shape.eps,
                                 case.x[b:b + 1], sel[b:b + 1], cnt[b:b + 1], case.kc[b:b + 1],
                                 case.vc[b:b + 1], case.y[b:b + 1], theta)
    sub = Case.__new__(Case)
    sub.kc, sub.vc, sub.y, sub.N = case.kc[b:b + 1], case.vc[b:b + 1], case.y[b:b + 1], 1024
    _compare(sub, tuple(t[b:b + 1] for t in got), ref, _rows(sel[b:b + 1], cnt[b:b + 1], 1, 1024))
    # every other sequence: untouched outside its selection
    for bb in range(8):
        keep = np.setdiff1d(np.arange(1024), sel[bb, :cnt[bb]])
        assert np.array_equal(got[2][bb, keep], case.y[bb, keep])


def test_full_size_batch8_n2048_sampled():
    """Batched layer at N = 2048 (1024 prompt + 1024 generated), batch 8, LLaDA-8B shapes, budget 64
    plus a 32-wide window per sequence (~96 rows each, some ragged); the oracle recomputes one
    sequence whole and every other sequence is checked untouched outside its selection."""
    _log("layer full size batch 8 N 2048")
    shape = synth.LLADA8B
    case = Case(shape, 8, 2048, seed=6)
    counts = [96, 130, 64, 100, 81, 120, 96, 111]
    sel, cnt = _random_selection(case.g, 8, 2048, counts)
    (got,) = case.run_gpu(sel, cnt)
    b = 5
    ref = olayer.selective_layer(case.w, shape.n_heads, shape.head_dim, shape.eps,
                                 case.x[b:b + 1], sel[b:b + 1], cnt[b:b + 1], case.kc[b:b + 1],
                                 case.vc[b:b + 1], case.y[b:b + 1])
    sub = Case.__new__(Case)
    sub.kc, sub.vc, sub.y, sub.N = case.kc[b:b + 1], case.vc[b:b + 1], case.y[b:b + 1], 2048
    _compare(sub, tuple(t[b:b + 1] for t in got), ref, _rows(sel[b:b + 1], cnt[b:b + 1], 1, 2048))
    for bb in range(8):
        keep = np.setdiff1d(np.arange(2048), sel[bb, :cnt[bb]])
        assert np.array_equal(got[2][bb, keep], case.y[bb, keep])
        assert np.array_equal(got[0][bb, keep], case.kc[bb, keep])


@pytest.mark.parametrize("d,dh", [(128, 64), (256, 32), (512, 128), (4096, 128)])
def test_pack_qkv_layout(d, dh):
    """dcu_pack_qkv against its header, bit for bit: the blocked layout (dcu_pack_weights, itself
    checked against its formula above) of W_qkv with each Q and K head's rows reordered in groups
    of 16: dims 0..15, h..h+15, 16..31, h+16..h+31, ... (h = dh/2); the V rows in order."""
    _log(f"pack qkv d={d} dh={dh}")
    g = np.random.default_rng(d + dh)
    w = g.integers(0, 1 << 16, size=(3 * d, d), dtype=np.uint16)
    h = dh // 2
    order = np.concatenate([np.r_[16 * k:16 * k + 16, h + 16 * k:h + 16 * k + 16]
                            for k in range(h // 16)])
    rows = np.concatenate([hd * dh + order for hd in range(2 * d // dh)] + [np.arange(2 * d, 3 * d)])
    got = host_bf16(stc.dcu_pack_qkv(dev_bf16(w), dh))
    want = host_bf16(stc.dcu_pack_weights(dev_bf16(np.ascontiguousarray(w[rows]))))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("shape,B,N,counts,max_rows,theta", [
    (synth.TINY, 2, 64, [20, 41], 0, 1e4),
    (synth.LayerShape(d=128, n_heads=4, head_dim=32, ffn=192), 4, 77, [77, 5, 33, 64], 0, 1e4),
    (synth.LayerShape(d=512, n_heads=4, head_dim=128, ffn=768), 2, 300, [64, 257], 0, 5e5),
    # split K on every projection (fixup epilogue), one and few rows
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 1, 256, [1], 1, 5e5),
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 2, 256, [100, 37], 0, 5e5),
    (synth.LayerShape(d=1024, n_heads=8, head_dim=128, ffn=2048), 3, 90, [17, 40, 7], 64, 5e5),
    # ragged QKV tiles (960 output columns) with 64- and 128-row tiles
    (synth.LayerShape(d=320, n_heads=5, head_dim=64, ffn=448), 2, 100, [30, 23], 60, 1e4),
    (synth.LayerShape(d=320, n_heads=5, head_dim=64, ffn=448), 2, 100, [70, 41], 0, 1e4),
])
def test_selective_layer_rope(shape, B, N, counts, max_rows, theta):
    """Rotary embedding in the QKV epilogue (direct and split-K fixup, 64-row and 128-row tiles):
    keys cached rotated by their row's position; outputs against the oracle's rotated layer."""
    _log(f"layer rope d={shape.d} dh={shape.head_dim} B={B} N={N} theta={theta}")
    case = Case(shape, B, N, seed=shape.d + N + 5, theta=theta)
    sel, cnt = _random_selection(case.g, B, N, counts)
    (got, got2) = case.run_gpu(sel, cnt, max_rows=max_rows, reps=2)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, B, N))


def test_selective_layer_rope_dense():
    """Dense mode (no selection) with rotary embedding: every row rotated by its own position."""
    shape = synth.LayerShape(d=256, n_heads=2, head_dim=128, ffn=320)
    case = Case(shape, 2, 150, seed=17, theta=5e5)
    (got,) = case.run_gpu(None, None)
    _compare(case, got, case.run_oracle(None, None), _rows(None, None, 2, 150))


def test_full_size_rope_single_sequence_n2048():
    """LLaDA-8B shapes with rotary base 500000, batch 1, N = 2048, 64 rows spread over the whole
    sequence (positions up to 2047)."""
    _log("layer rope full size N 2048")
    case = Case(synth.LLADA8B, 1, 2048, seed=19, theta=5e5)
    sel, cnt = _random_selection(case.g, 1, 2048, [64])
    (got,) = case.run_gpu(sel, cnt)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, 1, 2048))


@pytest.mark.parametrize("shape,B,N", [
    (synth.LayerShape(d=256, n_heads=4, head_dim=64, ffn=512), 2, 100),
    (synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=192), 1, 37),
    (synth.LLADA8B, 1, 1024),
])
def test_v_features_and_v_distance(shape, B, N):
    """dcu_v_features (RMSNorm + the W_v rows of the blocked W_qkv, every row) against the oracle,
    then the V-feature distance: dcu_distance on the new Value vectors and the V cache, and the
    selection it drives, on the same GPU inputs as the oracle's."""
    from oracle import distance as odist
    from oracle import select as osel
    _log(f"v features d={shape.d} B={B} N={N}")
    case = Case(shape, B, N, seed=shape.d + N + 5)
    L = case.layer()
    v = stc.dcu_v_features(L, dev_bf16(case.x))
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(host_bf16(v)).reshape(B * N, shape.d)
    ref = olayer.v_features(case.w, shape.eps, case.x).reshape(B * N, shape.d)
    e = rel_l2(got, ref)
    _log(f"  rel-L2 V {e:.2e}")
    assert e <= TOL
    vc = dev_bf16(case.vc).view(B, N, shape.d)
    dist, mean = stc.dcu_distance(v, vc)
    vh = host_bf16(v)
    rd, rm = odist.distance_and_mean(vh, case.vc.reshape(B, N, shape.d))
    assert np.allclose(dist.cpu().numpy(), rd, rtol=1e-5, atol=1e-6)
    budgets = np.full((B, 1), 16, np.int32)
    keys = np.full((B, 1), N // 2, np.int32)
    sel, cnt = stc.dcu_select(dist, dev(budgets), 0, dev(keys), 8)
    rs, rc = osel.select(dist.cpu().numpy(), budgets, 0, keys, 8)
    assert np.array_equal(cnt.cpu().numpy(), rc) and np.array_equal(sel.cpu().numpy(), rs)


def test_v_features_with_the_rotary_layout():
    """The V rows keep their order in dcu_pack_qkv, so the Value vectors of a rotary layer are
    bit-identical to those of the same weights in the plain layout (no rotation on V)."""
    shape = synth.LayerShape(d=256, n_heads=2, head_dim=128, ffn=320)
    case = Case(shape, 2, 70, seed=23)
    plain = case.layer()
    case.theta = 5e5
    rot = case.layer()
    x = dev_bf16(case.x)
    assert torch.equal(stc.dcu_v_features(plain, x).view(torch.int16),
                       stc.dcu_v_features(rot, x).view(torch.int16))


@pytest.mark.parametrize("shape,B,N,theta", [
    (synth.LayerShape(d=128, n_heads=4, head_dim=32, ffn=192), 2, 77, 0.0),
    (synth.LayerShape(d=256, n_heads=4, head_dim=64, ffn=512), 3, 100, 1e4),
    (synth.LayerShape(d=512, n_heads=4, head_dim=128, ffn=768), 1, 300, 5e5),
    (synth.LLADA8B, 1, 1024, 5e5),
])
def test_attention_context(shape, B, N, theta):
    """dcu_attention_context (RMSNorm, W_q, rotary, attention of every row over the caches as
    given) against the oracle; the caches are read only; the attention-context distance between two
    steps' contexts against the oracle's distance of the GPU contexts."""
    from oracle import distance as odist
    _log(f"attention context d={shape.d} dh={shape.head_dim} B={B} N={N} theta={theta}")
    case = Case(shape, B, N, seed=shape.d + N + 31, theta=theta)
    L = case.layer()
    kc, vc = dev_bf16(case.kc), dev_bf16(case.vc)
    ctx = stc.dcu_attention_context(L, dev_bf16(case.x), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(kc), case.kc) and np.array_equal(host_bf16(vc), case.vc)
    got = synth.bf16_to_f32(host_bf16(ctx)).reshape(B * N, shape.d)
    ref = olayer.attention_context(case.w, shape.n_heads, shape.head_dim, shape.eps, case.x,
                                   case.kc, case.vc, theta).reshape(B * N, shape.d)
    e = rel_l2(got, ref)
    _log(f"  rel-L2 ctx {e:.2e}")
    assert e <= TOL
    # a second step: inputs drifted on a third of the rows
    x2 = case.x.copy()
    rows = case.g.choice(B * N, (B * N) // 3, replace=False)
    flat = x2.reshape(B * N, shape.d)
    flat[rows] = synth.normal_bf16(case.g, (len(rows), shape.d))
    ctx2 = stc.dcu_attention_context(L, dev_bf16(x2), kc, vc)
    dist, _ = stc.dcu_distance(ctx2, ctx)
    rd, _ = odist.distance_and_mean(host_bf16(ctx2), host_bf16(ctx))
    assert np.allclose(dist.cpu().numpy(), rd, rtol=1e-5, atol=1e-6)


def test_maximum_sequence_length_with_rotary():
    """N = 65536 (the largest sequence the layer accepts), one sequence, 40 rows spread over it
    (positions up to 65535 for the rotary angles and cache addressing), attention of each over all
    65536 cached rows."""
    shape = synth.LayerShape(d=128, n_heads=2, head_dim=64, ffn=128)
    N = 65536
    _log(f"layer max N {N}")
    case = Case(shape, 1, N, seed=41, theta=1e4)
    sel = np.full((1, N), -1, np.int32)
    rows = np.sort(np.concatenate([case.g.choice(N - 1, 39, replace=False), [N - 1]]))
    sel[0, :40] = rows
    cnt = np.array([40], np.int32)
    (got,) = case.run_gpu(sel, cnt)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, 1, N))


def test_maximum_sequence_count():
    """B = 4096 sequences (the most one call accepts) of N = 8 with ragged counts 0..8: row offsets,
    per-sequence attention tiles and the scatter for every sequence."""
    shape = synth.LayerShape(d=64, n_heads=1, head_dim=64, ffn=64)
    B, N = 4096, 8
    _log(f"layer max B {B}")
    case = Case(shape, B, N, seed=43)
    counts = case.g.integers(0, N + 1, B)
    sel, cnt = _random_selection(case.g, B, N, counts.tolist())
    (got,) = case.run_gpu(sel, cnt)
    _compare(case, got, case.run_oracle(sel, cnt), _rows(sel, cnt, B, N))
