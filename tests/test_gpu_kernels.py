"""GPU parity of the distance, budget, select, confidence and commit kernels against the oracle.

Bars: distance, mean and confidence within 1e-5 relative (exact 0 where the oracle gives 0);
budgets, selections, tokens, commit counts and sort orders bit-exact given the same inputs;
every kernel bitwise deterministic across two runs."""
import numpy as np
import pytest
import torch

import selective_token_cache_amd as stc
from oracle import budget as obud
from oracle import confidence as oconf
from oracle import distance as odist
from oracle import frechet as ofre
from oracle import select as osel
from tests.util import assert_rel, dev, dev_bf16
from workloads import synth

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------- distance
@pytest.mark.parametrize("G,N,d,frac,sigma", [(3, 37, 8, 0.5, 0.1), (2, 100, 72, 0.3, 0.01),
                                              (1, 1, 4096, 1.0, 0.01), (5, 64, 640, 0.25, 0.2),
                                              (1, 5, 16384, 1.0, 0.01), (2, 3, 8200, 0.7, 0.05)])
def test_distance_bf16_small(G, N, d, frac, sigma):
    _log(f"distance bf16 G={G} N={N} d={d}")
    g = synth.rng(900, G, N, d)
    cur = np.empty((G, N, d), np.uint16)
    prev = np.empty_like(cur)
    for k in range(G):
        cur[k], prev[k], _ = synth.drift_pair(g, N, d, int(round(frac * N)), sigma)
    dist, mean = stc.dcu_distance(dev_bf16(cur), dev_bf16(prev))
    rd, rm = odist.distance_and_mean(cur, prev)
    assert_rel(dist.cpu().numpy(), rd)
    assert_rel(mean.cpu().numpy(), rm)


def test_distance_full_size_32_layers():
    """32 layers x N=1024 x d=4096 bf16, 30% of rows drifted by sigma_l = 0.01 (1 + l/8)."""
    _log("distance full size")
    L, N, d = 32, 1024, 4096
    cur = np.empty((L, N, d), np.uint16)
    prev = np.empty_like(cur)
    for l in range(L):
        cur[l], prev[l], _ = synth.drift_pair(synth.rng(2, 0, l), N, d, 307, 0.01 * (1 + l / 8))
    dc, dp = dev_bf16(cur), dev_bf16(prev)
    dist, mean = stc.dcu_distance(dc, dp)
    dist2, mean2 = stc.dcu_distance(dc, dp)
    rd, rm = odist.distance_and_mean(cur, prev)
    got = dist.cpu().numpy()
    assert_rel(got, rd)
    assert_rel(mean.cpu().numpy(), rm)
    assert np.array_equal(got, dist2.cpu().numpy())
    assert np.array_equal(mean.cpu().numpy(), mean2.cpu().numpy())
    assert np.sum(got > 0) > 0.25 * L * N


def test_distance_fp32_and_edge_rows():
    _log("distance fp32 edges")
    g = synth.rng(901, 0)
    d = 64
    a = g.standard_normal((1, 10, d)).astype(np.float32)
    b = a.copy()
    b[0, 1] = -a[0, 1]                 # 2
    b[0, 2] = 4 * a[0, 2]              # ~0
    a[0, 3] = 0.0                      # one zero row -> 1
    a[0, 4] = 0.0
    b[0, 4] = -0.0                     # two zero rows -> 0
    b[0, 5] = a[0, 5] + 1e-3 * g.standard_normal(d).astype(np.float32)
    b[0, 6, 0] = np.nextafter(a[0, 6, 0], np.float32(10))   # one ulp apart
    b[0, 7] = g.standard_normal(d).astype(np.float32)
    dist, mean = stc.dcu_distance(dev(a), dev(b))
    rd, rm = odist.distance_and_mean(a, b)
    got = dist.cpu().numpy()
    assert got[0, 0] == 0.0 and got[0, 9] == 0.0
    assert got[0, 3] == 1.0 and got[0, 4] == 0.0
    assert got[0, 1] == 2.0
    assert abs(got[0, 2]) <= 1e-7            # scaled copy: zero up to fp64 rounding
    assert abs(got[0, 6]) <= 1e-12           # one ulp apart: zero up to fp64 rounding
    keep = [0, 1, 3, 4, 5, 7, 8, 9]
    assert_rel(got[:, keep], rd[:, keep])
    assert_rel(mean.cpu().numpy(), rm, rtol=1e-5 if rm[0] > 1e-6 else 1e-3)


def test_distance_tiny_fp32_config():
    """2 layers, N=64, d=64 fp32, 25% of rows drifted by N(0, (0.05 (1+l))^2)."""
    cur = np.empty((2, 64, 64), np.float32)
    prev = np.empty_like(cur)
    for l in range(2):
        cur[l], prev[l], _ = synth.drift_pair(synth.rng(1, 2, l), 64, 64, 16, 0.05 * (1 + l),
                                              bf16=False)
    dist, mean = stc.dcu_distance(dev(cur), dev(prev))
    rd, rm = odist.distance_and_mean(cur, prev)
    assert_rel(dist.cpu().numpy(), rd)
    assert_rel(mean.cpu().numpy(), rm)


# ----------------------------------------------------------------------------- budget
def test_budget_bit_exact():
    _log("budget")
    g = synth.rng(902, 0)
    for B, L, bl in [(8, 32, 32), (3, 1, 5), (2, 64, 64), (1, 1024, 3), (4, 7, 0)]:
        s = g.uniform(0, 1e-3, (B, L)).astype(np.float32)
        if B > 1:
            s[1] = 0.0                                  # uniform row
        if B > 2:
            s[2] = 0.0
            s[2, L // 2] = 1e-4                         # one-hot row
        if B > 3:
            s[3] = np.float32(2.5e-4)                   # equal shares / ties
        got = stc.dcu_budget(dev(s.T.copy()), B, L, bl).cpu().numpy()
        ref = obud.layer_budget(s, B, L, bl)
        assert np.array_equal(got, ref), (B, L, bl)
        assert np.all(got.sum(1) == bl * L)
    got = stc.dcu_budget(None, 3, 5, 9).cpu().numpy()
    assert np.all(got == 9)
    # depth-increasing means from the drift workload
    s = np.array([[(1 + l / 8) ** 2 * 1e-5 for l in range(32)]], np.float32)
    assert np.array_equal(stc.dcu_budget(dev(s.T.copy()), 1, 32, 32).cpu().numpy(),
                          obud.layer_budget(s, 1, 32, 32))


def test_budget_negative_and_extreme_means():
    """Negative means read as 0; means spread over the fp32 exponent range; a total close to 2^31
    with 1024 layers; equal means in long runs: bit-exact against the oracle, rows summing to T."""
    _log("budget extremes")
    g = synth.rng(902, 1)
    cases = []
    s = g.uniform(-1e-3, 1e-3, (4, 16)).astype(np.float32)
    s[3] = -1.0                                                        # all negative: uniform
    cases.append((s, 7))
    cases.append(((2.0 ** g.uniform(-126, 100, (3, 1024))).astype(np.float32), (2 ** 31 - 1) // 1024))
    e = np.full((2, 300), np.float32(0.1))
    e[1, ::7] = np.float32(1e-45)
    cases.append((e, 1000))
    for s, bl in cases:
        B, L = s.shape
        got = stc.dcu_budget(dev(s.T.copy()), B, L, bl).cpu().numpy()
        ref = obud.layer_budget(s, B, L, bl)
        assert np.array_equal(got, ref), (B, L, bl)
        assert np.all(got.astype(np.int64).sum(1) == bl * L) and np.all(got >= 0)


# ----------------------------------------------------------------------------- select
def _check_select(d, budgets, layer, keys, bw):
    sel, cnt = stc.dcu_select(dev(d), dev(budgets), layer, dev(keys) if keys is not None else None, bw)
    mean = torch.empty((d.shape[0],), dtype=torch.float32, device="cuda")
    sel2, cnt2 = stc.dcu_select(dev(d), dev(budgets), layer, dev(keys) if keys is not None else None, bw,
                                mean=mean)
    # the optional layer mean: the fp64 sum of the fp32 distances over N
    ref_mean = d.astype(np.float64).mean(axis=1)
    assert np.allclose(mean.cpu().numpy(), ref_mean, rtol=1e-6, atol=0)
    B, N = d.shape
    kp = keys if keys is not None else np.zeros((B, 0), np.int32)
    rs, rc = osel.select(d, budgets, layer, kp, bw)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(sel.cpu().numpy(), rs)
    assert np.array_equal(sel.cpu().numpy(), sel2.cpu().numpy())


@pytest.mark.parametrize("N", [1, 7, 64, 1000, 1024, 2048, 4097, 8192])
def test_select_bit_exact(N):
    _log(f"select N={N}")
    g = synth.rng(903, N)
    B, L = 4, 6
    d = g.uniform(0, 1e-3, (B, N)).astype(np.float32)
    d[g.random((B, N)) < 0.3] = 0.0                           # unchanged rows
    d[g.random((B, N)) < 0.1] = np.float32(5e-4)              # ties
    d[1] = np.float32(7e-5)                                   # a row of all-equal distances
    budgets = g.integers(-2, max(3, N // 3), (B, L)).astype(np.int32)
    budgets[0, 2] = N + 5                                     # more than the candidates
    budgets[2, 2] = 0
    keys = g.integers(-2, N + 2, (B, 4)).astype(np.int32)
    keys[3] = [-1, 0, N - 1, N // 2]
    for bw in [0, 1, 8, 32]:
        _check_select(d, budgets, 2, keys, bw)
    _check_select(d, budgets, 5, None, 0)


@pytest.mark.parametrize("N,frac", [(2048, 0.3), (2048, 0.9), (8192, 0.1), (8192, 0.6), (1024, 1.0)])
def test_select_candidate_fractions(N, frac):
    """Few and many candidates (distance > 0 outside the windows), ties included, at 1, 2 and 8
    positions per thread: the oracle's selection bit for bit."""
    _log(f"select paths N={N} frac={frac}")
    g = synth.rng(905, N)
    B, L = 3, 4
    d = g.uniform(1e-6, 1e-3, (B, N)).astype(np.float32)
    d[g.random((B, N)) >= frac] = 0.0
    ties = g.random((B, N)) < 0.15
    d[ties & (d > 0)] = np.float32(2.5e-4)
    budgets = g.integers(1, max(2, int(N * frac)), (B, L)).astype(np.int32)
    keys = g.integers(0, N, (B, 4)).astype(np.int32)
    for bw in [0, 16]:
        _check_select(d, budgets, 1, keys, bw)


@pytest.mark.parametrize("N", [64, 3000])
def test_select_threshold_paths(N):
    """The radix search's exits: the threshold bin taken whole at the first pass (every key of the
    top exponent byte), a run of equal keys cut by the budget (the position-order tie ranks after
    the last pass), no budget, and a budget of every candidate; 256- and 1024-thread workgroups."""
    _log(f"select threshold paths N={N}")
    g = synth.rng(907, N)
    d = np.zeros((4, N), np.float32)
    for b in range(4):
        hi = g.choice(N, 10, replace=False)
        rest = np.setdiff1d(np.arange(N), hi)
        lo = g.choice(rest, 20, replace=False)
        d[b, hi] = np.float32(2.0)     # exponent byte 0x40
        d[b, lo] = np.float32(0.5)     # exponent byte 0x3f
    # budgets: 10 (the 2.0 keys: their first-pass bin whole), 5 (part of a tie run), 0, 30 (all)
    budgets = np.array([[10], [5], [0], [30]], np.int32)
    keys = np.zeros((4, 0), np.int32)
    sel, cnt = stc.dcu_select(dev(d), dev(budgets), 0, None, 0)
    rs, rc = osel.select(d, budgets, 0, keys, 0)
    assert rc.tolist() == [10, 5, 0, 30]
    assert np.array_equal(cnt.cpu().numpy(), rc) and np.array_equal(sel.cpu().numpy(), rs)


def test_select_identical_inputs_give_only_windows():
    d = np.zeros((2, 1024), np.float32)
    budgets = np.full((2, 32), 32, np.int32)
    keys = np.array([[600, 900, -1, -1], [0, 1023, 512, 513]], np.int32)
    sel, cnt = stc.dcu_select(dev(d), dev(budgets), 31, dev(keys), 32)
    rs, rc = osel.select(d, budgets, 31, keys, 32)
    assert np.array_equal(sel.cpu().numpy(), rs) and np.array_equal(cnt.cpu().numpy(), rc)
    assert cnt.cpu().numpy().tolist() == [64, 16 + 17 + 33]


def test_select_on_drift_distances():
    """Distances of the 32-layer drift workload feed the selection (budgets from the means)."""
    L, N, d = 8, 1024, 4096
    B = 1
    cur = np.empty((L, N, d), np.uint16)
    prev = np.empty_like(cur)
    for l in range(L):
        cur[l], prev[l], _ = synth.drift_pair(synth.rng(2, 1, l), N, d, 307, 0.01 * (1 + l / 8))
    dist, mean = stc.dcu_distance(dev_bf16(cur), dev_bf16(prev))
    budgets = stc.dcu_budget(mean.view(L, 1), 1, L, 32)
    keys = synth.key_positions(synth.rng(2, 2), 1, 4, 512, 1024)
    dk = dev(keys)
    dist_h = dist.cpu().numpy()
    bud_h = budgets.cpu().numpy()
    assert np.array_equal(bud_h, obud.layer_budget(mean.cpu().numpy().reshape(1, L), 1, L, 32))
    for l in range(L):
        m = torch.empty((1,), dtype=torch.float32, device="cuda")
        sel, cnt = stc.dcu_select(dist[l:l + 1].contiguous(), budgets, l, dk, 32, mean=m)
        rs, rc = osel.select(dist_h[l:l + 1], bud_h, l, keys, 32)
        assert np.array_equal(sel.cpu().numpy(), rs) and np.array_equal(cnt.cpu().numpy(), rc)
        # the select kernel's layer mean is dcu_distance's, bit for bit
        assert m.cpu().numpy().view(np.uint32)[0] == mean.cpu().numpy()[l:l + 1].view(np.uint32)[0]


# ----------------------------------------------------------------------------- confidence
@pytest.mark.parametrize("R,V,ld,bf16", [(16, 1000, 1000, False), (64, 126464, 126464, True),
                                         (7, 1001, 1008, True), (5, 3, 4, False), (3, 9, 16, True)])
def test_confidence(R, V, ld, bf16):
    _log(f"confidence R={R} V={V}")
    g = synth.rng(904, R, V)
    z, _ = synth.planted_logits(g, R, ld, bf16=bf16)
    if R > 2:
        z[2] = z[2, 0]                                 # every logit equal: c = 1/V, token 0
        if bf16:
            z[1, [5 % V, 1 % V]] = synth.f32_to_bf16(np.array([30.0], np.float32))[0]
        else:
            z[1, [5 % V, 1 % V]] = 30.0                # tie between two maxima -> lower index
    t = dev_bf16(z) if bf16 else dev(z)
    c, tok = stc.dllm_confidence(t, V)
    c2, tok2 = stc.dllm_confidence(t, V)
    rc, rt = oconf.confidence64(z, V)
    assert np.array_equal(tok.cpu().numpy(), rt)
    assert_rel(c.cpu().numpy(), rc)
    assert np.array_equal(c.cpu().numpy(), c2.cpu().numpy())


@pytest.mark.parametrize("peak", [16.0, 300.0, 1000.0, -500.0])
def test_confidence_large_logits(peak):
    """Rows whose maximum is far from 0 (a planted peak at +300, +1000, or every logit near -500):
    the exponentials are taken of z - max z, so the confidence carries no bias that grows with
    |max z|; 1e-5 relative against the fp64 oracle."""
    _log(f"confidence peak {peak}")
    R, V = 24, 126464
    g = synth.rng(904, 7, int(abs(peak)))
    z = g.standard_normal((R, V)).astype(np.float32) * np.float32(3.0)
    if peak > 0:
        z[np.arange(R), g.integers(0, V, R)] = np.float32(peak) + g.uniform(0, 4, R).astype(np.float32)
    else:
        z += np.float32(peak)
    zb = synth.f32_to_bf16(z)
    for t, arr in ((dev_bf16(zb), zb), (dev(z), z)):
        c, tok = stc.dllm_confidence(t, V)
        rc, rt = oconf.confidence64(arr, V)
        assert np.array_equal(tok.cpu().numpy(), rt)
        assert_rel(c.cpu().numpy(), rc)


def test_confidence_full_size_sampled():
    """[8 x 256, 126464] bf16 planted logits; the oracle checks a sample of rows."""
    _log("confidence full size")
    R, V = 2048, 126464
    z, _ = synth.planted_logits(synth.rng(5, 0), R, V)
    c, tok = stc.dllm_confidence(dev_bf16(z), V)
    rows = np.arange(0, R, 16)
    rc, rt = oconf.confidence64(z[rows], V)
    assert np.array_equal(tok.cpu().numpy()[rows], rt)
    assert_rel(c.cpu().numpy()[rows], rc)


# ----------------------------------------------------------------------------- commit
def _check_commit(c, delta, m_valid=None):
    t = dev(c)
    mv = dev(m_valid) if m_valid is not None else None
    n, order = stc.frechet_commit(t, delta, mv)
    rn, ro = ofre.frechet_commit(c, m_valid, delta)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(order.cpu().numpy(), ro)


def test_commit_bit_exact():
    _log("commit")
    g = synth.rng(905, 0)
    c = synth.confidence_profile(g, 8, 256, 0.0, 1.0)
    for delta in [0.0, 0.1, 0.25, 0.9]:
        _check_commit(c, delta)
    # high-confidence heterogeneous profiles commit many
    c = (1 - g.uniform(0, 0.02, (4, 64)) ** 2).astype(np.float32)
    _check_commit(c, 0.1)
    _check_commit(c, 0.0)
    # ties, the page's profile, valid counts and empty rows
    c = np.zeros((4, 16), np.float32)
    c[0, :5] = [0.99, 0.95, 0.82, 0.78, 0.74]
    c[1] = 0.9
    c[2, ::2] = 0.97
    c[3] = g.uniform(0, 1, 16)
    _check_commit(c, 0.3, np.array([5, 16, 16, 0], np.int32))
    _check_commit(c, 0.25, np.array([5, 3, 1, 17], np.int32))


@pytest.mark.parametrize("m", [1, 2, 255, 1000, 4096, 8192])
def test_commit_sizes(m):
    g = synth.rng(905, m)
    c = (1 - g.uniform(0, 0.05, (3, m)) ** 3).astype(np.float32)
    _check_commit(c, 0.1)
    _check_commit(c, 0.0, np.array([m, m // 2, 0], np.int32))


def test_commit_outside_exactness_precondition_uses_sequential_sums():
    g = synth.rng(905, 77)
    c = g.uniform(0.9, 1.0, (2, 300)).astype(np.float32)
    c[0, 5] = np.float32(1e-30)       # below 2^-17
    c[1, 7] = np.float32(1.5)         # above 1
    _check_commit(c, 0.1)


def _check_rule(c, rule, param, m_valid=None):
    n, order = stc.dllm_commit(dev(c), rule, param, dev(m_valid) if m_valid is not None else None)
    rn, ro = ofre.commit(c, m_valid, rule, param)
    assert np.array_equal(n.cpu().numpy(), rn), (rule, param)
    assert np.array_equal(order.cpu().numpy(), ro)
    return n.cpu().numpy()


@pytest.mark.parametrize("m", [1, 5, 256, 1000, 8192])
def test_commit_rules_bit_exact(m):
    """dllm_commit under the Frechet, factor and threshold rules against the oracle, bit for bit;
    on the same profiles Frechet(delta) >= factor(1 - delta) (Corollary 4.4)."""
    _log(f"commit rules m={m}")
    g = synth.rng(906, m)
    c = (1 - g.uniform(0, 0.3, (6, m)) ** 2).astype(np.float32)
    c[1] = g.uniform(0, 1, m)
    c[2] = np.float32(0.9)                                   # all tied, equal to tau below
    if m >= 5:
        c[3, :5] = [0.99, 0.95, 0.82, 0.78, 0.74]
    mv = np.array([m, m, m, min(m, 5), m // 2, 0], np.int32)
    for delta in [0.0, 0.1, 0.25]:
        nf = _check_rule(c, "frechet", delta, mv)
        nc = _check_rule(c, "factor", 1.0 - delta, mv)
        assert np.all(nf >= nc)
    for f in [0.0, 0.5, 0.75, 2.0]:
        _check_rule(c, "factor", f, mv)
    for tau in [0.0, 0.5, float(np.float32(0.9)), 0.95, 1.5]:
        _check_rule(c, "threshold", tau)
        _check_rule(c, "threshold", tau, mv)


def test_confidence_then_commit_full_end_of_step():
    """End of step at full size: confidence over [8 x 256, 126464] logits, then commit with
    delta = 0.1; the commit must agree exactly with the oracle rule applied to the GPU confidences
    (same-input parity), and the confidences with the oracle's within 1e-5."""
    R, V = 2048, 126464
    z, _ = synth.planted_logits(synth.rng(5, 1), R, V)
    c, tok = stc.dllm_confidence(dev_bf16(z), V)
    n, order = stc.frechet_commit(c.view(8, 256), 0.1)
    ch = c.cpu().numpy().reshape(8, 256)
    rn, ro = ofre.frechet_commit(ch, None, 0.1)
    assert np.array_equal(n.cpu().numpy(), rn)
    assert np.array_equal(order.cpu().numpy(), ro)


# ----------------------------------------------------------------------------- APD (next row f2)
from oracle import apd as oapd  # noqa: E402


def _apd_case(g, R, V, bf16):
    z, _ = synth.planted_logits(g, R, V, bf16=bf16)
    zp, _ = synth.planted_logits(g, R, V, bf16=bf16)
    if R > 3:
        zp[1] = z[1]                               # an unchanged distribution: H = 0
        vals = synth.bf16_to_f32(z[2]) if bf16 else z[2]
        z[2, 3 % V] = z[2, int(np.argmax(vals))]   # a tie at the top (same bit pattern)
    # rows padded to whole 16-byte chunks with large values that must be ignored (columns >= V)
    ld = -(-V // (8 if bf16 else 4)) * (8 if bf16 else 4)
    big = synth.f32_to_bf16(np.array([30.0], np.float32))[0] if bf16 else np.float32(30.0)
    pad = lambda a: np.concatenate([a, np.full((R, ld - V), big, a.dtype)], axis=1)  # noqa: E731
    return pad(z), pad(zp)


@pytest.mark.parametrize("R,V,bf16", [(9, 1, False), (16, 5, True), (37, 1000, True),
                                      (12, 1003, False), (4, 126464, True)])
def test_apd_signals_and_thresholds(R, V, bf16):
    """dllm_apd over two consecutive steps against the oracle: confidence, argmax, concentration,
    instability and the threshold update; the row max it keeps feeds the next step."""
    _log(f"apd R={R} V={V} bf16={bf16}")
    g = synth.rng(907, R, V)
    z1, z2 = _apd_case(g, R, V, bf16)
    to_dev = dev_bf16 if bf16 else dev
    alpha, beta = 0.1, 0.2
    tau = torch.full((R,), 0.9, dtype=torch.float32, device="cuda")
    zmax = torch.empty((R,), dtype=torch.float32, device="cuda")
    c1 = torch.empty_like(tau)
    h1 = torch.empty_like(tau)
    # step 1: no previous distribution (H = 0)
    conf, tok, _, _ = stc.dllm_apd(to_dev(z1), None, V, alpha, beta, tau, zmax, c_conc=c1, h_instab=h1)
    pm, rt, rc, rh = oapd.signals(z1, None, V)
    assert np.array_equal(tok.cpu().numpy(), rt)
    assert_rel(conf.cpu().numpy(), pm)
    assert np.allclose(c1.cpu().numpy(), rc, rtol=0, atol=2e-6)
    assert np.all(h1.cpu().numpy() == 0)
    tau_ref = oapd.update_threshold(np.full(R, 0.9, np.float32), rc, rh, alpha, beta)
    assert np.allclose(tau.cpu().numpy(), tau_ref, rtol=0, atol=1e-6)
    zv = synth.bf16_to_f32(z1[:, :V]) if bf16 else z1[:, :V]
    assert np.array_equal(zmax.cpu().numpy(), zv.max(axis=1))
    # step 2: the previous logits and the row max kept by step 1
    tau_prev = tau.cpu().numpy().copy()
    conf, tok, _, _ = stc.dllm_apd(to_dev(z2), to_dev(z1), V, alpha, beta, tau, zmax, c_conc=c1,
                                   h_instab=h1)
    pm, rt, rc, rh = oapd.signals(z2, z1, V)
    assert np.array_equal(tok.cpu().numpy(), rt)
    assert_rel(conf.cpu().numpy(), pm)
    assert np.allclose(c1.cpu().numpy(), rc, rtol=0, atol=2e-6)
    assert np.allclose(h1.cpu().numpy(), rh, rtol=0, atol=1e-5)
    assert np.allclose(tau.cpu().numpy(), oapd.update_threshold(tau_prev, rc, rh, alpha, beta),
                       rtol=0, atol=2e-6)


@pytest.mark.parametrize("m", [1, 7, 256, 2048])
def test_commit_per_position_thresholds(m):
    """dllm_commit with per-candidate thresholds against the oracle's unmask rule, bit for bit
    (same conf and tau on both sides)."""
    g = synth.rng(908, m)
    B = 5
    conf = g.uniform(0.3, 1.0, (B, m)).astype(np.float32)
    conf[1, ::3] = conf[1, 0]                          # ties
    tau = g.uniform(0.5, 1.0, (B, m)).astype(np.float32)
    tau[2] = 2.0                                        # nothing passes: the most confident commits
    tau[3, : m // 2] = conf[3, : m // 2]                # passes on equality
    mv = np.array([m, m, m, m // 2, 0], np.int32)
    for mvalid in (None, mv):
        n, order = stc.dllm_commit(dev(conf), "tau", m_valid=dev(mvalid) if mvalid is not None else None,
                                   tau=dev(tau))
        rn, ro = oapd.unmask(conf, tau, mvalid)
        assert np.array_equal(n.cpu().numpy(), rn)
        assert np.array_equal(order.cpu().numpy(), ro)


# ----------------------------------------------------------------------------- closed loop (f1)
@pytest.mark.parametrize("bf16", [True, False])
def test_distance_rows_equals_full_distance_and_rolls(bf16):
    """Only listed rows differ between x_cur and x_prev: dcu_distance_rows gives dcu_distance's
    result bit for bit, and the roll leaves x_prev equal to x_cur."""
    g = synth.rng(970, int(bf16))
    B, N, d = 3, 300, 256
    prev = g.standard_normal((B, N, d)).astype(np.float32)
    cur = prev.copy()
    sel = np.full((B, N), -1, np.int32)
    cnt = np.array([40, 0, 300], np.int32)
    for b in range(B):
        rows = np.sort(g.choice(N, cnt[b], replace=False))
        sel[b, :cnt[b]] = rows
        changed = rows[: cnt[b] * 3 // 4]                       # a listed row may also be unchanged
        cur[b, changed] += g.normal(0, 0.05, (len(changed), d)).astype(np.float32)
    to_dev = (lambda a: dev_bf16(synth.f32_to_bf16(a))) if bf16 else dev
    xc, xp = to_dev(cur), to_dev(prev)
    full, _ = stc.dcu_distance(xc, xp, want_mean=False)
    xp2 = xp.clone()
    got = stc.dcu_distance_rows(xc, xp2, dev(sel), dev(cnt), roll=True)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), full.cpu().numpy().view(np.uint32))
    assert torch.equal(xp2.view(torch.uint8) if bf16 else xp2, xc.view(torch.uint8) if bf16 else xc)
    assert float(got[1].abs().sum()) == 0.0
    # every position is written (an output full of NaN beforehand), also with the lists shuffled
    # and out-of-range entries among the counted ones
    sel2 = sel.copy()
    cnt2 = cnt.copy()
    for b in range(B):
        lst = np.concatenate([sel[b, :cnt[b]], np.array([-1, N, 7 * N], np.int32)[: min(3, N - cnt[b])]])
        g.shuffle(lst)
        sel2[b, :len(lst)] = lst
        cnt2[b] = len(lst)
    out = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    xp3 = xp.clone()
    got2 = stc.dcu_distance_rows(xc, xp3, dev(sel2), dev(cnt2), dist=out, roll=True)
    assert np.array_equal(got2.cpu().numpy().view(np.uint32), full.cpu().numpy().view(np.uint32))
    assert torch.equal(xp3.view(torch.uint8) if bf16 else xp3, xc.view(torch.uint8) if bf16 else xc)


def test_distance_rows_longest_sequence():
    """N = 65536 (the bitmap's limit): 200 listed rows spread over the sequence, the rest exact 0."""
    g = synth.rng(970, 7)
    N, d = 65536, 64
    prev = synth.normal_bf16(g, (1, N, d))
    cur = prev.copy()
    rows = np.sort(g.choice(N, 200, replace=False))
    cur[0, rows] = synth.f32_to_bf16(synth.bf16_to_f32(prev[0, rows]) + np.float32(0.1))
    sel = np.full((1, N), -1, np.int32)
    sel[0, :200] = rows
    xc, xp = dev_bf16(cur), dev_bf16(prev)
    full, _ = stc.dcu_distance(xc, xp, want_mean=False)
    out = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
    got = stc.dcu_distance_rows(xc, xp.clone(), dev(sel), dev(np.array([200], np.int32)), dist=out)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), full.cpu().numpy().view(np.uint32))


def test_commit_positions():
    g = synth.rng(971, 0)
    B, m, P = 4, 32, 4
    conf = g.uniform(0, 1, (B, m)).astype(np.float32)
    n, order = stc.frechet_commit(dev(conf), 0.0)
    n_h = n.cpu().numpy()
    n_h[2] = 0
    n_h[3] = 9
    slot_pos = (512 + g.permutation(m * B).reshape(B, m)).astype(np.int32)
    keys = stc.dllm_commit_positions(order, dev(n_h), dev(slot_pos), P).cpu().numpy()
    o = order.cpu().numpy()
    for b in range(B):
        k = min(int(n_h[b]), P)
        want = [int(slot_pos[b, o[b, j]]) for j in range(k)] + [-1] * (P - k)
        assert keys[b].tolist() == want
