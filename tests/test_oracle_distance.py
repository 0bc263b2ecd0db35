"""Pins of the oracle's token distance and layer mean against closed forms and 50-digit brute force.

The distance is the cosine distance of the Dynamic-dLLM notes (Key design 1, d_i^{t,l} equation);
the mean is the layer dynamics s^{t,l} = (1/N) sum_i d_i.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import distance as od
from workloads import synth


def _row_pair(a, b):
    return np.asarray([a], np.float32), np.asarray([b], np.float32)


def test_identical_rows_are_exactly_zero():
    g = synth.rng(100, 0)
    x = synth.normal_bf16(g, (3, 17, 64))
    d = od.cosine_distance(x, x.copy())
    assert np.all(d == 0.0)
    s = od.layer_mean(d)
    assert np.all(s == 0.0)


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_scaling_is_zero(k):
    g = synth.rng(100, 1)
    a = g.standard_normal((5, 33)).astype(np.float32)
    d = od.cosine_distance64(a, a * np.float32(2.0 ** k))
    assert np.all(np.abs(d) <= 1e-15)


def test_negation_is_two_and_orthogonal_is_one():
    a = np.array([1.0, 2.0, -3.0, 0.5], np.float32)
    d = od.cosine_distance64(*_row_pair(a, -a))
    assert d[0] == pytest.approx(2.0, abs=1e-15)
    b = np.array([2.0, -1.0, 0.0, 0.0], np.float32)  # <a, b> = 0
    d = od.cosine_distance64(*_row_pair(a, b))
    assert d[0] == pytest.approx(1.0, abs=1e-15)


@pytest.mark.parametrize("theta", [1e-3, 0.1, 0.7, 1.5, 2.5, 3.0])
def test_plane_rotation_closed_form(theta):
    # unit vector and its rotation by theta in a 2-D plane embedded in 8 dims: d = 1 - cos(theta)
    u = np.zeros(8)
    v = np.zeros(8)
    u[2] = 1.0
    v[2] = math.cos(theta)
    v[5] = math.sin(theta)
    d = od.cosine_distance64(u[None], v[None])[0]
    assert d == pytest.approx(1.0 - math.cos(theta), rel=1e-12, abs=1e-16)


def test_symmetric_and_scale_invariant():
    g = synth.rng(100, 2)
    a = g.standard_normal((7, 40))
    b = a + 0.1 * g.standard_normal((7, 40))
    d1 = od.cosine_distance64(a, b)
    d2 = od.cosine_distance64(b, a)
    d3 = od.cosine_distance64(3.7 * a, 0.25 * b)
    np.testing.assert_allclose(d1, d2, rtol=1e-13)
    np.testing.assert_allclose(d1, d3, rtol=1e-10)


def test_zero_norm_readings():
    z = np.zeros(6, np.float32)
    nz = -np.zeros(6, np.float32)
    a = np.arange(1, 7, dtype=np.float32)
    assert od.cosine_distance64(*_row_pair(z, a))[0] == 1.0
    assert od.cosine_distance64(*_row_pair(a, z))[0] == 1.0
    assert od.cosine_distance64(*_row_pair(z, nz))[0] == 0.0   # +0 vs -0 rows: both zero vectors


def _decimal_distance(a, b):
    getcontext().prec = 50
    A = [Decimal(float(x)) for x in a]
    B = [Decimal(float(x)) for x in b]
    dot = sum(x * y for x, y in zip(A, B))
    na = sum(x * x for x in A)
    nb = sum(y * y for y in B)
    return Decimal(1) - dot / (na * nb).sqrt()


@pytest.mark.parametrize("sigma", [1e-3, 1e-2, 0.3])
def test_fp64_against_50_digit_brute_force(sigma):
    g = synth.rng(100, 3, int(sigma * 1e4))
    x_cur, x_prev, rows = synth.drift_pair(g, 12, 48, 12, sigma, bf16=True)
    d = od.cosine_distance64(x_cur, x_prev)
    a = synth.bf16_to_f32(x_cur)
    b = synth.bf16_to_f32(x_prev)
    for i in range(12):
        ref = _decimal_distance(a[i], b[i])
        if ref == 0:
            assert d[i] == 0.0
        else:
            # fp64 evaluation of 1 - q with q ~ 1 is accurate to a few ulp of 1 in absolute terms
            assert abs(Decimal(float(d[i])) - ref) <= Decimal("1e-15") + Decimal("1e-12") * abs(ref)


def test_fp32_output_is_rounded_fp64():
    g = synth.rng(100, 4)
    x_cur, x_prev, _ = synth.drift_pair(g, 64, 96, 32, 0.05)
    d64 = od.cosine_distance64(x_cur, x_prev)
    d32 = od.cosine_distance(x_cur, x_prev)
    assert d32.dtype == np.float32
    assert np.array_equal(d32, d64.astype(np.float32))


def test_layer_mean_is_plain_average_per_group():
    g = synth.rng(100, 5)
    d = g.uniform(0, 1e-3, size=(4, 37)).astype(np.float32)
    d[2] = 0.0
    s = od.layer_mean(d)
    for k in range(4):
        ref = math.fsum(float(v) for v in d[k]) / 37
        assert abs(float(s[k]) - ref) <= abs(ref) * 2 ** -23
    assert s[2] == 0.0
    # a group whose distances are all equal averages to that value exactly
    e = np.full((1, 64), np.float32(3.0e-5))
    assert od.layer_mean(e)[0] == np.float32(3.0e-5)
