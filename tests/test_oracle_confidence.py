"""Pins of the oracle's confidence (argmax probability of a temperature-1 softmax over the vocab;
Fast-dLLM++ notes, overall framework) against closed forms and torch.softmax."""
import math

import numpy as np
import pytest
import torch

from oracle import confidence as oc
from workloads import synth


def test_uniform_logits():
    z = np.zeros((3, 1000), np.float32)
    c, t = oc.confidence64(z)
    np.testing.assert_allclose(c, 1e-3, rtol=1e-14)
    assert t.tolist() == [0, 0, 0]


@pytest.mark.parametrize("a,b,V", [(3.0, 0.0, 10), (0.5, -2.0, 126464), (-1.0, -1.5, 7)])
def test_two_level_closed_form(a, b, V):
    z = np.full((1, V), b, np.float64)
    z[0, V // 2] = a
    c, t = oc.confidence64(z)
    ref = math.exp(a) / (math.exp(a) + (V - 1) * math.exp(b))
    assert c[0] == pytest.approx(ref, rel=1e-12)
    assert t[0] == V // 2


def test_shift_invariance_and_dominant_logit():
    g = synth.rng(500, 0)
    z = g.standard_normal((4, 333))
    c1, t1 = oc.confidence64(z)
    c2, t2 = oc.confidence64(z + 17.25)
    np.testing.assert_allclose(c1, c2, rtol=1e-12)
    assert np.array_equal(t1, t2)
    z[:, 5] = 80.0
    c, t = oc.confidence64(z)
    assert np.all(t == 5) and np.all(c >= 1 - 1e-15)


def test_ties_take_the_lowest_index():
    z = np.zeros((1, 50), np.float32)
    z[0, [9, 3, 40]] = 2.0
    _, t = oc.confidence(z)
    assert t[0] == 3


def test_against_torch_softmax_on_planted_logits():
    g = synth.rng(500, 1)
    z, idx = synth.planted_logits(g, 16, 1000)
    c, t = oc.confidence64(z)
    zt = torch.tensor(synth.bf16_to_f32(z), dtype=torch.float64)
    p = torch.softmax(zt, dim=1)
    pm, pt = p.max(dim=1)
    np.testing.assert_allclose(c, pm.numpy(), rtol=1e-12)
    assert np.array_equal(t, pt.numpy())


def test_leading_dimension_is_respected():
    z = np.zeros((2, 12), np.float32)
    z[:, 11] = 9.0           # outside the first V = 10 columns
    z[:, 4] = 1.0
    c, t = oc.confidence64(z, V=10)
    assert np.all(t == 4)
    np.testing.assert_allclose(c, math.e / (math.e + 9), rtol=1e-13)
