"""Pins for the oracle's layer epilogue (CPU only): the sigmoid-gated shared
expert and the residual add (reading R-epilogue: the pages keep shared experts
and "gated-residual" weights on the GPU, "Strata - the details", "How it
works", and give no formula).

The gate is pinned by scipy's logistic function over an exactly rounded dot
(math.fsum), by its closed forms (0.5 at zero, 3/4 at ln 3, saturation), and by
unit vectors that pick single gate weights; the combine by dyadic inputs whose
sums are exact, so the residual and the gate must enter exactly once, in the
documented place.
"""
import math

import numpy as np
from scipy.special import expit

import oracle


def test_shared_gate_vs_scipy_over_an_exact_dot():
    g = np.random.default_rng(41)
    T, H = 5, 512
    x = g.standard_normal((T, H), dtype=np.float32)
    w = (g.standard_normal(H, dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    got = oracle.shared_gate(x, w)
    for t in range(T):
        z = math.fsum(float(a) * float(b) for a, b in zip(w, x[t]))
        assert abs(got[t] - expit(z)) <= 4e-16
    assert got.min() > 0.0 and got.max() < 1.0


def test_shared_gate_closed_forms():
    H = 256
    x = np.random.default_rng(42).standard_normal((3, H), dtype=np.float32)
    assert np.array_equal(oracle.shared_gate(x, np.zeros(H, np.float32)), [0.5, 0.5, 0.5])
    e = np.zeros((4, H), np.float32)
    e[0, 7], e[1, 7], e[2, 200], e[3, 200] = 1.0, -1.0, 1.0, -1.0
    w = np.zeros(H, np.float32)
    w[7] = np.float32(math.log(3.0))
    w[200] = 800.0
    s = oracle.shared_gate(e, w)
    z = float(np.float32(math.log(3.0)))          # the gate weight as stored
    assert abs(s[0] - 1.0 / (1.0 + 1.0 / 3.0)) <= abs(z - math.log(3.0)) + 1e-16   # 3/4 at ln 3
    assert abs(s[0] + s[1] - 1.0) <= 1e-16        # sigma(z) + sigma(-z) = 1
    assert s[2] == 1.0 and s[3] == 0.0            # saturation, no overflow


def test_shared_gate_picks_the_weight_of_a_unit_vector():
    H = 512
    w = np.arange(H, dtype=np.float32) / np.float32(64.0) - np.float32(4.0)
    for i in (0, 1, 255, 256, 511):
        x = np.zeros((1, H), np.float32)
        x[0, i] = 1.0
        assert oracle.shared_gate(x, w)[0] == 1.0 / (1.0 + math.exp(-float(w[i])))


def test_combine_residual_and_gate_enter_once_in_place():
    g = np.random.default_rng(43)
    T, k, H = 3, 4, 32
    dy = lambda *s: g.integers(-64, 65, s).astype(np.float64) / 8.0   # dyadic: sums are exact
    y, w, ys, r = dy(T * k, H), dy(T, k), dy(T, H), dy(T, H)
    ss = np.array([1.0, 0.5, -2.0])
    gate = np.array([0.25, 0.75, 0.5])
    base = oracle.combine(y, w)
    assert np.array_equal(oracle.combine(y, w, residual=r), base + r)
    assert np.array_equal(oracle.combine(y, w, ys, ss, gate), base + (ss * gate)[:, None] * ys)
    assert np.array_equal(oracle.combine(y, w, ys, None, gate), base + gate[:, None] * ys)
    full = oracle.combine(y, w, ys, ss, gate, r)
    assert np.array_equal(full, base + (ss * gate)[:, None] * ys + r)
    # without a shared expert the gate has nothing to scale
    assert np.array_equal(oracle.combine(y, w, None, ss, gate, r), base + r)
