"""Pins for the oracle's router projection (CPU only).

The router is the stage before top-k ("Strata - the details", "How it works":
routers are a GPU stage and their weights live in VRAM); its plain definition
is logit_e = sum_h W[e][h] x[h].  The oracle writes that sum out as a loop; it
is pinned here against numpy's float64 matrix product (an independent library
routine), closed forms (identity rows, rows of ones, powers of two), and
linearity, with non-square shapes so that a transposed operand fails.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("T,H,E", [(1, 256, 8), (3, 512, 37), (9, 2048, 256), (2, 2560, 512)])
def test_router_matches_numpy_matmul(T, H, E):
    g = np.random.default_rng(T * 1000 + E)
    x = g.standard_normal((T, H)).astype(np.float32)
    w = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    got = oracle.router_logits(x, w)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    scale = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert got.shape == (T, E)
    assert np.all(np.abs(got - ref) <= 1e-13 * scale)


def test_router_identity_rows_pick_coordinates():
    g = np.random.default_rng(3)
    H = 64
    x = g.standard_normal((4, H)).astype(np.float32)
    w = np.zeros((H + 3, H), np.float32)
    w[:H] = np.eye(H, dtype=np.float32)
    w[H] = 1.0                       # row of ones: the plain sum
    w[H + 1, 5] = 2.0 ** 20          # a power of two scales one coordinate exactly
    w[H + 2, H - 1] = -0.5
    got = oracle.router_logits(x, w)
    assert np.array_equal(got[:, :H], x.astype(np.float64))
    for t in range(4):
        assert got[t, H] == pytest.approx(math.fsum(float(v) for v in x[t]), rel=0, abs=1e-12)
        assert got[t, H + 1] == float(x[t, 5]) * 2.0 ** 20
        assert got[t, H + 2] == -0.5 * float(x[t, H - 1])


def test_router_is_linear_and_token_independent():
    g = np.random.default_rng(5)
    x1 = g.integers(-8, 9, (3, 128)).astype(np.float32)   # small integers: every sum is exact
    x2 = g.integers(-8, 9, (3, 128)).astype(np.float32)
    w = g.integers(-4, 5, (16, 128)).astype(np.float32)
    a = oracle.router_logits(x1, w)
    b = oracle.router_logits(x2, w)
    c = oracle.router_logits(x1 + x2, w)
    assert np.array_equal(c, a + b)
    both = oracle.router_logits(np.concatenate([x1, x2]), w)
    assert np.array_equal(both, np.concatenate([a, b]))


def test_router_then_topk_of_a_planted_winner():
    # x aligned with row 11 of W gives row 11 the largest logit by construction
    g = np.random.default_rng(8)
    E, H = 32, 256
    w = g.standard_normal((E, H)).astype(np.float32)
    w /= np.linalg.norm(w, axis=1, keepdims=True).astype(np.float32)
    x = (w[11] * 10.0)[None, :].astype(np.float32)
    idx, _ = oracle.route_topk(oracle.router_logits(x, w).astype(np.float32), 1)
    assert idx[0, 0] == 11
