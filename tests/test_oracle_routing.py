"""Pins for the oracle's routing, bucketing and activation quantisation (CPU only).

Routing ("Strata-Sage-A1.5-GGUF" card: 256 experts / top-8; "Strata: a 125B MoE
at 94 tok/s" article: 10 routed of 512) is pinned against library routines
(numpy's stable argsort, scipy's softmax) and special cases; bucketing against
numpy's stable argsort; the activation quantiser (the "one quantization per
token" of the "Strata-Sage-A1.5-GGUF" round-2 table) against closed-form cases
and its defining invariants.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _stable_topk(lg, k):
    # descending logit, ties to the lower index: stable argsort of -logits
    return np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]


@pytest.mark.parametrize("T,E,k", [(5, 8, 2), (7, 256, 8), (3, 512, 10), (4, 64, 64)])
def test_topk_matches_stable_sort(T, E, k):
    g = np.random.default_rng(E + k)
    lg = g.standard_normal((T, E)).astype(np.float32)
    idx, w = oracle.route_topk(lg, k)
    assert np.array_equal(idx, _stable_topk(lg, k))
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_topk_ties_go_to_lower_index():
    g = np.random.default_rng(7)
    lg = g.integers(-3, 4, size=(50, 32)).astype(np.float32)   # many exact ties
    for k in (1, 4, 9, 32):
        idx, _ = oracle.route_topk(lg, k)
        assert np.array_equal(idx, _stable_topk(lg, k))


def test_topk_signed_zeros_tie():
    lg = np.array([[-0.0, 0.0, -1.0, 0.0], [0.0, -0.0, -0.0, -2.0]], np.float32)
    idx, w = oracle.route_topk(lg, 3)
    assert idx.tolist() == [[0, 1, 3], [0, 1, 2]]
    assert np.allclose(w, 1.0 / 3.0, atol=1e-15)


def test_k1_is_first_argmax():
    g = np.random.default_rng(8)
    lg = g.integers(-2, 3, size=(40, 16)).astype(np.float32)
    idx, w = oracle.route_topk(lg, 1)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)


def test_k_equals_E_is_softmax():
    g = np.random.default_rng(9)
    lg = (3 * g.standard_normal((6, 24))).astype(np.float32)
    idx, w = oracle.route_topk(lg, 24)
    ref = softmax(lg.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, idx, w, axis=1)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


def test_plain_softmax_without_renorm():
    g = np.random.default_rng(10)
    lg = g.standard_normal((5, 40)).astype(np.float32)
    idx, w = oracle.route_topk(lg, 6, renorm=False)
    ref = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, idx, axis=1), rtol=1e-13, atol=0)
    assert np.all(w.sum(axis=1) < 1.0)


def test_renorm_equals_softmax_of_selected():
    g = np.random.default_rng(11)
    lg = g.standard_normal((9, 256)).astype(np.float32)
    idx, w = oracle.route_topk(lg, 8)
    sel = np.take_along_axis(lg.astype(np.float64), idx, axis=1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-13, atol=0)
    # renormalised over the top-k of the full softmax, too
    full = softmax(lg.astype(np.float64), axis=1)
    topp = np.take_along_axis(full, idx, axis=1)
    assert np.allclose(w, topp / topp.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)


def test_relabelling_experts_permutes_indices():
    g = np.random.default_rng(12)
    lg = g.standard_normal((8, 64)).astype(np.float32)
    perm = g.permutation(64)
    idx, w = oracle.route_topk(lg, 8)
    idx2, w2 = oracle.route_topk(lg[:, perm], 8)
    assert np.array_equal(perm[idx2], idx)
    assert np.array_equal(w2, w)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (3, 256, 8), (64, 16, 4), (200, 256, 8)])
def test_bucket_matches_stable_sort(T, E, k):
    g = np.random.default_rng(T * 1000 + E)
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    b = oracle.bucket(idx, E)
    flat = idx.ravel()
    assert np.array_equal(b["count"], np.bincount(flat, minlength=E))
    assert b["offset"][0] == 0 and np.array_equal(np.diff(b["offset"]), b["count"])
    assert b["offset"][-1] == T * k
    assert np.array_equal(b["pair"], np.argsort(flat, kind="stable"))
    assert np.array_equal(b["active"], np.nonzero(b["count"])[0])
    assert b["n_active"] == np.count_nonzero(b["count"])
    # every pair exactly once
    assert np.array_equal(np.sort(b["pair"]), np.arange(T * k))


def test_quant_act_exact_integers():
    # amax = 127 and integer entries: id = 1, q = x, d = 1 exactly
    x = np.zeros((2, 512), np.float32)
    x[0, :256] = np.append(np.arange(-127, 128), 0.0)
    x[0, 256:] = np.linspace(-127, 127, 256).round()
    x[1, :] = 0.0
    x[1, 300] = -127.0
    xq, xd = oracle.quantize_act(x)
    assert np.array_equal(xq[0].astype(np.float32), np.clip(x[0], -127, 127))
    assert xd[0].tolist() == [1.0, 1.0]
    assert xd[1].tolist() == [0.0, 1.0]       # an all-zero block quantizes to 0 with d = 0
    assert np.all(xq[1, :256] == 0) and xq[1, 300] == -127


def test_quant_act_ties_to_even():
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 127.0
    x[0, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    xq, xd = oracle.quantize_act(x)
    assert xq[0, :7].tolist() == [127, 2, 4, -2, -4, 0, 0]


def test_quant_act_invariants_random():
    g = np.random.default_rng(13)
    x = g.standard_normal((16, 2048)).astype(np.float32) * g.uniform(0.01, 100, (16, 1)).astype(np.float32)
    xq, xd = oracle.quantize_act(x)
    blocks = x.reshape(16, 8, 256)
    q = xq.reshape(16, 8, 256).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    assert np.array_equal(xd, (amax / np.float32(127)).astype(np.float32))
    am = np.abs(blocks).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(q, am[..., None], axis=2)) == 127)
    assert np.abs(q).max() <= 127
    # reconstruction within half a step (plus fp32 rounding of the scaled value)
    err = np.abs(blocks - q * xd[..., None])
    assert np.all(err <= xd[..., None] * (0.5 + 1e-5))
