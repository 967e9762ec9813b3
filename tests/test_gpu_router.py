"""GPU parity of the router projection (moe_router_logits) through the C ABI.

logits[t][e] = sum_h W[e][h] x[t][h] ("Strata - the details", "How it works":
routers are a GPU stage) against the oracle's fp64 sums.  Bound: fp32
summation of H products, each a rounding of at most u = 2^-24 relative, gives
|gpu - exact| <= gamma_H * sum_h |W x| with gamma_H = H u / (1 - H u); the RMS
error over a case must also stay below 2e-6 of the RMS scale (rounding errors
of a length-H sum grow like sqrt(H) u on average).  Both kernels are covered:
up to 16 tokens the matrix-vector kernel, above it the fp32 MFMA tiles, with
ragged token and expert tiles.  The top-k taken on the GPU's logits equals the
oracle's top-k of the same logits (the decision in one precision).
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _inputs(T, H, E, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)).astype(np.float32)
    w = (g.standard_normal((E, H)) * (1.0 / np.sqrt(H))).astype(np.float32)
    return x, w


def _run(m, x, w):
    xt = torch.from_numpy(x).to(DEV)
    wt = torch.from_numpy(w).to(DEV)
    out = torch.full((x.shape[0], w.shape[0]), float("nan"), dtype=torch.float32, device=DEV)
    m.moe_router_logits(xt, wt, out)
    m.moe_check_device_errors()
    return out


def _check(got, x, w, rows=None):
    xs = x if rows is None else x[rows]
    ref = oracle.router_logits(xs, w)
    scale = np.abs(xs.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    H = x.shape[1]
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= gamma * scale), float((err / scale).max())
    rms = float(np.sqrt((err ** 2).mean()) / np.sqrt((scale ** 2).mean()))
    print("router err: max %.2e of scale, rms %.2e" % (float((err / scale).max()), rms), flush=True)
    assert rms <= 2e-6


@pytest.mark.parametrize("T,H,E", [
    (1, 2048, 256),     # Sage-like decode token
    (3, 2048, 256),     # 3-token window
    (1, 2560, 512),     # Flash-Next-like router
    (16, 256, 8),       # largest batch of the matrix-vector kernel
    (17, 512, 37),      # smallest batch of the MFMA kernel, ragged token and expert tiles
    (100, 2048, 256),
    (5, 8, 3),          # smallest hidden size
    (2, 8192, 64),      # largest hidden size
])
def test_router_matches_oracle(T, H, E):
    m = qm()
    x, w = _inputs(T, H, E, seed=T * 7 + E)
    got = _run(m, x, w).cpu().numpy()
    _check(got, x, w)


def test_router_prompt_chunk_sampled_rows():
    """4,096 tokens x 2,048 x 256 (the prompt-chunk shape): every logit is checked
    against the bound on 64 sampled tokens spread over all token tiles."""
    m = qm()
    x, w = _inputs(4096, 2048, 256, seed=4)
    got = _run(m, x, w).cpu().numpy()
    rows = np.sort(np.random.default_rng(1).choice(4096, 64, replace=False))
    rows[0], rows[-1] = 0, 4095
    _check(got[rows], x, w, rows)


@pytest.mark.parametrize("T", [1, 8, 40])
def test_router_deterministic_and_row_independent(T):
    m = qm()
    x, w = _inputs(T, 2048, 256, seed=11)
    a = _run(m, x, w)
    b = _run(m, x, w)
    assert torch.equal(a, b)
    # same rows inside a batch of the same kernel (both above or both below 16 tokens)
    x2 = x.copy()
    x2[T // 2:] = np.random.default_rng(12).standard_normal(x2[T // 2:].shape).astype(np.float32)
    c = _run(m, x2, w)
    assert torch.equal(a[: T // 2], c[: T // 2])


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (3, 256, 8), (1, 512, 10), (64, 256, 8)])
def test_router_then_topk(T, E, k):
    """Router then top-k, both on the GPU: the selection equals the oracle's top-k
    of the GPU logits, and the logits pass the bound."""
    m = qm()
    x, w = _inputs(T, 2048, E, seed=20 + T)
    lg = _run(m, x, w)
    r = m.Routing(T, E, k, DEV)
    ws = torch.empty(max(m.moe_route_workspace_bytes(T, E, k), 1), dtype=torch.uint8, device=DEV)
    m.moe_route_topk(lg, k, r, True, ws)
    m.moe_check_device_errors()
    idx_ref, w_ref = oracle.route_topk(lg.cpu().numpy(), k)
    assert np.array_equal(r.idx.cpu().numpy(), idx_ref)
    assert np.allclose(r.w.cpu().numpy(), w_ref, rtol=0, atol=1e-6)
    _check(lg.cpu().numpy(), x, w)
