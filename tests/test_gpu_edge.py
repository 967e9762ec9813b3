"""GPU parity on the degenerate and boundary cases of the layer, through the C ABI.

Covered here: a single expert (E = 1, k = 1); every expert selected (k = E);
every token routed to the same experts (one bucket spanning several MFMA
tiles); all-zero activations (the quantiser's amax = 0 rule, outputs exactly 0);
the largest hidden and intermediate sizes the library takes (3,584); the
boundary of the AUTO path choice (T = 8 decode, T = 9 int8); logits tied
within one lane of the extracting wave (E = 256, 512, 1024); and graph replay
of the int8 path.  References come from the CPU oracle on the same seeded
inputs; tolerances as in the other parity tests.
"""
import numpy as np
import pytest

import oracle
from quantized_moe_ffn_amd import synth

from tests.gpu_helpers import TOL_DECODE, TOL_INT8, normwise_err, oracle_pairs, oracle_shared

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _say(*a):
    print(*a, flush=True)


def _layer(**over):
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS["tiny"].__dict__, **over})
    return layers.make_layer(w, seed=11, index=0, device=DEV), w


def _forward(m, dl, logits, x, k, flags, fused):
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    bufs = m.forward(dl.layer, lg, xt, k, flags=flags, fused=fused)
    m.moe_check_device_errors()
    return bufs


def _reference(dl, w, logits, x, mode):
    k = w.top_k
    T = x.shape[0]
    idx, wts = oracle.route_topk(logits, k)
    y, hb = oracle_pairs(dl, idx.reshape(-1), np.repeat(np.arange(T), k), x, mode)
    ys = oracle_shared(dl, hb, np.arange(T), x, mode) if w.shared else None
    return y, ys, oracle.combine(y, wts, ys), idx


def _check(m, dl, w, logits, x, flags, fused, tol):
    mode = 1 if flags == m.MOE_FFN_INT8 else 0
    bufs = _forward(m, dl, logits, x, w.top_k, flags, fused)
    y, ys, out, idx = _reference(dl, w, logits, x, mode)
    assert np.array_equal(bufs.routing.idx.cpu().numpy(), idx)
    ey = normwise_err(bufs.y_pair.cpu().numpy(), y)
    eo = normwise_err(bufs.out.cpu().numpy(), out)
    _say("  y_pair err max %.3e  out err max %.3e" % (ey.max(), eo.max()))
    assert ey.max() <= tol and eo.max() <= tol
    if ys is not None:
        assert normwise_err(bufs.y_shared.cpu().numpy(), ys).max() <= tol
    return bufs


PATHS = [("decode", False), ("decode", True), ("int8", False), ("int8", True)]


def _flags(m, path):
    return m.MOE_FFN_INT8 if path == "int8" else m.MOE_FFN_DECODE


@pytest.mark.parametrize("path,fused", PATHS)
@pytest.mark.parametrize("over", [
    dict(n_experts=1, top_k=1, tokens=5),                     # a single expert
    dict(n_experts=4, top_k=4, tokens=3, shared=True),        # every expert selected, plus the shared one
    dict(n_experts=4, top_k=4, tokens=70),                    # k = E with 70 tokens per bucket
])
def test_degenerate_expert_counts(over, path, fused):
    m = qm()
    _say("edge", over, path, fused)
    dl, w = _layer(**over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=12)
    _check(m, dl, w, logits, x, _flags(m, path), fused, TOL_INT8 if path == "int8" else TOL_DECODE)


@pytest.mark.parametrize("path,fused", PATHS)
def test_every_token_on_the_same_experts(path, fused):
    """Identical logit rows: all pairs land in k buckets; the int8 path then tiles one
    expert's bucket of 300 tokens into several 64-token tiles."""
    m = qm()
    dl, w = _layer(n_experts=16, top_k=3, tokens=300 if path == "int8" else 4)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=13)
    logits[:] = logits[0]
    bufs = _check(m, dl, w, logits, x, _flags(m, path), fused, TOL_INT8 if path == "int8" else TOL_DECODE)
    counts = bufs.routing.count.cpu().numpy()
    assert sorted(counts[counts > 0].tolist()) == [x.shape[0]] * 3


@pytest.mark.parametrize("path,fused", PATHS)
@pytest.mark.parametrize("E,k", [(256, 8), (512, 10), (1024, 8)])
def test_tied_logits_held_by_one_lane(E, k, path, fused):
    """Logits drawn from three values, so every lane of the extracting wave holds
    equal keys (experts e, e + 64, ...): 4, 8 or 16 keys per lane, the first two on
    the sorted per-lane lists, the last on the rescan.  The selection must still
    take equal logits in ascending expert order, on the routing outputs and inside
    the decode layer's gate/up kernel, whose waves pick their slots themselves."""
    m = qm()
    dl, w = _layer(n_experts=E, top_k=k, tokens=3)
    from quantized_moe_ffn_amd import layers
    _, x = layers.inputs_np(w, seed=17)
    logits = np.random.default_rng(E + k).integers(-1, 2, size=(3, E)).astype(np.float32)
    _check(m, dl, w, logits, x, _flags(m, path), fused, TOL_INT8 if path == "int8" else TOL_DECODE)


@pytest.mark.parametrize("path,fused", PATHS)
def test_zero_activations_give_zero_outputs(path, fused):
    """x = 0: the int8 quantiser's amax = 0 rule gives d = 0 and q = 0, h = silu(0)*0 = 0,
    and every output is exactly +-0 on both paths."""
    m = qm()
    dl, w = _layer(n_experts=8, top_k=2, tokens=6, shared=True)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=14)
    x[:] = 0.0
    bufs = _forward(m, dl, logits, x, w.top_k, _flags(m, path), fused)
    assert not np.any(bufs.out.cpu().numpy())
    assert not np.any(bufs.y_pair.cpu().numpy())
    assert not np.any(bufs.y_shared.cpu().numpy())


@pytest.mark.parametrize("path", ["decode", "int8"])
@pytest.mark.parametrize("over", [
    dict(hidden=3584, inter=256, n_experts=3, top_k=2, tokens=3),    # largest hidden: 14 blocks per gate row
    dict(hidden=256, inter=3584, n_experts=3, top_k=2, tokens=3),    # largest inter: 14 blocks per down row
])
def test_largest_dimensions(over, path):
    m = qm()
    _say("largest dims", over, path)
    dl, w = _layer(**over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=15)
    _check(m, dl, w, logits, x, _flags(m, path), True, TOL_INT8 if path == "int8" else TOL_DECODE)


@pytest.mark.parametrize("T,mode", [(8, 0), (9, 1)])
def test_auto_path_boundary(T, mode):
    """MOE_FFN_AUTO runs the fp-activation path up to 8 tokens and the int8 path above."""
    m = qm()
    dl, w = _layer(n_experts=8, top_k=2, tokens=T)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=16)
    bufs = _forward(m, dl, logits, x, w.top_k, m.MOE_FFN_AUTO, True)
    y, ys, out, idx = _reference(dl, w, logits, x, mode)
    e = normwise_err(bufs.out.cpu().numpy(), out)
    assert e.max() <= (TOL_INT8 if mode else TOL_DECODE)
    # the other path's reference is farther away (quantisation-sized) for the int8 case
    if mode == 1:
        _, _, out_fp, _ = _reference(dl, w, logits, x, 0)
        assert normwise_err(bufs.out.cpu().numpy(), out_fp).max() > 10 * e.max()


def test_int8_graph_replay_matches_eager():
    """The int8 path (routing, quantisation, tile list, MFMA GEMMs, combine) captured in a
    graph replays to the eager bits, with unrelated eager work between replays."""
    m = qm()
    dl, w = _layer(n_experts=8, top_k=2, tokens=200)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=17)
    lg = torch.from_numpy(logits).to(DEV)
    xt = torch.from_numpy(x).to(DEV)
    bufs = m.LayerBuffers(dl.layer, x.shape[0], w.top_k, m.MOE_FFN_INT8, device=DEV)
    m.forward(dl.layer, lg, xt, w.top_k, bufs, flags=m.MOE_FFN_INT8)
    torch.cuda.synchronize()
    eager = bufs.out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            m.forward(dl.layer, lg, xt, w.top_k, bufs, flags=m.MOE_FFN_INT8)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        bufs.out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()
        g.replay()
        torch.cuda.synchronize()
        float(junk)
        assert torch.equal(bufs.out, eager), rep
    m.moe_check_device_errors()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 5, dict(n_experts=64)),
    ("sage_decode", 6, dict(n_experts=64)),
    ("sage_decode", 8, dict(n_experts=64)),                 # T*k = 64, the fused path's maximum
    ("flash_next_decode", 6, dict(n_experts=64)),           # shared expert in two 4-token groups, Q8_0 down
])
def test_decode_batches_up_to_eight_tokens(name, T, over, fused):
    """Decode batches of 5-8 tokens (verify windows of prompt lookup, parallel slots) on the
    two-kernel layer (fused) and the separate calls, against the oracle."""
    m = qm()
    _say("decode batch", name, T, fused)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=18, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=18)
    _check(m, dl, w, logits, x, m.MOE_FFN_DECODE, fused, TOL_DECODE)


@pytest.mark.parametrize("path,fused", PATHS)
@pytest.mark.parametrize("T", [1, 3, 12])
def test_plain_softmax_and_shared_scale_through_the_layer(T, path, fused):
    """Routing weights from the plain softmax over all E (no renormalisation) and a
    per-token scale on the shared expert, through the whole layer (the two-kernel
    decode layer forms both in its down kernel), against the oracle."""
    m = qm()
    # (decode at 12 tokens runs the general decode kernels: past the two-kernel layer's 8)
    dl, w = _layer(n_experts=16, top_k=4, tokens=T, shared=True)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=30 + T)
    scale = np.random.default_rng(31).uniform(0.1, 2.0, T).astype(np.float32)
    lg = torch.from_numpy(logits).to(DEV)
    xt = torch.from_numpy(x).to(DEV)
    st = torch.from_numpy(scale).to(DEV)
    bufs = m.forward(dl.layer, lg, xt, w.top_k, flags=_flags(m, path), renorm=False, shared_scale=st,
                     fused=fused)
    m.moe_check_device_errors()
    mode = 1 if path == "int8" else 0
    idx, wts = oracle.route_topk(logits, w.top_k, renorm=False)
    assert np.array_equal(bufs.routing.idx.cpu().numpy(), idx)
    assert np.allclose(bufs.routing.w.cpu().numpy(), wts, rtol=0, atol=1e-6)
    assert wts.sum(axis=1).max() < 1.0    # the plain softmax leaves mass on the unselected experts
    y, hb = oracle_pairs(dl, idx.reshape(-1), np.repeat(np.arange(T), w.top_k), x, mode)
    ys = oracle_shared(dl, hb, np.arange(T), x, mode)
    out = oracle.combine(y, wts, ys, scale.astype(np.float64))
    tol = TOL_INT8 if path == "int8" else TOL_DECODE
    e = normwise_err(bufs.out.cpu().numpy(), out)
    _say("  plain softmax + shared scale, out err max %.3e" % e.max())
    assert e.max() <= tol


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 9, {}),                                  # T*k = 72: just past the two-kernel layer
    ("sage_decode", 40, {}),                                 # 320 pairs: routed through the bucket kernels
    ("sage_decode", 64, dict(n_experts=16)),                 # ~32 pairs per expert: eight tiles of four each
    ("sage_decode_q5k", 16, {}),                             # Q5_K experts
    ("flash_next_decode", 12, dict(n_experts=64)),           # shared expert (three token tiles), Q8_0 down, H 2560
])
def test_decode_batches_past_eight_tokens_expert_grouped(name, T, over, fused):
    """Decode batches past the two-kernel layer (T*k > 64) on the expert-grouped kernels:
    each tile of four pairs of one expert streams that expert's rows once.  Against the
    oracle, on the layer call (fused) and the separate calls."""
    m = qm()
    _say("decode batch, expert-grouped", name, T, over, fused)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=19, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=19)
    _check(m, dl, w, logits, x, m.MOE_FFN_DECODE, fused, TOL_DECODE)


@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 24, {}),
    ("sage_decode_q5k", 12, {}),
])
def test_expert_grouped_rows_equal_the_two_kernel_layer_bitwise(name, T, over):
    """On the Sage-like shape (H 2,048: a row's 64 slices in one wave; Q4_K or Q5_K down) a
    token's per-pair outputs and layer output on the expert-grouped kernels equal, bit for
    bit, those of the two-kernel layer run on that token alone: both take the same per-lane
    slices, the same per-token dot products and lane sums in the same order, and the
    combine in slot order.  (The Q8_0 dot and the five-wave rows of H 2,560 are compiled
    with other fused multiply-adds in the two kernels' instances and agree to a few ulps;
    those shapes are checked against the oracle above.)"""
    m = qm()
    _say("expert-grouped vs two-kernel layer", name, T, over)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=20, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=20)
    big = _forward(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, True)
    k = w.top_k
    for t in (0, T // 2, T - 1):
        one = _forward(m, dl, logits[t:t + 1], x[t:t + 1], k, m.MOE_FFN_DECODE, True)
        assert torch.equal(big.routing.idx[t], one.routing.idx[0]), t
        assert torch.equal(big.y_pair[t * k:(t + 1) * k].view(torch.int32), one.y_pair.view(torch.int32)), t
        if w.shared:
            assert torch.equal(big.y_shared[t].view(torch.int32), one.y_shared[0].view(torch.int32)), t
        assert torch.equal(big.out[t].view(torch.int32), one.out[0].view(torch.int32)), t
