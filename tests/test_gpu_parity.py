"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Exact: dequantized weights (bit for bit, as the "Strata v0.1.31" release notes
require of GPU dequantizers), top-k indices, bucket lists, int8 activation codes.
Toleranced: routing weights (1e-6), FFN outputs (2e-3 decode / 5e-3 int8 path,
normwise per row).  Inputs are seeded synthetic layers with the workloads' shapes
and value laws.
"""
import numpy as np
import pytest

import oracle
from quantized_moe_ffn_amd import synth

from tests.gpu_helpers import TOL_DECODE, TOL_INT8, TOL_W, bf16_rne, normwise_err, oracle_pairs, oracle_shared

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- dequantization

def _finite_scale_blocks(g, n, qt):
    if qt == oracle.Q8_0:
        b = synth.q80_blocks_np(g, n)
    elif qt == oracle.Q5_1:
        b = synth.q51_blocks_np(g, n)
    else:
        b = synth.q4k_blocks_np(g, n, oracle.BLOCK_BYTES[qt])
    # random fp16 scale bit patterns, finite (subnormals included)
    bits = g.integers(0, 0x7C00, size=(n, 1 if qt == oracle.Q8_0 else 2), dtype=np.uint16)
    bits |= (g.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15)
    b[:, : 2 * bits.shape[1]] = bits.view(np.uint8).reshape(n, -1)
    return b


@pytest.mark.parametrize("qt", [oracle.Q4_K, oracle.Q5_K, oracle.Q8_0, oracle.Q5_1])
def test_dequant_bit_exact(qt):
    m = qm()
    from tests.golden import load_block
    g = np.random.default_rng(100 + qt)
    blocks = _finite_scale_blocks(g, 3000, qt)
    if qt == oracle.Q4_K:
        gold = np.stack([load_block(f) for f in ("q4k_block_a.txt", "q4k_block_b.txt", "q4k_block_c.txt",
                                                  "q4k_block_e.txt")])
    elif qt == oracle.Q5_K:
        gold = load_block("q5k_block_f.txt")[None]
    elif qt == oracle.Q5_1:
        gold = load_block("q51_block_g.txt")[None]
    else:
        gold = load_block("q80_block.txt")[None]
    blocks = np.concatenate([gold, blocks])
    n_w = blocks.shape[0] * oracle.BLOCK_WEIGHTS[qt]
    _say("dequant", qt, blocks.shape)
    dev = torch.from_numpy(blocks.copy()).to(DEV)
    out = torch.empty(n_w, dtype=torch.float32, device=DEV)
    m.moe_dequant_q(dev, qt, n_w, out)
    m.moe_check_device_errors()
    got = out.cpu().numpy()
    ref = oracle.dequant(blocks, qt).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------- routing

def _route(m, logits_np, k, renorm=True):
    T, E = logits_np.shape
    r = m.Routing(T, E, k, DEV)
    ws = torch.empty(max(1, m.moe_route_workspace_bytes(T, E, k)), dtype=torch.uint8, device=DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits_np)).to(DEV)
    m.moe_route_topk(lg, k, r, renorm, ws)
    m.moe_check_device_errors()
    return r


def _check_routing(r, logits_np, k, renorm=True):
    E = logits_np.shape[1]
    idx, w = oracle.route_topk(logits_np, k, renorm)
    b = oracle.bucket(idx, E)
    assert np.array_equal(r.idx.cpu().numpy(), idx)
    assert np.abs(r.w.cpu().numpy() - w).max() <= TOL_W
    assert np.array_equal(r.count.cpu().numpy(), b["count"])
    assert np.array_equal(r.offset.cpu().numpy(), b["offset"])
    assert np.array_equal(r.pair.cpu().numpy(), b["pair"])
    na = int(r.n_active.cpu().numpy()[0])
    assert na == b["n_active"]
    assert np.array_equal(r.active.cpu().numpy()[:na], b["active"])


@pytest.mark.parametrize("T,E,k,zipf", [
    (1, 8, 2, 0.0), (4, 8, 2, 0.0), (1, 256, 8, 0.0), (3, 256, 8, 0.0), (1, 512, 10, 0.0),
    (32, 256, 8, 0.0), (33, 256, 8, 0.0), (1000, 300, 5, 0.0), (4096, 256, 8, 1.1), (2, 8, 8, 0.0),
    (7, 1024, 16, 0.0), (5, 65, 1, 0.0),
])
def test_route_matches_oracle(T, E, k, zipf):
    m = qm()
    _say("route", T, E, k, zipf)
    lg = synth.logits_np(synth.rng(200, T, E, k), T, E, zipf)
    r = _route(m, lg, k)
    _check_routing(r, lg, k)


def test_route_ties_signed_zeros_and_plain_softmax():
    m = qm()
    g = np.random.default_rng(201)
    lg = g.integers(-2, 3, size=(40, 64)).astype(np.float32)
    lg[lg == 0] = np.where(g.random(np.count_nonzero(lg == 0)) < 0.5, -0.0, 0.0).astype(np.float32)
    for k in (1, 3, 8, 16):
        _say("route ties", k)
        _check_routing(_route(m, lg, k), lg, k)
    lg2 = synth.logits_np(synth.rng(202), 300, 128)   # large path, plain softmax
    _check_routing(_route(m, lg2, 6, renorm=False), lg2, 6, renorm=False)


@pytest.mark.parametrize("E", [128, 256, 512, 1024])
def test_route_ties_held_by_one_lane(E):
    """Ties between experts of one lane (e and e + 64, ...): 2 to 16 keys per lane,
    sorted once per lane up to 8, rescanned above; equal logits in ascending
    expert order either way."""
    m = qm()
    lg = np.random.default_rng(203 + E).integers(-1, 2, size=(24, E)).astype(np.float32)
    for k in (1, 5, 8, 16):
        _say("route ties in a lane", E, k)
        _check_routing(_route(m, lg, k), lg, k)


# --------------------------------------------------------------------------- activation quantisation

def test_quantize_act_bit_exact():
    m = qm()
    g = np.random.default_rng(300)
    x = (g.standard_normal((37, 2048)) * g.uniform(1e-3, 1e3, (37, 1))).astype(np.float32)
    x[3, 256:512] = 0.0
    x[4, :256] = np.round(x[4, :256])
    x[4, 0] = 127.0
    x[4, 1:5] = [2.5, -2.5, 0.5, 3.5]
    # values a few ulps from rounding ties, where rint(x/d) or rint(x*127/amax) would give
    # other codes than the rule's rint(x * fl(127/amax))
    from tests.test_oracle_int8_pins import _near_ties
    for t in range(8, 16):
        amax = np.float32(g.uniform(0.1, 300.0))
        vals = _near_ties(amax, g)
        x[t, :256] = np.float32(0.01) * amax
        x[t, 0] = amax
        x[t, 1:1 + len(vals)] = vals
    xt = torch.from_numpy(x).to(DEV)
    xq = torch.empty((37, 2048), dtype=torch.int8, device=DEV)
    xd = torch.empty((37, 8), dtype=torch.float32, device=DEV)
    m.moe_quantize_act(xt, xq, xd)
    m.moe_check_device_errors()
    rq, rd = oracle.quantize_act(x)
    assert np.array_equal(xq.cpu().numpy(), rq)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), rd.view(np.uint32))


def test_quantize_act_nonfinite_raises_error_word():
    m = qm()
    x = np.ones((2, 256), np.float32)
    x[1, 7] = np.inf
    xt = torch.from_numpy(x).to(DEV)
    xq = torch.empty((2, 256), dtype=torch.int8, device=DEV)
    xd = torch.empty((2, 1), dtype=torch.float32, device=DEV)
    m.moe_quantize_act(xt, xq, xd)
    with pytest.raises(m.MoeError, match="non-finite activation"):
        m.moe_check_device_errors()
    assert np.all(xq.cpu().numpy()[1] == 0) and xd.cpu().numpy()[1, 0] == 0.0
    m.moe_check_device_errors()   # cleared


# --------------------------------------------------------------------------- whole layer

def _layer(name, **over):
    from quantized_moe_ffn_amd import layers
    w = synth.WORKLOADS[name]
    if over:
        w = synth.Workload(**{**w.__dict__, **over})
    return layers.make_layer(w, seed=0, index=0, device=DEV), w


def _run_layer(m, dl, logits, x, k, flags, fused=True):
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    bufs = m.forward(dl.layer, lg, xt, k, flags=flags, fused=fused)
    m.moe_check_device_errors()
    return bufs


def _check_layer(m, dl, w, logits, x, bufs, mode, tol, token_subset=None):
    k = w.top_k
    T = x.shape[0]
    idx, wts = oracle.route_topk(logits, k)
    assert np.array_equal(bufs.routing.idx.cpu().numpy(), idx)
    assert np.abs(bufs.routing.w.cpu().numpy() - wts).max() <= TOL_W
    toks = np.arange(T) if token_subset is None else np.asarray(token_subset)
    pe = idx[toks].reshape(-1)
    pt = np.repeat(toks, k)
    y_ref, hb = oracle_pairs(dl, pe, pt, x, mode)
    pairs = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    y_got = bufs.y_pair.cpu().numpy()[pairs]
    ep = normwise_err(y_got, y_ref)
    ys = None
    if w.shared:
        ys = oracle_shared(dl, hb, toks, x, mode)
        es = normwise_err(bufs.y_shared.cpu().numpy()[toks], ys)
        assert es.max() <= tol, es.max()
    out_ref = oracle.combine(y_ref, wts[toks], ys)
    out_got = bufs.out.cpu().numpy()[toks]
    eo = normwise_err(out_got, out_ref)
    _say("  y_pair err max %.3e  out err max %.3e" % (ep.max(), eo.max()))
    if mode == 1 and (ep.max() > tol or eo.max() > tol):
        _int8_tie_check(dl, w, x, toks, pe, hb, y_got, ep, out_got, eo, wts[toks], ys, tol)
        return
    assert ep.max() <= tol, ep.max()
    assert eo.max() <= tol, eo.max()


def _int8_tie_check(dl, w, x, toks, pe, hb, y_got, ep, out_got, eo, wts, ys, tol):
    """Int8 path: where the exact h of a pair lies within float rounding of a quantisation
    tie, the GPU (deciding on its fp32 h) and the oracle (on its fp64 h) may take neighbouring
    codes, and both are correct.  Pairs or tokens over the bound must match the oracle with
    some choice of the neighbouring code at exactly those positions (found on the oracle's
    side); every other code is unique."""
    from tests.gpu_helpers import best_candidate_err, int8_pair_candidates
    k, H, I = w.top_k, w.hidden, w.inter
    qt = (w.qt_gate, w.qt_up, w.qt_down)
    uniq = np.unique(pe)
    mats = {}

    def expert(e):
        if e not in mats:
            j = int(np.searchsorted(uniq, e))
            mats[e] = [oracle.dequant(hb[n][j], q).reshape(r, c) for n, q, r, c in
                       (("gate", qt[0], I, H), ("up", qt[1], I, H), ("down", qt[2], H, I))]
        return mats[e]

    cand = {}

    def pair(i):
        if i not in cand:
            cand[i] = int8_pair_candidates(*expert(int(pe[i])), x[toks[i // k]])
        return cand[i]

    n_fixed = 0
    for i in np.nonzero(ep > tol)[0]:
        y, deltas = pair(i)
        err = best_candidate_err(y_got[i], y, deltas)
        assert err <= tol, ("pair", i, err, len(deltas))
        n_fixed += 1
    for ti in np.nonzero(eo > tol)[0]:
        ps = [ti * k + j for j in range(k)]
        base = sum(wts[ti, j] * pair(p)[0] for j, p in enumerate(ps)) + (ys[ti] if ys is not None else 0.0)
        deltas = [wts[ti, j] * dlt for j, p in enumerate(ps) for dlt in pair(p)[1]]
        err = best_candidate_err(out_got[ti], base, deltas)
        assert err <= tol, ("token", ti, err, len(deltas))
        n_fixed += 1
    _say("  %d rows over the bound matched the oracle with tie codes flipped" % n_fixed)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", ["tiny", "sage_decode", "mtp_window", "flash_next_decode"])
def test_decode_layer_parity(name, fused):
    m = qm()
    _say("decode layer", name, "fused" if fused else "separate calls")
    dl, w = _layer(name)
    from quantized_moe_ffn_amd import layers
    for replay in range(3):
        logits, x = layers.inputs_np(w, seed=0, index=0, replay=replay)
        bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused)
        _check_layer(m, dl, w, logits, x, bufs, 0, TOL_DECODE)
        _check_routing(bufs.routing, logits, w.top_k)


@pytest.mark.parametrize("over", [dict(hidden=256, inter=768, n_experts=3, top_k=3, tokens=5),
                                  dict(hidden=768, inter=256, n_experts=70, top_k=4, tokens=9, qt_down=oracle.Q8_0),
                                  dict(hidden=512, inter=512, n_experts=16, top_k=2, tokens=1, qt_gate=oracle.Q8_0,
                                       qt_up=oracle.Q8_0),
                                  # Q5_K experts (the "Strata v0.1.31" Unsloth bullet): all Q5_K, and Q5_K
                                  # gate/up with Q4_K down, with and without a shared expert
                                  dict(hidden=512, inter=256, n_experts=16, top_k=4, tokens=3, qt_gate=oracle.Q5_K,
                                       qt_up=oracle.Q5_K, qt_down=oracle.Q5_K),
                                  dict(hidden=768, inter=512, n_experts=12, top_k=3, tokens=2, qt_gate=oracle.Q5_K,
                                       qt_up=oracle.Q5_K, shared=True),
                                  dict(hidden=256, inter=512, n_experts=8, top_k=2, tokens=1, qt_down=oracle.Q5_K)])
@pytest.mark.parametrize("fused", [True, False])
def test_decode_ragged_shapes(over, fused):
    m = qm()
    _say("decode ragged", over, fused)
    dl, w = _layer("tiny", **over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=1)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused)
    _check_layer(m, dl, w, logits, x, bufs, 0, TOL_DECODE)


@pytest.mark.parametrize("fused", [True, False])
def test_int8_path_tiny_full(fused):
    m = qm()
    _say("int8 tiny T=96", fused)
    dl, w = _layer("tiny", tokens=96)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=2)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8, fused)
    if not fused:   # the separate calls leave the int8 activations in the caller's buffers
        xq, xd = oracle.quantize_act(x)
        assert np.array_equal(bufs.xq.cpu().numpy(), xq)
        assert np.array_equal(bufs.xd.cpu().numpy(), xd)
    _check_layer(m, dl, w, logits, x, bufs, 1, TOL_INT8)


@pytest.mark.parametrize("name", ["prefill_chunk", "prefill_chunk_q5k"])
def test_int8_prefill_chunk_full(name):
    """The whole 4,096-token Zipf-loaded prompt chunk (32,768 pairs; the hottest expert
    holds nearly every token, so dozens of tiles share its weights) against the oracle:
    every pair's y and every token's output."""
    m = qm()
    _say("int8 prompt chunk T=4096 (all tokens)", name)
    dl, w = _layer(name)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=0)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8)
    _check_routing(bufs.routing, logits, w.top_k)
    counts = bufs.routing.count.cpu().numpy()
    assert counts.max() > 30 * 64            # the load the chunk is built to have
    _check_layer(m, dl, w, logits, x, bufs, 1, TOL_INT8)


@pytest.mark.parametrize("over", [
    dict(hidden=256, inter=768, n_experts=3, top_k=3, tokens=70),                  # odd block count along I
    dict(hidden=768, inter=512, n_experts=40, top_k=4, tokens=130, shared=True),   # shared expert, 3 blocks along H
    dict(hidden=2560, inter=512, n_experts=16, top_k=2, tokens=40),                # 32-token tiles (hidden > 2048)
    dict(hidden=512, inter=256, n_experts=8, top_k=2, tokens=20, qt_down=oracle.Q8_0),  # Q8_0 down: in-register path
    dict(hidden=512, inter=256, n_experts=8, top_k=2, tokens=20, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K,
         qt_down=oracle.Q5_K, shared=True),                                          # Q5_K experts: MFMA GEMMs
    dict(hidden=768, inter=512, n_experts=24, top_k=4, tokens=70, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K,
         shared=True),                                                               # Q5_K gate/up, Q4_K down
    dict(hidden=512, inter=768, n_experts=6, top_k=2, tokens=130, qt_down=oracle.Q5_K),  # Q4_K gate/up, Q5_K down
    dict(hidden=2560, inter=512, n_experts=16, top_k=2, tokens=40, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K,
         qt_down=oracle.Q5_K),                                                       # Q5_K, 32-token tiles
    dict(hidden=768, inter=512, n_experts=10, top_k=3, tokens=24, qt_gate=oracle.Q5_1, qt_up=oracle.Q5_1,
         qt_down=oracle.Q5_1, shared=True),                                          # Q5_1 experts: in-register path
    # past 256 pairs the layer call routes and quantises in one launch and the bucket scan writes
    # the tile list: eight and sixteen keys per lane, shared-expert tiles, a token count not a
    # multiple of four
    dict(hidden=512, inter=256, n_experts=512, top_k=10, tokens=41, shared=True),
    dict(hidden=256, inter=256, n_experts=1024, top_k=4, tokens=83),
])
@pytest.mark.parametrize("fused", [True, False])
def test_int8_ragged_shapes(over, fused):
    m = qm()
    _say("int8 ragged", over, fused)
    dl, w = _layer("tiny", **over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=6)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8, fused)
    _check_layer(m, dl, w, logits, x, bufs, 1, TOL_INT8)


def test_int8_determinism_and_batch_invariance():
    """The int8 path gives the same bits run to run, and a token's output does not depend on
    which other tokens share its experts' tiles."""
    m = qm()
    dl, w = _layer("tiny", tokens=150, n_experts=4)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=7)
    a = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8).y_pair.cpu().numpy()
    b = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8).y_pair.cpu().numpy()
    assert np.array_equal(a, b)
    sub = np.array([3, 77, 149])
    c = _run_layer(m, dl, logits[sub], x[sub], w.top_k, m.MOE_FFN_INT8).y_pair.cpu().numpy()
    k = w.top_k
    rows = (sub[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    assert np.array_equal(c, a[rows])


# --------------------------------------------------------------------------- MOE_FFN_PAIR_BF16

def _pair_bf16_pair(m, dl, logits, x, k, flags):
    """The layer call with and without MOE_FFN_PAIR_BF16 on the same inputs.  The flagged
    call gets a y_pair buffer full of a sentinel, which it must leave alone."""
    ref = _run_layer(m, dl, logits, x, k, flags)
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    bufs = m.LayerBuffers(dl.layer, x.shape[0], k, flags | m.MOE_FFN_PAIR_BF16, device=DEV)
    bufs.y_pair.fill_(7.0)
    m.forward(dl.layer, lg, xt, k, bufs=bufs, flags=flags | m.MOE_FFN_PAIR_BF16)
    m.moe_check_device_errors()
    assert bool((bufs.y_pair == 7.0).all())
    assert torch.equal(bufs.routing.idx, ref.routing.idx) and torch.equal(bufs.routing.pair, ref.routing.pair)
    if ref.y_shared is not None:
        assert torch.equal(bufs.y_shared, ref.y_shared)
    return ref, bufs


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(hidden=768, inter=512, n_experts=40, top_k=4, tokens=130, shared=True)),
    ("tiny", dict(hidden=2560, inter=512, n_experts=16, top_k=2, tokens=40, qt_gate=oracle.Q5_K,
                  qt_up=oracle.Q5_K, qt_down=oracle.Q5_K)),
    ("prefill_chunk", {}),
])
def test_pair_bf16_int8_mfma_is_the_combine_of_rounded_pairs(name, over):
    """On the int8 MFMA GEMMs the flagged layer call's out equals, bit for bit, the fp32
    combine (moe_combine) of the same call's fp32 per-pair outputs rounded to bf16 (nearest
    even) on the host; and out stays within the int8 path's tolerance of the oracle (checked
    with the unflagged call's y_pair, which the existing tests hold to the oracle)."""
    import types
    m = qm()
    _say("pair bf16, int8 MFMA", name, over)
    dl, w = _layer(name, **over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=11)
    ref, bufs = _pair_bf16_pair(m, dl, logits, x, w.top_k, m.MOE_FFN_INT8)
    yb = torch.from_numpy(bf16_rne(ref.y_pair.cpu().numpy())).to(DEV)
    out_ref = torch.empty_like(ref.out)
    m.moe_combine(yb, ref.routing.w, out_ref, ref.y_shared)
    m.moe_check_device_errors()
    assert torch.equal(bufs.out, out_ref)
    # the rounding moves out by at most 2^-8 sum_j |w_j y_j| per element, plus the fp32
    # roundings of the two k + 1 step fmaf chains
    T, k, H = x.shape[0], w.top_k, w.hidden
    wy = (ref.routing.w.double().reshape(T, k, 1) * ref.y_pair.double().reshape(T, k, H)).abs().sum(1)
    mag = wy + (ref.y_shared.double().abs() if ref.y_shared is not None else 0.0)
    bound = wy * 2.0 ** -8 + mag * (k + 2) * 2.0 ** -23
    assert bool(((bufs.out.double() - ref.out.double()).abs() <= bound).all())
    mixed = types.SimpleNamespace(routing=bufs.routing, y_pair=ref.y_pair, y_shared=bufs.y_shared, out=bufs.out)
    _check_layer(m, dl, w, logits, x, mixed, 1, TOL_INT8)


@pytest.mark.parametrize("name,T,flags,over", [
    ("sage_decode", 1, 0, {}),                                         # two-kernel decode layer
    ("flash_next_decode", 2, 0, {}),                                   # with the shared expert
    ("tiny", 16, 1, dict(hidden=512, inter=256, n_experts=8, top_k=2)),   # general decode stages
    ("tiny", 20, 2, dict(hidden=512, inter=256, n_experts=8, top_k=2, qt_down=oracle.Q8_0)),  # int8, no MFMA
])
def test_pair_bf16_leaves_the_fp32_paths_unchanged(name, T, flags, over):
    """Off the MFMA GEMMs the per-pair outputs stay fp32 (in the workspace, or in LDS in the
    two-kernel decode layer): the flagged call gives the same out bits."""
    m = qm()
    _say("pair bf16, fp32 paths", name, T, flags, over)
    dl, w = _layer(name, tokens=T, **over)
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=12)
    ref, bufs = _pair_bf16_pair(m, dl, logits, x, w.top_k, flags)
    assert torch.equal(bufs.out, ref.out)


def test_integer_exact_layer_is_bitwise():
    """Gate weights all 1/8, up row i all (i mod 4), down row o all (o mod 3), x = 1 (H = I = 256):
    g = 32 (so silu(g) = g in fp32), h_i = 8192 (i mod 4), y_o = (o mod 3) * 8192 * 384.  Every
    partial sum is an integer-valued float below 2^24, so the GPU result must equal the closed form
    exactly, whatever the summation order."""
    m = qm()
    H, I = 256, 256
    def rows(n, cols, q_of, d_bits=0x3C00):
        nb = cols // 256
        return np.stack([np.tile(oracle.q4k_pack(d_bits, 0, np.ones(8), np.zeros(8), np.full(256, q_of(r))), nb)
                         for r in range(n)])
    gate = rows(I, H, lambda r: 1, d_bits=0x3000)[None]     # d = 2^-3
    up = rows(I, H, lambda r: r % 4)[None]
    down = rows(H, I, lambda r: r % 3)[None]
    mats = [m.QMatrix(torch.from_numpy(np.ascontiguousarray(a)).to(DEV), m.MOE_Q4_K, c)
            for a, c in ((gate, H), (up, H), (down, I))]
    layer = m.Layer(*mats)
    x = torch.ones((1, H), dtype=torch.float32, device=DEV)
    lg = torch.zeros((1, 1), dtype=torch.float32, device=DEV)
    bufs = m.forward(layer, lg, x, 1, flags=m.MOE_FFN_DECODE)
    m.moe_check_device_errors()
    expect = np.array([(o % 3) * 8192 * 384 for o in range(H)], np.float32)
    assert 2 * 8192 * 384 < 2 ** 24
    assert np.array_equal(bufs.out.cpu().numpy()[0], expect)
    assert np.array_equal(bufs.y_pair.cpu().numpy()[0], expect)


@pytest.mark.parametrize("fused", [True, False])
def test_determinism_and_batch_invariance(fused):
    m = qm()
    dl, w = _layer("mtp_window")
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=3)
    a = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused).out.cpu().numpy()
    b = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused).out.cpu().numpy()
    assert np.array_equal(a, b)
    for t in range(3):
        one = _run_layer(m, dl, logits[t:t + 1], x[t:t + 1], w.top_k, m.MOE_FFN_DECODE, fused).out.cpu().numpy()
        assert np.array_equal(one[0], a[t])


def test_fused_equals_separate_calls_bitwise_for_routing():
    """The fused layer call and the three separate calls select the same experts and weights."""
    m = qm()
    dl, w = _layer("flash_next_decode")
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=5)
    a = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, True)
    b = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, False)
    for f in ("idx", "count", "offset", "pair", "n_active"):
        assert torch.equal(getattr(a.routing, f), getattr(b.routing, f)), f
    assert torch.equal(a.routing.w, b.routing.w)


@pytest.mark.parametrize("T,flags", [(1, 1), (300, 2), (300, 2 | 16)])
def test_graph_replay_matches_eager(T, flags):
    """A captured stack of layers replays correctly, with eager work between replays: the
    two-kernel decode layer, and the int8 path (routing and quantisation in one launch, the
    tile list from the bucket scan), also with the bf16 hand-off of MOE_FFN_PAIR_BF16."""
    m = qm()
    from quantized_moe_ffn_amd import layers
    _say("graph replay T=%d flags=%d" % (T, flags))
    w = synth.Workload(**{**synth.WORKLOADS["sage_decode"].__dict__, "tokens": T})
    stack = [layers.make_layer(w, seed=9, index=l, device=DEV) for l in range(3)]
    ins = [layers.inputs_np(w, seed=9, index=l) for l in range(3)]
    lgs = [torch.from_numpy(a).to(DEV) for a, _ in ins]
    xs = [torch.from_numpy(b).to(DEV) for _, b in ins]
    bufs = [m.LayerBuffers(dl.layer, T, w.top_k, flags, device=DEV) for dl in stack]
    for l in range(3):
        m.forward(stack[l].layer, lgs[l], xs[l], w.top_k, bufs[l], flags=flags)
    torch.cuda.synchronize()
    eager = [b.out.clone() for b in bufs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for l in range(3):
                m.forward(stack[l].layer, lgs[l], xs[l], w.top_k, bufs[l], flags=flags)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for b in bufs:
            b.out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=DEV).sum()   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        float(junk)
        for l in range(3):
            assert torch.equal(bufs[l].out, eager[l]), (rep, l)
    m.moe_check_device_errors()


def test_corrupted_routing_sets_error_word():
    """A routing buffer handed in with an expert id out of range is caught on the device:
    the kernel skips the slot (no out-of-bounds access) and raises the error word."""
    m = qm()
    dl, w = _layer("tiny")
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=4)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE)
    bufs.routing.active[0] = w.n_experts + 5
    xt = torch.from_numpy(x).to(DEV)
    m.moe_expert_ffn_q(dl.layer, bufs.routing, x.shape[0], w.top_k, bufs.y_pair, x=xt, flags=m.MOE_FFN_DECODE,
                       workspace=bufs.ffn_ws)
    with pytest.raises(m.MoeError, match="expert id out of range"):
        m.moe_check_device_errors()
    m.moe_check_device_errors()


def test_sync_debug_reports_the_error_from_the_call_itself():
    """With MOE_SYNC_DEBUG=1 the call that enqueued the faulty work synchronises and
    returns MOE_ERR_DEVICE itself (the error word is read and cleared there)."""
    import os
    m = qm()
    dl, w = _layer("tiny")
    from quantized_moe_ffn_amd import layers
    logits, x = layers.inputs_np(w, seed=4)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE)
    bufs.routing.active[0] = w.n_experts + 5
    xt = torch.from_numpy(x).to(DEV)
    os.environ["MOE_SYNC_DEBUG"] = "1"
    try:
        with pytest.raises(m.MoeError, match=r"moe_expert_ffn_q \(MOE_SYNC_DEBUG\).*expert id out of range"):
            m.moe_expert_ffn_q(dl.layer, bufs.routing, x.shape[0], w.top_k, bufs.y_pair, x=xt,
                               flags=m.MOE_FFN_DECODE, workspace=bufs.ffn_ws)
        m.moe_check_device_errors()                    # already cleared by the call
        ok = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE)   # a good call passes
        assert np.all(np.isfinite(ok.out.cpu().numpy()))
    finally:
        del os.environ["MOE_SYNC_DEBUG"]


def test_combine_shared_scale_and_one_hot():
    m = qm()
    g = np.random.default_rng(500)
    T, k, H = 3, 4, 512
    y = g.standard_normal((T * k, H)).astype(np.float32)
    wts = np.zeros((T, k), np.float32)
    wts[0, 1] = wts[1, 3] = wts[2, 0] = 1.0
    ys = g.standard_normal((T, H)).astype(np.float32)
    sc = np.array([0.5, 1.0, 2.0], np.float32)
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    m.moe_combine(torch.from_numpy(y).to(DEV), torch.from_numpy(wts).to(DEV), out)
    assert np.array_equal(out.cpu().numpy(), y[[1, 7, 8]])
    m.moe_combine(torch.from_numpy(y).to(DEV), torch.from_numpy(wts).to(DEV), out, torch.from_numpy(ys).to(DEV),
                  torch.from_numpy(sc).to(DEV))
    ref = oracle.combine(y.astype(np.float64), wts.astype(np.float64), ys.astype(np.float64), sc.astype(np.float64))
    assert np.abs(out.cpu().numpy() - ref).max() <= 1e-6 * np.abs(ref).max()


def test_combine_vector_and_scalar_paths_agree():
    """16-byte aligned buffers take the 4-wide combine; buffers offset by one float take
    the scalar one; both sum in slot order, then the shared expert, so the bits agree."""
    m = qm()
    g = np.random.default_rng(501)
    T, k, H = 5, 3, 768
    y = torch.from_numpy(g.standard_normal((T * k, H)).astype(np.float32)).to(DEV)
    wts = torch.from_numpy(g.random((T, k)).astype(np.float32)).to(DEV)
    ys = torch.from_numpy(g.standard_normal((T, H)).astype(np.float32)).to(DEV)
    out_a = torch.empty((T, H), dtype=torch.float32, device=DEV)
    m.moe_combine(y, wts, out_a, ys)

    def shifted(t):   # same values, data pointer 4 bytes past a 16-byte boundary
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    out_b = shifted(torch.zeros((T, H), dtype=torch.float32, device=DEV))
    m.moe_combine(shifted(y), wts, out_b, shifted(ys))
    m.moe_check_device_errors()
    assert out_b.data_ptr() % 16 == 4
    assert torch.equal(out_a, out_b)
    ref = oracle.combine(y.cpu().numpy().astype(np.float64), wts.cpu().numpy().astype(np.float64),
                         ys.cpu().numpy().astype(np.float64))
    assert np.abs(out_a.cpu().numpy() - ref).max() <= 1e-6 * np.abs(ref).max()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 1, dict(n_experts=64, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K, qt_down=oracle.Q5_K)),
    ("sage_decode", 5, dict(n_experts=64, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K, qt_down=oracle.Q5_K)),
    ("flash_next_decode", 2, dict(n_experts=64, qt_gate=oracle.Q5_K, qt_up=oracle.Q5_K)),   # Q8_0 down, shared
    ("flash_next_decode", 1, dict(n_experts=64, qt_down=oracle.Q5_K)),                       # Q4_K gate/up
])
def test_q5k_decode_layers(name, T, over, fused):
    """Q5_K experts (the "Strata v0.1.31" Unsloth bullet) at the decode shapes: the
    two-kernel layer streams Q5_K slices (header, fifth-bit bytes, low nibbles);
    the separate calls use the general kernels."""
    m = qm()
    _say("q5k decode", name, T, over, fused)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=21, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=21)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused)
    _check_layer(m, dl, w, logits, x, bufs, 0, TOL_DECODE)
    _check_routing(bufs.routing, logits, w.top_k)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 1, dict(n_experts=64, qt_gate=oracle.Q8_0, qt_up=oracle.Q8_0)),
    ("sage_decode", 3, dict(n_experts=64, qt_gate=oracle.Q8_0, qt_up=oracle.Q8_0, qt_down=oracle.Q8_0)),
    ("flash_next_decode", 1, dict(n_experts=64, qt_gate=oracle.Q8_0, qt_up=oracle.Q8_0)),   # Q8_0 down, shared
    ("flash_next_decode", 6, dict(n_experts=64, qt_gate=oracle.Q8_0, qt_up=oracle.Q8_0, qt_down=oracle.Q5_K)),
])
def test_q8_gateup_decode_layers(name, T, over, fused):
    """Q8_0 gate/up experts (the Q8_0 of the "Strata v0.1.31" Unsloth bullet, here
    on the gate and up projections too): the two-kernel layer gives each lane one
    34-byte block of a row (odd blocks start 2 bytes past a dword); the shared
    expert's 4-token groups run at 6 tokens."""
    m = qm()
    _say("q8_0 gate/up decode", name, T, over, fused)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=23, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=23)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused)
    _check_layer(m, dl, w, logits, x, bufs, 0, TOL_DECODE)
    _check_routing(bufs.routing, logits, w.top_k)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over", [
    ("sage_decode", 1, dict(n_experts=64, qt_gate=oracle.Q5_1, qt_up=oracle.Q5_1, qt_down=oracle.Q5_1)),
    ("sage_decode", 4, dict(n_experts=64, qt_gate=oracle.Q5_1, qt_up=oracle.Q5_1)),                 # Q4_K down
    ("flash_next_decode", 1, dict(n_experts=64, qt_gate=oracle.Q5_1, qt_up=oracle.Q5_1)),           # Q8_0 down, shared
    ("flash_next_decode", 5, dict(n_experts=64, qt_down=oracle.Q5_1)),                              # Q4_K gate/up
    ("tiny", 3, dict(hidden=256, inter=256, qt_gate=oracle.Q5_1, qt_up=oracle.Q5_1, qt_down=oracle.Q5_1,
                     shared=True)),
])
def test_q51_decode_layers(name, T, over, fused):
    """Q5_1 experts (a format of the "Strata v0.1.31" Unsloth bullet): the two-kernel
    layer gives each lane one 24-byte block (fifth bits moved to bit 4 of each
    byte four at a time); the separate calls use the general kernels."""
    m = qm()
    _say("q5_1 decode", name, T, over, fused)
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=25, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=25)
    bufs = _run_layer(m, dl, logits, x, w.top_k, m.MOE_FFN_DECODE, fused)
    _check_layer(m, dl, w, logits, x, bufs, 0, TOL_DECODE)
    _check_routing(bufs.routing, logits, w.top_k)
