"""GPU parity of the layer epilogue through the C ABI: the sigmoid-gated shared
expert and the residual add (reading R-epilogue of the oracle; the pages keep
shared experts and the gated-residual weights on the GPU, "Strata - the
details", "How it works").

On the two-kernel decode layer the gate is computed by the routing workgroup
and the residual is added in the down kernel's combine; the separate stages use
a gate kernel and the combine kernel.  Checked against the oracle at the decode
and int8 shapes, plus two exact identities: the gate values are the same bits
as moe_shared_gate's, so moe_forward_ep equals moe_forward with those values as
shared_scale followed by one fp32 add of the residual, bit for bit; and an
in-place residual update (out = residual) gives the same bits as a separate one.
"""
import numpy as np
import pytest

import oracle
from quantized_moe_ffn_amd import synth

from tests.gpu_helpers import TOL_DECODE, TOL_INT8, bf16_rne, normwise_err, oracle_pairs, oracle_shared

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _say(*a):
    print(*a, flush=True)


def _case(name, T, over, seed):
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS[name].__dict__, **over, "tokens": T})
    dl = layers.make_layer(w, seed=seed, index=0, device=DEV)
    logits, x = layers.inputs_np(w, seed=seed)
    g = np.random.default_rng((seed, 0x6A7E))
    gate_w = (g.standard_normal(w.hidden) / np.sqrt(w.hidden)).astype(np.float32)
    resid = g.standard_normal((T, w.hidden)).astype(np.float32)
    return w, dl, logits, x, gate_w, resid


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = [
    ("flash_next_decode", 1, dict(n_experts=64), 0),                   # two-kernel decode, shared expert
    ("flash_next_decode", 3, dict(n_experts=64), 0),
    ("tiny", 5, dict(shared=True), 0),
    ("tiny", 24, dict(shared=True), 1),                                  # int8 path (MFMA GEMMs)
    ("tiny", 20, dict(shared=True, qt_down=oracle.Q8_0), 1),            # int8 path, general kernels
]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over,mode", CASES)
def test_epilogue_matches_oracle(name, T, over, mode, fused):
    """The residual is scaled to each token's output magnitude (the oracle's MoE part), so
    a residual dropped, doubled or added to the wrong token fails the comparison."""
    m = qm()
    _say("epilogue", name, T, over, "int8" if mode else "decode", fused)
    w, dl, logits, x, gate_w, resid = _case(name, T, over, seed=31)
    k = w.top_k
    idx, wts = oracle.route_topk(logits, k)
    toks = np.arange(T)
    y_ref, hb = oracle_pairs(dl, idx.reshape(-1), np.repeat(toks, k), x, mode)
    ys = oracle_shared(dl, hb, toks, x, mode)
    sg = oracle.shared_gate(x, gate_w)
    moe_ref = oracle.combine(y_ref, wts, ys, None, sg)
    resid = (resid * np.abs(moe_ref).max(axis=1, keepdims=True)).astype(np.float32)
    out_ref = oracle.combine(y_ref, wts, ys, None, sg, resid)
    flags = m.MOE_FFN_INT8 if mode else m.MOE_FFN_DECODE
    bufs = m.forward(dl.layer, _dev(logits), _dev(x), k, flags=flags, fused=fused,
                     residual=_dev(resid), shared_gate=_dev(gate_w))
    m.moe_check_device_errors()
    assert np.array_equal(bufs.routing.idx.cpu().numpy(), idx)
    tol = TOL_INT8 if mode else TOL_DECODE
    got = bufs.out.cpu().numpy()
    eo = normwise_err(got, out_ref)
    # without the residual the comparison must fail: it is of the output's own size
    e_nores = normwise_err(got, moe_ref)
    _say("  out err %.3e (against the MoE part alone: %.3e)" % (eo.max(), e_nores.min()))
    assert eo.max() <= tol
    assert e_nores.min() > 100 * tol


def test_shared_gate_kernel_vs_oracle():
    m = qm()
    g = np.random.default_rng(5)
    for T, H in [(1, 2560), (7, 256), (33, 2048), (5, 3584)]:
        x = g.standard_normal((T, H)).astype(np.float32)
        gw = (g.standard_normal(H) * (3.0 / np.sqrt(H))).astype(np.float32)
        s = torch.empty(T, dtype=torch.float32, device=DEV)
        m.moe_shared_gate(_dev(x), _dev(gw), s)
        m.moe_check_device_errors()
        ref = oracle.shared_gate(x, gw)
        assert np.abs(s.cpu().numpy() - ref).max() <= 2e-6, (T, H)
    # saturation: exp overflow on the way to 0, underflow on the way to 1
    x = np.zeros((2, 256), np.float32)
    x[0, 3], x[1, 3] = 200.0, -200.0
    gw = np.zeros(256, np.float32)
    gw[3] = 1.0
    s = torch.empty(2, dtype=torch.float32, device=DEV)
    m.moe_shared_gate(_dev(x), _dev(gw), s)
    assert s.cpu().numpy().tolist() == [1.0, 0.0]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name,T,over,mode", [CASES[1], CASES[3]])
def test_epilogue_is_gate_as_scale_plus_residual_bitwise(name, T, over, mode, fused):
    """forward_ep(gate, residual) == forward(shared_scale = moe_shared_gate values) + residual,
    bit for bit, on the fused and the separate paths; and the in-place update (residual
    passed as out) gives the same bits."""
    m = qm()
    _say("epilogue identities", name, T, mode, fused)
    w, dl, logits, x, gate_w, resid = _case(name, T, over, seed=32)
    flags = m.MOE_FFN_INT8 if mode else m.MOE_FFN_DECODE
    lg, xt, gw, rt = _dev(logits), _dev(x), _dev(gate_w), _dev(resid)
    s = torch.empty(T, dtype=torch.float32, device=DEV)
    m.moe_shared_gate(xt, gw, s)
    plain = m.forward(dl.layer, lg, xt, w.top_k, flags=flags, fused=fused, shared_scale=s)
    expect = plain.out + rt
    ep = m.forward(dl.layer, lg, xt, w.top_k, flags=flags, fused=fused, residual=rt, shared_gate=gw)
    m.moe_check_device_errors()
    assert torch.equal(ep.out, expect)
    # in place: the output buffer holds the residual on entry
    bufs = m.LayerBuffers(dl.layer, T, w.top_k, flags, device=DEV)
    bufs.out.copy_(rt)
    m.forward(dl.layer, lg, xt, w.top_k, bufs=bufs, flags=flags, fused=fused, residual=bufs.out, shared_gate=gw)
    m.moe_check_device_errors()
    assert torch.equal(bufs.out, expect)


def test_epilogue_on_the_bf16_hand_off_bitwise():
    """With MOE_FFN_PAIR_BF16 on the int8 MFMA GEMMs (shared expert, gate and residual), the
    layer call's out equals moe_combine_ep of the unflagged call's y_pair rounded to bf16 on the
    host, with the same gate values and residual, bit for bit."""
    m = qm()
    name, T, over, _ = CASES[3]
    _say("epilogue on the bf16 hand-off", name, T)
    w, dl, logits, x, gate_w, resid = _case(name, T, over, seed=33)
    lg, xt, gw, rt = _dev(logits), _dev(x), _dev(gate_w), _dev(resid)
    plain = m.forward(dl.layer, lg, xt, w.top_k, flags=m.MOE_FFN_INT8)
    s = torch.empty(T, dtype=torch.float32, device=DEV)
    m.moe_shared_gate(xt, gw, s)
    expect = torch.empty_like(plain.out)
    m.moe_combine_ep(_dev(bf16_rne(plain.y_pair.cpu().numpy())), plain.routing.w, expect, plain.y_shared, None, s, rt)
    flags = m.MOE_FFN_INT8 | m.MOE_FFN_PAIR_BF16
    bufs = m.LayerBuffers(dl.layer, T, w.top_k, flags, device=DEV)
    m.forward(dl.layer, lg, xt, w.top_k, bufs=bufs, flags=flags, residual=rt, shared_gate=gw)
    m.moe_check_device_errors()
    assert torch.equal(bufs.y_shared, plain.y_shared)
    assert torch.equal(bufs.out, expect)
