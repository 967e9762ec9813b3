"""moe_forward_router, the layer from the activations and the router matrix in
one call, through the C ABI.

Against moe_router_logits followed by moe_forward on the same inputs: the same
kernels run in both, so the logits, every routing result and every output agree
bit for bit (two or three calls in a row on one workspace, other inputs each
time).  Against the oracle: the layer on the GPU's own logits (the top-k
decision taken in one precision, as in the router tests) within the decode
path's 2e-3 normwise bound.
"""
import numpy as np
import pytest

import oracle
from quantized_moe_ffn_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _router_w(E, H, seed):
    g = np.random.default_rng((seed, 0x52))
    return (g.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _buffers(m, dl, T, k, flags):
    b = m.LayerBuffers(dl.layer, T, k, flags, device=DEV)
    for t in (b.y_pair, b.out) + ((b.y_shared,) if b.y_shared is not None else ()):
        t.fill_(float("nan"))
    return b


def _results(b, logits):
    r = b.routing
    res = {"logits": logits, "idx": r.idx, "w": r.w, "count": r.count, "offset": r.offset, "pair": r.pair,
           "n_active": r.n_active, "out": b.out, "y_pair": b.y_pair}
    if b.y_shared is not None:
        res["y_shared"] = b.y_shared
    out = {n: t.cpu().numpy() for n, t in res.items()}
    n_act = int(out["n_active"][0])
    out["active"] = r.active.cpu().numpy()[:n_act]
    return out


@pytest.mark.parametrize("name,flags,Ts", [
    ("sage_decode", 1, (1, 3, 1)),          # two-kernel decode path
    ("flash_next_decode", 1, (1, 2)),       # shared expert, Q8_0 down, five-wave rows (H = 2560)
    ("sage_decode_q5k", 1, (2,)),           # Q5_K experts
    ("sage_decode", 2, (40,)),              # int8 path (router MFMA kernel above 16 tokens)
])
def test_forward_router_equals_router_then_forward(name, flags, Ts):
    m = _qm()
    from quantized_moe_ffn_amd import layers
    w0 = synth.WORKLOADS[name]
    dl = layers.make_layer(w0, seed=43, index=0, device=DEV)
    E, H, k = w0.n_experts, w0.hidden, w0.top_k
    W = torch.from_numpy(_router_w(E, H, 43)).to(DEV)
    ws = torch.empty(m.moe_forward_workspace_bytes(dl.layer, max(Ts), k, flags), dtype=torch.uint8, device=DEV)
    for i, T in enumerate(Ts):
        print("forward_router", name, "flags", flags, "T", T, flush=True)
        w = synth.Workload(**{**w0.__dict__, "tokens": T})
        _, x = layers.inputs_np(w, seed=43, index=0, replay=i)
        xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)

        b1 = _buffers(m, dl, T, k, flags)
        lg1 = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
        m.moe_forward_router(dl.layer, xt, W, lg1, k, b1.routing, b1.y_pair, b1.out, ws, b1.y_shared, flags=flags)
        m.moe_check_device_errors()
        got = _results(b1, lg1)

        b2 = _buffers(m, dl, T, k, flags)
        lg2 = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
        m.moe_router_logits(xt, W, lg2)
        m.moe_forward(dl.layer, lg2, xt, k, b2.routing, b2.y_pair, b2.out, b2.y_shared, flags=flags,
                      workspace=b2.fwd_ws)
        m.moe_check_device_errors()
        ref = _results(b2, lg2)
        for n in ref:
            assert np.array_equal(_bits(got[n]), _bits(ref[n])), (n, T)
        assert np.all(np.isfinite(got["out"]))


def test_forward_router_matches_oracle_on_its_logits():
    m = _qm()
    from quantized_moe_ffn_amd import layers
    w = synth.Workload(**{**synth.WORKLOADS["sage_decode"].__dict__, "tokens": 2})
    dl = layers.make_layer(w, seed=44, index=0, device=DEV)
    E, H, k, T = w.n_experts, w.hidden, w.top_k, w.tokens
    Wn = _router_w(E, H, 44)
    _, x = layers.inputs_np(w, seed=44, index=0)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    b = _buffers(m, dl, T, k, m.MOE_FFN_DECODE)
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(m.moe_forward_workspace_bytes(dl.layer, T, k, m.MOE_FFN_DECODE), dtype=torch.uint8,
                     device=DEV)
    m.moe_forward_router(dl.layer, xt, torch.from_numpy(Wn).to(DEV), lg, k, b.routing, b.y_pair, b.out, ws,
                         flags=m.MOE_FFN_DECODE)
    m.moe_check_device_errors()
    logits = lg.cpu().numpy()
    # the logits against the oracle's projection (fp32 summation bound, as the router tests)
    ref_lg = oracle.router_logits(x, Wn)
    scale = np.abs(x.astype(np.float64)) @ np.abs(Wn.astype(np.float64)).T
    u = 2.0 ** -24
    assert np.all(np.abs(logits.astype(np.float64) - ref_lg) <= H * u / (1 - H * u) * scale)
    banks = {n: t.cpu().numpy() for n, t in dl.banks.items()}
    ref = oracle.moe_layer(logits, x, banks["gate"], banks["up"], banks["down"], (w.qt_gate, w.qt_up, w.qt_down), k)
    assert np.array_equal(b.routing.idx.cpu().numpy(), ref["idx"])
    out = b.out.cpu().numpy().astype(np.float64)
    err = (np.abs(out - ref["out"]).max(axis=1) / np.abs(ref["out"]).max(axis=1)).max()
    print("forward_router vs oracle: normwise %.2e" % err, flush=True)
    assert err <= 2e-3


def test_forward_router_rejects_a_short_workspace_before_any_device_call():
    m = _qm()
    from quantized_moe_ffn_amd import layers
    w = synth.WORKLOADS["sage_decode"]
    dl = layers.make_layer(w, seed=45, index=0, device=DEV)
    b = _buffers(m, dl, 1, w.top_k, m.MOE_FFN_DECODE)
    xt = torch.zeros((1, w.hidden), dtype=torch.float32, device=DEV)
    W = torch.zeros((w.n_experts, w.hidden), dtype=torch.float32, device=DEV)
    lg = torch.zeros((1, w.n_experts), dtype=torch.float32, device=DEV)
    short = torch.zeros(128, dtype=torch.uint8, device=DEV)
    with pytest.raises(m.MoeError, match="forward workspace"):
        m.moe_forward_router(dl.layer, xt, W, lg, w.top_k, b.routing, b.y_pair, b.out, short,
                             flags=m.MOE_FFN_DECODE)
