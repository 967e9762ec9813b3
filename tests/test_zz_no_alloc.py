"""moe_forward_noalloc (for callers that cannot allocate: code under graph capture,
tight serving loops) against moe_forward with a caller-owned workspace, through
the C ABI.  The same kernels run on the same inputs, so the outputs must agree bit
for bit; two calls in a row, the second smaller, check that the shared static
scratch keeps no state that a later call depends on.  With MOE_FFN_PAIR_BF16 the
per-pair outputs live in the scratch too, and y_pair (filled with NaN) stays
untouched by both calls."""
import numpy as np
import pytest

from quantized_moe_ffn_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def _qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _outputs(m, dl, w, logits, x, flags, noalloc):
    T, k = x.shape[0], w.top_k
    lg = torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    b = m.LayerBuffers(dl.layer, T, k, flags, device=DEV)
    for t in (b.y_pair, b.out) + ((b.y_shared,) if b.y_shared is not None else ()):
        t.fill_(float("nan"))
    if noalloc:
        m.moe_forward_noalloc(dl.layer, lg, xt, k, b.routing, b.y_pair, b.out, b.y_shared, flags=flags)
    else:
        m.moe_forward(dl.layer, lg, xt, k, b.routing, b.y_pair, b.out, b.y_shared, flags=flags, workspace=b.fwd_ws)
    m.moe_check_device_errors()
    res = {"out": b.out, "y_pair": b.y_pair, "idx": b.routing.idx, "w": b.routing.w, "pair": b.routing.pair}
    if b.y_shared is not None:
        res["y_shared"] = b.y_shared
    return {n: t.cpu().numpy() for n, t in res.items()}


@pytest.mark.parametrize("name,flags,t1,t2", [
    ("sage_decode", 1, 8, 2),            # two-kernel decode layer
    ("flash_next_decode", 1, 3, 1),      # with the shared expert, Q8_0 down
    ("sage_decode", 2, 300, 40),         # int8 MFMA path
    ("sage_decode", 2 | 16, 200, 40),    # MOE_FFN_PAIR_BF16: bf16 per-pair outputs in the scratch
    ("flash_next_decode", 1 | 16, 3, 1), # the flag on the decode layer: y_pair left untouched
])
def test_noalloc_equals_forward_bitwise(name, flags, t1, t2):
    m = _qm()
    from quantized_moe_ffn_amd import layers
    w0 = synth.WORKLOADS[name]
    dl = layers.make_layer(w0, seed=41, index=0, device=DEV)
    for i, T in enumerate((t1, t2)):
        w = synth.Workload(**{**w0.__dict__, "tokens": T})
        print("noalloc", name, "flags", flags, "T", T, flush=True)
        logits, x = layers.inputs_np(w, seed=41, index=0, replay=i)
        a = _outputs(m, dl, w, logits, x, flags, noalloc=True)
        b = _outputs(m, dl, w, logits, x, flags, noalloc=False)
        for n in b:
            assert np.array_equal(a[n].view(np.uint32) if a[n].dtype == np.float32 else a[n],
                                  b[n].view(np.uint32) if b[n].dtype == np.float32 else b[n]), (n, T)
        assert np.all(np.isfinite(a["out"]))


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    m = _qm()
    from quantized_moe_ffn_amd import layers
    w = synth.WORKLOADS["sage_decode"]
    dl = layers.make_layer(w, seed=42, index=0, device=DEV)
    T = 4096
    need = m.moe_forward_workspace_bytes(dl.layer, T, w.top_k, m.MOE_FFN_INT8)
    assert need > m.MOE_NOALLOC_SCRATCH_BYTES
    b = m.LayerBuffers(dl.layer, T, w.top_k, m.MOE_FFN_INT8, device=DEV)
    lg = torch.zeros((T, w.n_experts), dtype=torch.float32, device=DEV)
    xt = torch.zeros((T, w.hidden), dtype=torch.float32, device=DEV)
    with pytest.raises(m.MoeError, match="static scratch"):
        m.moe_forward_noalloc(dl.layer, lg, xt, w.top_k, b.routing, b.y_pair, b.out, flags=m.MOE_FFN_INT8)
