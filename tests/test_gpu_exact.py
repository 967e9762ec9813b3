"""Bitwise pins of the timed kernels: layers whose every intermediate value is exact.

The two-kernel decode layer and the int8 MFMA GEMMs decode the block formats with
code of their own (per-lane 16-byte slices with masked scale words and the 1/16
folded into the high-nibble scale; 3-bit scale limbs and an fp16 hi/lo min term),
not with the dequantization hook's helpers.  Here the weights carry varied 6-bit
scales and mins (high bits set in sub-blocks 4..7), power-of-two d and dmin, and
activations chosen so that every product and every partial sum, in any order, is a
multiple of one power of two below 2^24 of it (asserted on the host): then fp32
and int32 evaluate them exactly, silu(g) = g for g >= 17, and the results must
equal the closed form bit for bit.  ("Strata v0.1.31" release notes, Unsloth
UD-Q4_K_XL bullet: the GPU dequantizers match the reference bit for bit and the
dot products agree within float rounding.)

- Decode (moe_forward, the two-kernel layer), at the Sage-like and Flash-Next-like
  shapes: gate/up exact through h (read from the layer's workspace) with Q4_K or
  Q5_K experts; down and the combine exact through y_pair and out with Q4_K, Q5_K
  or Q8_0 down experts (equal top logits give weights of exactly 1/k).
- Int8 path (the grouped MFMA GEMMs): gate/up exact through the int8 codes and
  scales of h; down exact through y_pair, with h built so that its per-256 scales
  are powers of two.
"""
import numpy as np
import pytest

import oracle
from quantized_moe_ffn_amd import synth

from tests.gpu_helpers import TOL_DECODE, normwise_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"
Q4K, Q5K, Q80 = oracle.Q4_K, oracle.Q5_K, oracle.Q8_0
F16 = {0: 0x3C00, -2: 0x3400, -3: 0x3000, -4: 0x2C00, -5: 0x2800}   # 2^e as fp16 bits


def qm():
    import quantized_moe_ffn_amd as m
    m.load_library()
    return m


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- exact matrices

def rand_blocks(g, qt, n, d_e, dmin_e):
    """n blocks of random fields (uniform 6-bit scales and mins, quants; the packing is a
    bijection so random bytes give them) with d = 2^d_e and dmin = 2^dmin_e."""
    nb = oracle.BLOCK_BYTES[qt]
    b = g.integers(0, 256, size=(n, nb), dtype=np.uint8)
    if qt == Q80:
        b[:, 2:] = g.integers(-127, 128, size=(n, 32)).astype(np.int8).view(np.uint8)
        b[:, 0:2] = np.array([F16[d_e]], np.uint16).view(np.uint8)
    else:
        b[:, 0:2] = np.array([F16[d_e]], np.uint16).view(np.uint8)
        b[:, 2:4] = np.array([F16[dmin_e]], np.uint16).view(np.uint8)
    return b


def rand_matrix(g, qt, rows, cols, d_e, dmin_e):
    nbr = cols // oracle.BLOCK_WEIGHTS[qt]
    return rand_blocks(g, qt, rows * nbr, d_e, dmin_e).reshape(rows, -1)


def dense(mat, qt, cols):
    return oracle.dequant(mat, qt).reshape(mat.shape[0], cols)


def q4k_row_single(cols, col, v, d_bits=0x3C00):
    """A Q4_K row whose only nonzero weight is v (0..15) at column `col` (sc = 1, m = 0)."""
    nb = cols // 256
    row = np.zeros((nb, 144), np.uint8)
    zero = oracle.q4k_pack(d_bits, 0, np.ones(8), np.zeros(8), np.zeros(256))
    row[:] = zero
    q = np.zeros(256)
    q[col % 256] = v
    row[col // 256] = oracle.q4k_pack(d_bits, 0, np.ones(8), np.zeros(8), q)
    return row.reshape(-1)


def q4k_uniform_rows(rows, cols, d_bits):
    """Every weight d (quants 1, sc 1, m 0)."""
    blk = oracle.q4k_pack(d_bits, 0, np.ones(8), np.zeros(8), np.ones(256))
    return np.tile(blk, (rows, cols // 256))


def exact_bound(W, x, unit):
    """Sum of |W_ij x_j| over each row, in units of `unit`: every partial sum of the row's
    products, in any order, is a multiple of unit and at most this in magnitude."""
    return (np.abs(W) @ np.abs(x)).max() / unit


def assert_exact(W, x, unit):
    b = exact_bound(W, x, unit)
    assert b < 2 ** 24, b
    prods = W * x[None, :]
    assert np.all(np.mod(prods / unit, 1.0) == 0.0)


# --------------------------------------------------------------------------- device layers

class Bank:
    """Device banks of E experts, zero except for the experts filled in."""

    def __init__(self, m, E, H, I, qg, qd, shared):
        self.m, self.E, self.H, self.I, self.qg, self.qd = m, E, H, I, qg, qd
        rb = lambda qt, cols: cols // oracle.BLOCK_WEIGHTS[qt] * oracle.BLOCK_BYTES[qt]
        self.t = {
            "gate": torch.zeros((E, I, rb(qg, H)), dtype=torch.uint8, device=DEV),
            "up": torch.zeros((E, I, rb(qg, H)), dtype=torch.uint8, device=DEV),
            "down": torch.zeros((E, H, rb(qd, I)), dtype=torch.uint8, device=DEV),
        }
        if shared:
            for n, src in (("sh_gate", "gate"), ("sh_up", "up"), ("sh_down", "down")):
                self.t[n] = torch.zeros((1,) + tuple(self.t[src].shape[1:]), dtype=torch.uint8, device=DEV)
        mats = {n: m.QMatrix(t, qd if n.endswith("down") else qg, I if n.endswith("down") else H)
                for n, t in self.t.items()}
        sh = (mats["sh_gate"], mats["sh_up"], mats["sh_down"]) if shared else None
        self.layer = m.Layer(mats["gate"], mats["up"], mats["down"], sh)

    def put(self, name, e, arr):
        self.t[name][e].copy_(torch.from_numpy(np.ascontiguousarray(arr)))


SHAPES = {
    # name: H, I, E, k, shared
    "sage": (2048, 512, 256, 8, False),
    "flash_next": (2560, 512, 512, 10, True),
}


def equal_top_logits(g, E, k):
    """Logits with k experts at 1.0 and the rest at 0.0: the top-k are those experts in
    ascending order, each with routing weight exactly 1/k."""
    sel = np.sort(g.choice(E, k, replace=False))
    lg = np.zeros((1, E), np.float32)
    lg[0, sel] = 1.0
    return sel, lg


def run_forward(m, bank, lg, x, k, flags):
    lgt = torch.from_numpy(lg).to(DEV)
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    bufs = m.LayerBuffers(bank.layer, x.shape[0], k, flags, device=DEV)
    bufs.fwd_ws.zero_()
    m.moe_forward(bank.layer, lgt, xt, k, bufs.routing, bufs.y_pair, bufs.out, bufs.y_shared, flags=flags,
                  workspace=bufs.fwd_ws)
    m.moe_check_device_errors()
    return bufs


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# --------------------------------------------------------------------------- decode: gate/up

@pytest.mark.parametrize("shape,qg", [("sage", Q4K), ("flash_next", Q4K), ("sage", Q5K)])
def test_decode_gateup_exact(shape, qg):
    """Gate and up with random 6-bit scales/mins, d = 2^-2 (Q5_K 2^-3), dmin = 2^-4; x in
    {0, 1, 2}.  g and u are exact, g >= 17, so the two-kernel layer's h must be exactly
    fp32(g * u) for every slot (and the shared expert)."""
    m = qm()
    H, I, E, k, shared = SHAPES[shape]
    _say("decode gate/up exact", shape, qg)
    g = np.random.default_rng(700 + H + qg)
    d_e = -3 if qg == Q5K else -2
    bank = Bank(m, E, H, I, qg, Q4K, shared)
    sel, lg = equal_top_logits(g, E, k)
    x = g.integers(0, 3, size=H).astype(np.float32)
    experts = [(e, "gate", "up", "down", e) for e in sel] + ([(0, "sh_gate", "sh_up", "sh_down", -1)] if shared
                                                             else [])
    want = []
    for e, gn, un, dn, tag in experts:
        Wg = rand_matrix(g, qg, I, H, d_e, -4)
        Wu = rand_matrix(g, qg, I, H, d_e, -4)
        Dg, Du = dense(Wg, qg, H), dense(Wu, qg, H)
        for D in (Dg, Du):
            assert_exact(D, x.astype(np.float64), 2.0 ** -4)
        gv, uv = Dg @ x, Du @ x
        assert gv.min() >= 17.0, gv.min()
        bank.put(gn, e, Wg.reshape(I, -1))
        bank.put(un, e, Wu.reshape(I, -1))
        bank.put(dn, e, rand_matrix(g, Q4K, H, I, -2, -4))
        want.append(np.float32(gv * uv))          # fp64 product exact (< 2^53), rounded once
    bufs = run_forward(m, bank, lg, x[None], k, m.MOE_FFN_DECODE)
    assert np.array_equal(bufs.routing.idx.cpu().numpy()[0], sel)
    assert np.all(bufs.routing.w.cpu().numpy() == np.float32(1.0 / k))
    off = -(-m.moe_route_workspace_bytes(1, E, k) // 256) * 256       # h starts the FFN part of the workspace
    h = bufs.fwd_ws[off: off + (k + (1 if shared else 0)) * I * 4].view(torch.float32).cpu().numpy()
    h = h.reshape(-1, I)
    for j in range(len(want)):
        assert np.array_equal(bits(h[j]), bits(want[j])), (j, np.nonzero(h[j] != want[j])[0][:5])


# --------------------------------------------------------------------------- decode: down and combine

@pytest.mark.parametrize("shape,qd", [("sage", Q4K), ("sage", Q5K), ("flash_next", Q80), ("flash_next", Q4K)])
def test_decode_down_and_combine_exact(shape, qd):
    """g = 64 exactly (uniform gate, x = +-1 on half the columns summing to 2^9), u in
    {-1, 0, 1} (one nonzero weight per up row), so h = 64 u.  Down rows with random
    6-bit scales/mins, d = 2^-2 (Q5_K 2^-3), dmin = 2^-4, or Q8_0 with d = 2^-2: every
    y_pair value and the combine (weights 1/k, shared expert weight 1) are exact."""
    m = qm()
    H, I, E, k, shared = SHAPES[shape]
    _say("decode down exact", shape, qd)
    g = np.random.default_rng(800 + H + qd)
    bank = Bank(m, E, H, I, Q4K, qd, shared)
    sel, lg = equal_top_logits(g, E, k)
    half = 1024                                                          # x nonzero on columns 0..1023
    x = np.zeros(H, np.float32)
    signs = np.ones(half, np.float32)
    signs[g.permutation(half)[: half // 4]] = -1.0                      # sum = half/2
    x[:half] = signs
    assert x.sum() == half // 2
    d_bits_gate = F16[int(6 - np.log2(half // 2))]                      # g = (half/2) * d = 64
    Wg = q4k_uniform_rows(I, H, d_bits_gate)
    assert np.all(dense(Wg, Q4K, H) @ x == 64.0)
    d_e = -3 if qd == Q5K else -2
    experts = [(e, "gate", "up", "down") for e in sel] + ([(0, "sh_gate", "sh_up", "sh_down")] if shared else [])
    ys = []
    for e, gn, un, dn in experts:
        cols = g.integers(0, half, size=I)
        nz = g.random(I) < 0.25
        Wu = np.stack([q4k_row_single(H, cols[i], 1 if nz[i] else 0) for i in range(I)])
        u = dense(Wu, Q4K, H) @ x
        assert set(np.unique(u)) <= {-1.0, 0.0, 1.0}
        h = 64.0 * u
        Wd = rand_matrix(g, qd, H, I, d_e, -4)
        Dd = dense(Wd, qd, I)
        assert_exact(Dd, h, 64.0 * 2.0 ** -4)
        bank.put(gn, e, Wg)
        bank.put(un, e, Wu)
        bank.put(dn, e, Wd)
        ys.append(Dd @ h)
    out = sum(y / k for y in ys[:k]) + (ys[k] if shared else 0.0)
    exact_out = (k & (k - 1)) == 0          # weights 1/k exact in fp32 only for k a power of two
    if exact_out:
        unit = 64.0 * 2.0 ** -4 / k
        assert np.abs(out).max() / unit < 2 ** 24 and np.all(np.mod(out / unit, 1.0) == 0.0)
    bufs = run_forward(m, bank, lg, x[None], k, m.MOE_FFN_DECODE)
    assert np.array_equal(bufs.routing.idx.cpu().numpy()[0], sel)
    yp = bufs.y_pair.cpu().numpy()
    for j in range(k):
        assert np.array_equal(bits(yp[j]), bits(ys[j])), (j, np.nonzero(yp[j] != np.float32(ys[j]))[0][:5])
    if shared:
        assert np.array_equal(bits(bufs.y_shared.cpu().numpy()[0]), bits(ys[k]))
    if exact_out:
        assert np.array_equal(bits(bufs.out.cpu().numpy()[0]), bits(out))
    else:   # k = 10: weights fl(1/10), the combine's fp32 rounding only
        assert normwise_err(bufs.out.cpu().numpy(), out[None]).max() <= 1e-6


# --------------------------------------------------------------------------- int8 path: MFMA GEMMs

MFMA_CASES = [
    # H, I, E, k, T: 64-token tiles with several tiles and a ragged tail per expert
    dict(H=2048, I=512, E=4, k=2, T=300, qg=Q4K, qd=Q4K),
    # 32-token tiles (few tokens per expert), three blocks along I
    dict(H=1024, I=768, E=16, k=3, T=40, qg=Q4K, qd=Q4K),
    # Q5_K experts (quants enter as q - 16)
    dict(H=2048, I=512, E=4, k=2, T=160, qg=Q5K, qd=Q5K),
]


def _int8_x(g, T, H, p_one=0.25):
    """Activations that quantize exactly: 127 at the first column of every 256-block
    (amax 127: id = 1, d = 1) and the rest in {0, 1}."""
    x = (g.random((T, H)) < p_one).astype(np.float32)
    x[:, ::256] = 127.0
    return x


def _run_int8(m, bank, lg, x, k):
    """The separate calls on the int8 path: route, quantize, expert FFN (the MFMA GEMMs),
    combine.  Returns the buffers and the FFN workspace."""
    T = x.shape[0]
    bufs = m.LayerBuffers(bank.layer, T, k, m.MOE_FFN_INT8, device=DEV)
    bufs.ffn_ws.zero_()
    bufs = m.forward(bank.layer, torch.from_numpy(lg).to(DEV), torch.from_numpy(x).to(DEV), k, bufs,
                     flags=m.MOE_FFN_INT8, fused=False)
    m.moe_check_device_errors()
    return bufs


def _np_quant_rows(h):
    """The activation quantiser in fp32 (numpy), per 256-block of each row."""
    h = np.asarray(h, np.float32)
    R, n = h.shape
    blk = h.reshape(R, n // 256, 256)
    amax = np.abs(blk).max(axis=2)
    idv = np.where(amax > 0, np.float32(127) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    q = np.clip(np.rint((blk * idv[..., None]).astype(np.float32)), -127, 127).astype(np.int8)
    return q.reshape(R, n), (amax / np.float32(127)).astype(np.float32)


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "H%d_I%d_E%d_k%d_T%d_q%d" % (
    c["H"], c["I"], c["E"], c["k"], c["T"], c["qg"]))
def test_mfma_gateup_exact_codes(case):
    """Int8 path, gate/up GEMMs with random 6-bit scales/mins and d, dmin powers of two:
    g and u are exact (the int32 sums and the fp32 block scaling and min term stay below
    2^24 of their unit), g >= 17, so h = fp32(g*u) exactly and its int8 codes and scales
    (the quantiser's rule) must equal the closed form bit for bit."""
    m = qm()
    H, I, E, k, T, qg = case["H"], case["I"], case["E"], case["k"], case["T"], case["qg"]
    _say("mfma gate/up exact", case)
    g = np.random.default_rng(900 + H + I + T)
    d_e = -3 if qg == Q5K else -2
    bank = Bank(m, E, H, I, qg, case["qd"], False)
    x = _int8_x(g, T, H)
    Dg, Du = [], []
    for e in range(E):
        Wg = rand_matrix(g, qg, I, H, d_e, -4)
        Wu = rand_matrix(g, qg, I, H, d_e, -4)
        Dg.append(dense(Wg, qg, H))
        Du.append(dense(Wu, qg, H))
        for D in (Dg[-1], Du[-1]):
            assert exact_bound(D, x.max(axis=0).astype(np.float64), 2.0 ** -4) < 2 ** 24
        bank.put("gate", e, Wg)
        bank.put("up", e, Wu)
        bank.put("down", e, rand_matrix(g, case["qd"], H, I, d_e, -4))
    lg = synth.logits_np(g, T, E)
    bufs = _run_int8(m, bank, lg, x, k)
    assert np.array_equal(bufs.xq.cpu().numpy(), x.astype(np.int8))
    assert np.all(bufs.xd.cpu().numpy() == 1.0)
    idx = bufs.routing.idx.cpu().numpy()
    rows = T * k
    hq = bufs.ffn_ws[: rows * I].cpu().numpy().view(np.int8).reshape(rows, I)
    off = -(-rows * I // 256) * 256
    hd = bufs.ffn_ws[off: off + rows * (I // 256) * 4].view(torch.float32).cpu().numpy().reshape(rows, I // 256)
    xf = x.astype(np.float64)
    for p in range(rows):
        t, e = p // k, idx.reshape(-1)[p]
        gv, uv = Dg[e] @ xf[t], Du[e] @ xf[t]
        assert gv.min() >= 17.0
        q, d = _np_quant_rows(np.float32(gv * uv)[None])
        assert np.array_equal(hq[p], q[0]), (p, np.nonzero(hq[p] != q[0])[0][:5])
        assert np.array_equal(bits(hd[p]), bits(d[0])), p


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "H%d_I%d_E%d_k%d_T%d_q%d" % (
    c["H"], c["I"], c["E"], c["k"], c["T"], c["qd"]))
def test_mfma_down_exact(case):
    """Int8 path, down GEMM with random 6-bit scales/mins.  g = 64 for every row (uniform
    gate; x per 256-block is 127 once and sums to 256), up rows hold one weight, so u is
    127*8 in one row per 256-block of h (its amax: scale 512, a power of two) and small
    elsewhere: the codes of h are exact decisions and y_pair must equal the closed form
    bit for bit."""
    m = qm()
    H, I, E, k, T, qd = case["H"], case["I"], case["E"], case["k"], case["T"], case["qd"]
    _say("mfma down exact", case)
    g = np.random.default_rng(1000 + H + I + T)
    d_e = -3 if qd == Q5K else -2
    bank = Bank(m, E, H, I, Q4K, qd, False)
    nb = H // 256
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        for b in range(nb):
            blk = np.zeros(256, np.float32)
            blk[0] = 127.0
            pos = 1 + g.permutation(255)
            blk[pos[:192]] = 1.0
            blk[pos[192:255]] = -1.0
            x[t, 256 * b: 256 * (b + 1)] = blk
    assert np.all(x.reshape(T, nb, 256).sum(axis=2) == 256)
    d_exp = int(6 - np.log2(256 * nb))                                   # g = 256 * nb * d = 64
    Wg = q4k_uniform_rows(I, H, F16[d_exp])
    Dd, U = [], []
    for e in range(E):
        rows_u = []
        for i in range(I):
            if i % 256 == 7:
                rows_u.append(q4k_row_single(H, 0, 8))                  # u = 127 * 8: the block's amax
            else:
                v = int(g.integers(0, 16)) if g.random() < 0.3 else 0
                rows_u.append(q4k_row_single(H, 1 + int(g.integers(0, 255)), v))
        Wu = np.stack(rows_u)
        Wd = rand_matrix(g, qd, H, I, d_e, -4)
        bank.put("gate", e, Wg)
        bank.put("up", e, Wu)
        bank.put("down", e, Wd)
        Dd.append(dense(Wd, qd, I))
        U.append(dense(Wu, Q4K, H))
    lg = synth.logits_np(g, T, E)
    bufs = _run_int8(m, bank, lg, x, k)
    idx = bufs.routing.idx.cpu().numpy().reshape(-1)
    yp = bufs.y_pair.cpu().numpy()
    xf = x.astype(np.float64)
    assert np.all(dense(Wg, Q4K, H) @ xf.T == 64.0)
    for p in range(T * k):
        t, e = p // k, idx[p]
        h = 64.0 * (U[e] @ xf[t])
        q, d = _np_quant_rows(np.float32(h)[None])
        assert np.all(d == 512.0)
        hhat = q[0].astype(np.float64) * 512.0
        assert_exact(Dd[e], hhat, 512.0 * 2.0 ** -4)
        y = Dd[e] @ hhat
        assert np.array_equal(bits(yp[p]), bits(y)), (p, np.nonzero(yp[p] != np.float32(y))[0][:5])
    # and the combine of exact pairs stays within fp32 rounding of the fp64 sum
    w = bufs.routing.w.cpu().numpy().astype(np.float64)
    ref = (yp.reshape(T, k, H).astype(np.float64) * w[..., None]).sum(axis=1)
    assert normwise_err(bufs.out.cpu().numpy(), ref).max() <= 1e-6
