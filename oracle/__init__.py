"""CPU oracle for the routed MoE FFN over GGUF block-quantized experts.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``quantized_moe_ffn_amd``) never imports it, and the two share no code.

This module is argument marshalling (numpy <-> ctypes) around ``moe_oracle.c``,
which holds every step of the arithmetic.  The C file is built with gcc into
``liboracle.so`` next to it (no fast-math, no FP contraction).

Every function states the passage of the pages it follows; the pages name the
method (routed top-k MoE, Q4_K / Q8_0 experts, SiLU-gated FFN, shared expert)
without printing its equations, and the readings taken are listed at the top of
``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q5_1 = 7
BLOCK_WEIGHTS = {Q4_K: 256, Q5_K: 256, Q8_0: 32, Q5_1: 32}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q5_1: 24}

_lib = None


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (OpenMP, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.orc_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_fp16_to_f64.restype = ctypes.c_double
    lib.orc_q4k_unpack.argtypes = [P, P, P, P, P, P]
    lib.orc_q4k_pack.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P, P, P]
    lib.orc_q4k_dequant.argtypes = [P, i64, P]
    lib.orc_q80_dequant.argtypes = [P, i64, P]
    lib.orc_q5k_unpack.argtypes = [P, P, P, P, P, P]
    lib.orc_q5k_pack.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P, P, P]
    lib.orc_q5k_dequant.argtypes = [P, i64, P]
    lib.orc_q51_unpack.argtypes = [P, P, P, P]
    lib.orc_q51_pack.argtypes = [ctypes.c_uint16, ctypes.c_uint16, P, P]
    lib.orc_q51_dequant.argtypes = [P, i64, P]
    lib.orc_route_topk.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.orc_router_logits.argtypes = [P, i32, i32, P, i32, P]
    lib.orc_bucket.argtypes = [P, i32, i32, i32, P, P, P, P, P]
    lib.orc_quant_act_f32.argtypes = [P, i32, i32, P, P]
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_expert_ffn.argtypes = [P, P, P, i32, i32, i32, i64, i64, i64, i32, i32, i32,
                                   P, P, i32, P, P]
    lib.orc_combine.argtypes = [P, P, P, P, i32, i32, i32, P]
    lib.orc_combine_ep.argtypes = [P, P, P, P, P, P, i32, i32, i32, P]
    lib.orc_shared_gate.argtypes = [P, i32, i32, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def threads() -> int:
    """Number of OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (a single-thread baseline
    runs the same code with n = 1)."""
    _load().orc_set_threads(int(n))


def fp16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact fp64 values (scale fields of both formats)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_fp16_to_f64(int(v)) for v in b], dtype=np.float64)


def q4k_unpack(block) -> dict:
    """One 144-byte Q4_K super-block -> its fields (d, dmin bits; sc[8]; m[8]; q[256])."""
    lib = _load()
    blk = np.ascontiguousarray(np.frombuffer(bytes(block), dtype=np.uint8))
    assert blk.size == 144
    d = np.zeros(1, np.uint16)
    dm = np.zeros(1, np.uint16)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib.orc_q4k_unpack(_ptr(blk), _ptr(d), _ptr(dm), _ptr(sc), _ptr(m), _ptr(q))
    return {"d_bits": int(d[0]), "dmin_bits": int(dm[0]), "sc": sc, "m": m, "q": q}


def q4k_pack(d_bits, dmin_bits, sc, m, q) -> np.ndarray:
    """Fields -> one 144-byte Q4_K super-block (inverse of ``q4k_unpack``)."""
    lib = _load()
    sc = np.ascontiguousarray(sc, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.int32)
    out = np.zeros(144, np.uint8)
    lib.orc_q4k_pack(int(d_bits), int(dmin_bits), _ptr(sc), _ptr(m), _ptr(q), _ptr(out))
    return out


def q4k_dequant(blocks) -> np.ndarray:
    """Q4_K blocks (uint8, any shape ending in a multiple of 144 bytes) -> fp64 weights."""
    lib = _load()
    b = np.ascontiguousarray(blocks, dtype=np.uint8).ravel()
    assert b.size % 144 == 0
    n = b.size // 144
    out = np.zeros(n * 256, np.float64)
    lib.orc_q4k_dequant(_ptr(b), n, _ptr(out))
    return out


def q80_dequant(blocks) -> np.ndarray:
    """Q8_0 blocks (uint8, a multiple of 34 bytes) -> fp64 weights."""
    lib = _load()
    b = np.ascontiguousarray(blocks, dtype=np.uint8).ravel()
    assert b.size % 34 == 0
    n = b.size // 34
    out = np.zeros(n * 32, np.float64)
    lib.orc_q80_dequant(_ptr(b), n, _ptr(out))
    return out


def q5k_unpack(block) -> dict:
    """One 176-byte Q5_K super-block -> its fields (d, dmin bits; sc[8]; m[8]; q[256] in 0..31)."""
    lib = _load()
    blk = np.ascontiguousarray(np.frombuffer(bytes(block), dtype=np.uint8))
    assert blk.size == 176
    d = np.zeros(1, np.uint16)
    dm = np.zeros(1, np.uint16)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q = np.zeros(256, np.int32)
    lib.orc_q5k_unpack(_ptr(blk), _ptr(d), _ptr(dm), _ptr(sc), _ptr(m), _ptr(q))
    return {"d_bits": int(d[0]), "dmin_bits": int(dm[0]), "sc": sc, "m": m, "q": q}


def q5k_pack(d_bits, dmin_bits, sc, m, q) -> np.ndarray:
    """Fields -> one 176-byte Q5_K super-block (inverse of ``q5k_unpack``)."""
    lib = _load()
    sc = np.ascontiguousarray(sc, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.int32)
    out = np.zeros(176, np.uint8)
    lib.orc_q5k_pack(int(d_bits), int(dmin_bits), _ptr(sc), _ptr(m), _ptr(q), _ptr(out))
    return out


def q5k_dequant(blocks) -> np.ndarray:
    """Q5_K blocks (uint8, a multiple of 176 bytes) -> fp64 weights."""
    lib = _load()
    b = np.ascontiguousarray(blocks, dtype=np.uint8).ravel()
    assert b.size % 176 == 0
    n = b.size // 176
    out = np.zeros(n * 256, np.float64)
    lib.orc_q5k_dequant(_ptr(b), n, _ptr(out))
    return out


def q51_unpack(block) -> dict:
    """One 24-byte Q5_1 block -> its fields (d and m bits; q[32] in 0..31)."""
    lib = _load()
    blk = np.ascontiguousarray(np.asarray(block, dtype=np.uint8).reshape(-1))
    assert blk.size == 24
    d = np.zeros(1, np.uint16)
    m = np.zeros(1, np.uint16)
    q = np.zeros(32, np.int32)
    lib.orc_q51_unpack(_ptr(blk), _ptr(d), _ptr(m), _ptr(q))
    return {"d_bits": int(d[0]), "m_bits": int(m[0]), "q": q}


def q51_pack(d_bits, m_bits, q) -> np.ndarray:
    """Fields -> one 24-byte Q5_1 block (inverse of ``q51_unpack``)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int32)
    assert q.shape == (32,)
    out = np.zeros(24, np.uint8)
    lib.orc_q51_pack(int(d_bits), int(m_bits), _ptr(q), _ptr(out))
    return out


def q51_dequant(blocks) -> np.ndarray:
    """Q5_1 blocks (uint8, a multiple of 24 bytes) -> fp64 weights."""
    lib = _load()
    b = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint8).reshape(-1))
    assert b.size % 24 == 0
    n = b.size // 24
    out = np.zeros(32 * n, np.float64)
    lib.orc_q51_dequant(_ptr(b), n, _ptr(out))
    return out


def dequant(blocks, qtype: int) -> np.ndarray:
    return {Q4_K: q4k_dequant, Q5_K: q5k_dequant, Q8_0: q80_dequant, Q5_1: q51_dequant}[qtype](blocks)


def router_logits(x, w_router) -> np.ndarray:
    """Router projection (R-router in moe_oracle.c; "Strata - the details",
    "How it works": routers are a GPU stage): fp32 x [T][H] and fp32 W [E][H]
    -> fp64 logits [T][E], each a sequential fp64 sum over h."""
    lib = _load()
    xa = np.ascontiguousarray(x, dtype=np.float32)
    wa = np.ascontiguousarray(w_router, dtype=np.float32)
    T, H = xa.shape
    E, H2 = wa.shape
    assert H == H2
    out = np.empty((T, E), dtype=np.float64)
    lib.orc_router_logits(_ptr(xa), T, H, _ptr(wa), E, _ptr(out))
    return out


def route_topk(logits, k: int, renorm: bool = True):
    """Top-k expert selection + routing weights, fp64 weights (readings R-topk, R-softmax)."""
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    assert lg.ndim == 2 and np.all(np.isfinite(lg)), "the oracle takes finite logits only"
    T, E = lg.shape
    assert 1 <= k <= E
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    lib.orc_route_topk(_ptr(lg), T, E, k, int(bool(renorm)), _ptr(idx), _ptr(w))
    return idx, w


def bucket(idx, E: int) -> dict:
    """Per-expert bucketing of (token, slot) pairs, stable in pair id."""
    lib = _load()
    ix = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = ix.shape
    assert ix.min() >= 0 and ix.max() < E
    count = np.zeros(E, np.int32)
    offset = np.zeros(E + 1, np.int32)
    pair = np.zeros(T * k, np.int32)
    active = np.zeros(max(1, min(E, T * k)), np.int32)
    na = np.zeros(1, np.int32)
    lib.orc_bucket(_ptr(ix), T, k, E, _ptr(count), _ptr(offset), _ptr(pair), _ptr(active), _ptr(na))
    return {"count": count, "offset": offset, "pair": pair,
            "active": active[: int(na[0])].copy(), "n_active": int(na[0])}


def quantize_act(x):
    """Per-token, per-256-block int8 activation quantisation evaluated in IEEE fp32."""
    lib = _load()
    xa = np.ascontiguousarray(x, dtype=np.float32)
    T, H = xa.shape
    assert H % 256 == 0
    xq = np.zeros((T, H), np.int8)
    xd = np.zeros((T, H // 256), np.float32)
    lib.orc_quant_act_f32(_ptr(xa), T, H, _ptr(xq), _ptr(xd))
    return xq, xd


def silu(g: float) -> float:
    return float(_load().orc_silu(float(g)))


def expert_ffn(gate, up, down, qtypes, H: int, I: int, pair_expert, pair_token, x,
               mode: int = 0) -> np.ndarray:
    """Expert FFN for each (expert, token) pair, fp64 (reading R-ffn).

    gate/up: uint8 [n_experts, I, row_bytes(H)]; down: uint8 [n_experts, H, row_bytes(I)].
    qtypes = (gate, up, down) qtype ids.  mode 0 = fp activations; mode 1 = the
    int8 path's quantisation points (x per token, h per pair, 256-wide blocks).
    Returns y [n_pairs, H] fp64.
    """
    lib = _load()
    g = np.ascontiguousarray(gate, dtype=np.uint8)
    u = np.ascontiguousarray(up, dtype=np.uint8)
    d = np.ascontiguousarray(down, dtype=np.uint8)
    qg, qu, qd = qtypes
    assert g.shape[1] == I and u.shape[1] == I and d.shape[1] == H
    assert g.shape[2] == H // BLOCK_WEIGHTS[qg] * BLOCK_BYTES[qg]
    assert u.shape[2] == H // BLOCK_WEIGHTS[qu] * BLOCK_BYTES[qu]
    assert d.shape[2] == I // BLOCK_WEIGHTS[qd] * BLOCK_BYTES[qd]
    pe = np.ascontiguousarray(pair_expert, dtype=np.int32)
    pt = np.ascontiguousarray(pair_token, dtype=np.int32)
    xa = np.ascontiguousarray(x, dtype=np.float32)
    assert xa.shape[1] == H
    assert pe.size == 0 or (pe.min() >= 0 and pe.max() < g.shape[0])
    assert pt.size == 0 or (pt.min() >= 0 and pt.max() < xa.shape[0])
    n = pe.size
    y = np.zeros((n, H), np.float64)
    if n:
        lib.orc_expert_ffn(_ptr(g), _ptr(u), _ptr(d), qg, qu, qd,
                           g.shape[1] * g.shape[2], u.shape[1] * u.shape[2], d.shape[1] * d.shape[2],
                           H, I, n, _ptr(pe), _ptr(pt), int(mode), _ptr(xa), _ptr(y))
    return y


def combine(y_pair, w, y_shared=None, shared_scale=None, shared_gate=None, residual=None) -> np.ndarray:
    """Routing-weighted combine in slot order, plus the shared expert (reading R-combine)
    scaled by shared_scale[t] * shared_gate[t], plus the residual (reading R-epilogue)."""
    lib = _load()
    wa = np.ascontiguousarray(w, dtype=np.float64)
    T, k = wa.shape
    yp = np.ascontiguousarray(y_pair, dtype=np.float64)
    H = yp.shape[1]
    assert yp.shape[0] == T * k
    f64 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float64)
    ys, ss, sg, rs = f64(y_shared), f64(shared_scale), f64(shared_gate), f64(residual)
    assert rs is None or rs.shape == (T, H)
    assert sg is None or sg.shape == (T,)
    out = np.zeros((T, H), np.float64)
    p = lambda a: None if a is None else _ptr(a)
    lib.orc_combine_ep(_ptr(yp), _ptr(wa), p(ys), p(ss), p(sg), p(rs), T, k, H, _ptr(out))
    return out


def shared_gate(x, g) -> np.ndarray:
    """Sigmoid gate of the shared expert per token, 1/(1 + exp(-(g . x_t))), fp64 (reading R-epilogue)."""
    lib = _load()
    xa = np.ascontiguousarray(x, dtype=np.float32)
    ga = np.ascontiguousarray(g, dtype=np.float32).reshape(-1)
    T, H = xa.shape
    assert ga.size == H
    out = np.zeros(T, np.float64)
    lib.orc_shared_gate(_ptr(xa), T, H, _ptr(ga), _ptr(out))
    return out


def moe_layer(logits, x, gate, up, down, qtypes, k: int, renorm: bool = True, mode: int = 0,
              shared=None, shared_qtypes=None, shared_scale=None, shared_gate_w=None, residual=None) -> dict:
    """The whole hot path for one layer: route -> bucket -> expert FFN -> combine.

    ``gate/up/down`` hold every expert the routing may touch, indexed by expert id.
    ``shared`` = (gate, up, down) arrays with a leading dimension of 1, or None.
    ``shared_gate_w`` [H] gates the shared expert by a sigmoid of its dot with the
    token; ``residual`` [T][H] is added to the output (reading R-epilogue).
    """
    logits = np.asarray(logits, dtype=np.float32)
    x = np.asarray(x, dtype=np.float32)
    T, E = logits.shape
    H = x.shape[1]
    I = gate.shape[1]
    idx, w = route_topk(logits, k, renorm)
    b = bucket(idx, E)
    pair_expert = idx.reshape(-1)
    pair_token = np.repeat(np.arange(T, dtype=np.int32), k)
    y_pair = expert_ffn(gate, up, down, qtypes, H, I, pair_expert, pair_token, x, mode)
    y_sh = None
    if shared is not None:
        sg, su, sd = shared
        y_sh = expert_ffn(sg, su, sd, shared_qtypes or qtypes, H, I,
                          np.zeros(T, np.int32), np.arange(T, dtype=np.int32), x, mode)
    sgv = None if shared_gate_w is None else shared_gate(x, shared_gate_w)
    out = combine(y_pair, w, y_sh, shared_scale, sgv, residual)
    res = {"idx": idx, "w": w, "y_pair": y_pair, "y_shared": y_sh, "out": out, "shared_gate": sgv}
    res.update(b)
    return res


# ----------------------------------------------------------------------------- int8-path decisions

# Error model of an fp32 evaluation of the int8 path's h (reading R-quant with the
# int8 path's quantisation points): g and u exact in int32 per 256-block, scaled and
# summed over the blocks in fp32, so their error is bounded by G_EPS * sum |w x|;
# silu and the product add a few ulps of h.  An h code is a float-rounding decision
# when its scaled value h*127/amax lies within that error of a rounding tie.
G_EPS = 2.0 ** -20
H_REL = 2.0 ** -20


def int8_pair_candidates(Wg, Wu, Wd, x_row):
    """One pair on the int8 path from dense fp64 matrices (Wg, Wu [I][H], Wd [H][I],
    rows decoded by ``dequant``): y as defined (x quantized per 256-block in fp32, h in
    fp64 requantized per 256-block), plus the change of y for each h position whose code
    is a float-rounding decision (its scaled value within the fp32 error bound of h of a
    tie): the other neighbouring code there.  Every result in {y + any subset of the
    deltas} is a correct int8-path output; outside these positions the codes are unique."""
    xq, xd = quantize_act(np.asarray(x_row, np.float32)[None])
    xh = np.repeat(xd[0].astype(np.float64), 256) * xq[0].astype(np.float64)
    g = Wg @ xh
    u = Wu @ xh
    with np.errstate(over="ignore"):
        sg = g / (1.0 + np.exp(-g))
    h = sg * u
    dg = G_EPS * (np.abs(Wg) @ np.abs(xh))
    du = G_EPS * (np.abs(Wu) @ np.abs(xh))
    dh = 1.1 * dg * np.abs(u) + np.abs(sg) * du + H_REL * np.abs(h)
    hh = np.zeros_like(h)
    deltas = []
    for b in range(len(h) // 256):
        sl = slice(256 * b, 256 * (b + 1))
        seg = h[sl]
        amax = np.abs(seg).max()
        if amax == 0.0:
            continue
        r = seg * (127.0 / amax)
        c = np.clip(np.rint(r), -127, 127)
        d = amax / 127.0
        hh[sl] = d * c
        rel_amax = dh[sl][np.argmax(np.abs(seg))] / amax
        band = dh[sl] * (127.0 / amax) + np.abs(r) * (rel_amax + 2.0 ** -22)
        fl = np.floor(r)
        near = np.abs((r - fl) - 0.5) <= band
        for i in np.nonzero(near)[0]:
            other = fl[i] if c[i] == fl[i] + 1 else fl[i] + 1
            if abs(other) <= 127:
                deltas.append(Wd[:, 256 * b + i] * (d * (other - c[i])))
    return Wd @ hh, deltas


def best_candidate_err(got, y, deltas, max_flips=12) -> float:
    """Smallest normwise error (max |got - ref| / max |ref|) of ``got`` over the candidate
    set {y + any subset of deltas} of ``int8_pair_candidates``."""
    import itertools
    got = np.asarray(got, np.float64)
    if len(deltas) > max_flips:
        raise ValueError("%d ambiguous h codes in one pair" % len(deltas))
    best = np.inf
    for n in range(len(deltas) + 1):
        for sub in itertools.combinations(range(len(deltas)), n):
            ref = y + sum((deltas[i] for i in sub), np.zeros_like(y))
            den = np.abs(ref).max()
            best = min(best, float(np.abs(got - ref).max() / (den if den > 0 else 1.0)))
    return best
