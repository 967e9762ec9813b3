"""Helpers shared by the GPU parity tests: oracle evaluation of device-resident
layers (only the experts a routing touches are copied back) and the error
metrics the tests grade with."""
from __future__ import annotations

import numpy as np

import oracle

# Tolerances: FFN outputs within a max relative error of 2e-3 of an fp64
# reference on the fp-activation (decode) path and 5e-3 on the int8-activation
# path, read normwise per output row: max_i |y_i - r_i| / max_i |r_i|.  Top-k
# indices and dequantized weights exact; routing weights within 1e-6.
TOL_DECODE = 2e-3
TOL_INT8 = 5e-3
TOL_W = 1e-6


def normwise_err(got, ref) -> np.ndarray:
    got = np.asarray(got, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    den = np.abs(ref).max(axis=1)
    den[den == 0] = 1.0
    return np.abs(got - ref).max(axis=1) / den


def host_banks(dl, experts):
    """Copies the listed experts of each routed bank (and the shared one) to the host."""
    import torch
    ex = torch.as_tensor(np.asarray(experts, np.int64), device=dl.banks["gate"].device)
    out = {n: dl.banks[n].index_select(0, ex).cpu().numpy() for n in ("gate", "up", "down")}
    if dl.workload.shared:
        for n in ("sh_gate", "sh_up", "sh_down"):
            out[n] = dl.banks[n].cpu().numpy()
    return out


def oracle_pairs(dl, pair_expert, pair_token, x, mode):
    """Oracle y for (expert, token) pairs of a device layer, copying back only the touched experts."""
    w = dl.workload
    pe = np.asarray(pair_expert, np.int64)
    uniq, inv = np.unique(pe, return_inverse=True)
    hb = host_banks(dl, uniq)
    qt = (w.qt_gate, w.qt_up, w.qt_down)
    y = oracle.expert_ffn(hb["gate"], hb["up"], hb["down"], qt, w.hidden, w.inter, inv.astype(np.int32),
                          np.asarray(pair_token, np.int32), x, mode)
    return y, hb


def oracle_shared(dl, hb, tokens, x, mode):
    w = dl.workload
    qt = (w.qt_gate, w.qt_up, w.qt_down)
    return oracle.expert_ffn(hb["sh_gate"], hb["sh_up"], hb["sh_down"], qt, w.hidden, w.inter,
                             np.zeros(len(tokens), np.int32), np.asarray(tokens, np.int32), x, mode)


# Error model of the int8 path's h on the GPU, for deciding which h codes are float-rounding
# decisions.  g and u are int32-exact per 256-block, scaled and summed over the blocks in
# fp32 (plus the fp16 hi/lo min term at about 2^-22): their error is bounded by
# G_EPS * sum |w x|.  silu and the product add a few ulps of h.  A code is a rounding
# decision when its scaled value h*127/amax lies within that error of a tie.
G_EPS = 2.0 ** -20
H_REL = 2.0 ** -20


def int8_pair_candidates(Wg, Wu, Wd, x_row):
    """One pair on the int8 path, evaluated as the oracle defines it (x quantized per
    256-block in fp32, h in fp64 requantized per 256-block), plus the change of y for each
    h position whose code is a float-rounding decision (its scaled value within the fp32
    error bound of h of a tie): the other neighbouring code there.  Returns
    (y, [delta_y, ...]); every result in {y + sum of any subset of the deltas} is a correct
    int8-path output, and outside these positions the codes are unique."""
    xq, xd = oracle.quantize_act(np.asarray(x_row, np.float32)[None])
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


def best_candidate_err(got, y, deltas, max_flips=12):
    """Smallest normwise error of `got` against the candidate set of int8_pair_candidates."""
    import itertools
    if len(deltas) > max_flips:
        raise AssertionError("%d ambiguous h codes in one pair" % len(deltas))
    best = np.inf
    for n in range(len(deltas) + 1):
        for sub in itertools.combinations(range(len(deltas)), n):
            ref = y + sum((deltas[i] for i in sub), np.zeros_like(y))
            best = min(best, float(normwise_err(got[None], ref[None])[0]))
    return best
