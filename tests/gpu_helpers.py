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


# The int8 path's float-rounding code decisions: the oracle's candidate set
# (oracle.int8_pair_candidates) and the best match against it.
int8_pair_candidates = oracle.int8_pair_candidates
best_candidate_err = oracle.best_candidate_err


def bf16_rne(a):
    """fp32 -> bf16 rounded to nearest, ties to even, widened back to fp32 (finite values)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)
