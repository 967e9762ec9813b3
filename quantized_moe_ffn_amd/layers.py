"""Synthetic MoE layers resident in device memory (plumbing for tests and benchmarks).

Banks are drawn with ``synth`` (host numpy for small layers, device torch for
large ones) and wrapped in the binding's ``Layer`` descriptors.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import QMatrix, Layer
from . import synth

TENSOR_IDS = {"gate": 1, "up": 2, "down": 3, "sh_gate": 4, "sh_up": 5, "sh_down": 6,
              "logits": 7, "x": 8}


@dataclass
class DeviceLayer:
    layer: Layer
    banks: dict          # name -> torch uint8 tensor [E][rows][row_bytes]
    workload: synth.Workload
    seed: int
    index: int


def _bank(w: synth.Workload, name: str, seed: int, index: int, device, host_limit: int):
    E = 1 if name.startswith("sh_") else w.n_experts
    if name.endswith("gate"):
        qt, rows, cols = w.qt_gate, w.inter, w.hidden
    elif name.endswith("up"):
        qt, rows, cols = w.qt_up, w.inter, w.hidden
    else:
        qt, rows, cols = w.qt_down, w.hidden, w.inter
    nbytes = E * rows * synth.row_bytes(qt, cols)
    parts = (seed, index, TENSOR_IDS[name])
    if nbytes <= host_limit:
        import torch
        arr = synth.bank_np(synth.rng(*parts), qt, E, rows, cols)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device), qt, cols
    return synth.bank_torch(synth.torch_gen(device, *parts), qt, E, rows, cols, device), qt, cols


def make_layer(w: synth.Workload, seed: int = 0, index: int = 0, device="cuda",
               host_limit: int = 64 << 20) -> DeviceLayer:
    names = ["gate", "up", "down"] + (["sh_gate", "sh_up", "sh_down"] if w.shared else [])
    banks, mats = {}, {}
    for n in names:
        t, qt, cols = _bank(w, n, seed, index, device, host_limit)
        banks[n] = t
        mats[n] = QMatrix(t, qt, cols)
    shared = (mats["sh_gate"], mats["sh_up"], mats["sh_down"]) if w.shared else None
    return DeviceLayer(Layer(mats["gate"], mats["up"], mats["down"], shared), banks, w, seed, index)


def inputs_np(w: synth.Workload, seed: int = 0, index: int = 0, replay: int = 0, T: int | None = None):
    """Router logits [T][E] and activations [T][H] (fp32, host) for one layer and replay."""
    T = w.tokens if T is None else T
    g = synth.rng(seed, index, replay, TENSOR_IDS["logits"])
    logits = synth.logits_np(g, T, w.n_experts, w.zipf_s)
    x = synth.activations_np(synth.rng(seed, index, replay, TENSOR_IDS["x"]), T, w.hidden)
    return logits, x
