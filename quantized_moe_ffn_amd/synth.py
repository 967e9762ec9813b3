"""Seeded synthetic inputs for the MoE FFN: expert banks, activations, router logits.

This module only draws random numbers with the value laws of the workloads; it
holds none of the method's arithmetic (no unpacking, no dot products, no
routing).  A Q4_K block is 144 random bytes with its two leading fp16 fields
(d, dmin) overwritten: random bytes make every 4-bit quant uniform on 0..15 and
every 6-bit scale and min uniform on 0..63, because the twelve packed scale
bytes and the 128 quant bytes are bijective images of those fields; a Q5_K
block (176 bytes) is drawn the same way, its 32 fifth-bit bytes included, so
every 5-bit quant is uniform on 0..31.  A Q8_0 block is an fp16 scale
followed by 32 int8 values uniform on -127..127.
d, dmin and the Q8_0 scale are fp16(|N(0,1)| * 0.01) (round to nearest even).
A Q5_1 block is 24 random bytes (quants uniform on 0..31) with d =
fp16(|N(0,1)| * 0.01) and offset m = fp16(-|N(0,1)| * 0.16): a block of
weights spread over [min, max] stores m = min and d = (max - min)/31, so m
sits near -16 d.

Host arrays come from numpy's PCG64; large banks are drawn on the device with
torch's generator so that tens of GB never cross PCIe.  The oracle reads back
exactly the bytes it checks, so host and device never need to reproduce each
other's stream.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q5_1 = 7
BLOCK_WEIGHTS = {Q4_K: 256, Q5_K: 256, Q8_0: 32, Q5_1: 32}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q5_1: 24}


def row_bytes(qtype: int, cols: int) -> int:
    return cols // BLOCK_WEIGHTS[qtype] * BLOCK_BYTES[qtype]


def seed_of(*parts: int) -> int:
    """Deterministic 62-bit seed from integers (splitmix-style mixing)."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h ^= (int(p) + 0x9E3779B97F4A7C15 + ((h << 6) & (2**64 - 1)) + (h >> 2)) & (2**64 - 1)
        h = (h * 0xBF58476D1CE4E5B9) & (2**64 - 1)
        h ^= h >> 31
    return h & (2**62 - 1)


# ----------------------------------------------------------------------------- host (numpy)

def rng(*parts: int) -> np.random.Generator:
    return np.random.default_rng(seed_of(*parts))


def _scale_f16(g: np.random.Generator, n: int) -> np.ndarray:
    v = np.abs(g.standard_normal(n, dtype=np.float32)) * np.float32(0.01)
    return v.astype(np.float16)


def q4k_blocks_np(g: np.random.Generator, n_blocks: int, nbytes: int = 144) -> np.ndarray:
    """Q4_K blocks (or, with nbytes = 176, Q5_K blocks: the same leading fp16 pair)."""
    b = g.integers(0, 256, size=(n_blocks, nbytes), dtype=np.uint8)
    b[:, 0:4] = _scale_f16(g, 2 * n_blocks).view(np.uint8).reshape(n_blocks, 4)
    return b


def q80_blocks_np(g: np.random.Generator, n_blocks: int) -> np.ndarray:
    b = np.empty((n_blocks, 34), np.uint8)
    b[:, 0:2] = _scale_f16(g, n_blocks).view(np.uint8).reshape(n_blocks, 2)
    b[:, 2:] = g.integers(-127, 128, size=(n_blocks, 32), dtype=np.int8).view(np.uint8)
    return b


def q51_blocks_np(g: np.random.Generator, n_blocks: int) -> np.ndarray:
    b = g.integers(0, 256, size=(n_blocks, 24), dtype=np.uint8)
    b[:, 0:2] = _scale_f16(g, n_blocks).view(np.uint8).reshape(n_blocks, 2)
    m = (-np.abs(g.standard_normal(n_blocks, dtype=np.float32)) * np.float32(0.16)).astype(np.float16)
    b[:, 2:4] = m.view(np.uint8).reshape(n_blocks, 2)
    return b


def bank_np(g: np.random.Generator, qtype: int, n_experts: int, rows: int, cols: int) -> np.ndarray:
    """[n_experts][rows][row_bytes] uint8."""
    nb = n_experts * rows * (cols // BLOCK_WEIGHTS[qtype])
    if qtype == Q8_0:
        blocks = q80_blocks_np(g, nb)
    elif qtype == Q5_1:
        blocks = q51_blocks_np(g, nb)
    else:
        blocks = q4k_blocks_np(g, nb, BLOCK_BYTES[qtype])
    return blocks.reshape(n_experts, rows, row_bytes(qtype, cols))


def activations_np(g: np.random.Generator, T: int, H: int) -> np.ndarray:
    return g.standard_normal((T, H), dtype=np.float32)


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert logit bias -s*ln(e+1): a Zipf(s) law over expert ranks (rank = e+1)."""
    return (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def logits_np(g: np.random.Generator, T: int, E: int, zipf_s: float = 0.0) -> np.ndarray:
    lg = g.standard_normal((T, E), dtype=np.float32)
    if zipf_s:
        lg = (lg + zipf_bias(E, zipf_s)[None, :]).astype(np.float32)
    return lg


# ----------------------------------------------------------------------------- device (torch)

def torch_gen(device, *parts: int):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(*parts))
    return gen


def bank_torch(gen, qtype: int, n_experts: int, rows: int, cols: int, device):
    """[n_experts][rows][row_bytes] uint8 drawn on ``device``."""
    import torch
    nb = n_experts * rows * (cols // BLOCK_WEIGHTS[qtype])
    bb = BLOCK_BYTES[qtype]
    out = torch.empty((nb, bb), dtype=torch.uint8, device=device)
    step = 1 << 22  # blocks per draw, bounds the temporaries
    for s0 in range(0, nb, step):
        n = min(step, nb - s0)
        sl = out[s0:s0 + n]
        sc = (torch.randn((n, 1 if qtype == Q8_0 else 2), generator=gen, device=device,
                          dtype=torch.float32).abs_() * 0.01).to(torch.float16)
        if qtype == Q5_1:
            sc[:, 1:2] = (torch.randn((n, 1), generator=gen, device=device, dtype=torch.float32).abs_()
                          * -0.16).to(torch.float16)
        if qtype != Q8_0:
            sl.copy_(torch.randint(0, 256, (n, bb), generator=gen, device=device, dtype=torch.uint8))
            sl[:, 0:4] = sc.view(torch.uint8).view(n, 4)
        else:
            sl[:, 0:2] = sc.view(torch.uint8).view(n, 2)
            sl[:, 2:] = torch.randint(-127, 128, (n, 32), generator=gen, device=device,
                                      dtype=torch.int8).view(torch.uint8)
    return out.view(n_experts, rows, row_bytes(qtype, cols))


# ----------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class Workload:
    """One synthetic MoE layer shape with its value laws."""
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    tokens: int
    qt_gate: int = Q4_K
    qt_up: int = Q4_K
    qt_down: int = Q4_K
    shared: bool = False
    zipf_s: float = 0.0
    layers: int = 1
    int8_path: bool = False
    notes: str = field(default="", compare=False)

    def expert_bytes(self) -> int:
        return (self.inter * (row_bytes(self.qt_gate, self.hidden) + row_bytes(self.qt_up, self.hidden))
                + self.hidden * row_bytes(self.qt_down, self.inter))


# Shapes from the pages: Sage-A1.5 (256 experts / top-8, Q4_K down experts) in the
# "Strata-Sage-A1.5-GGUF" card; Flash-Next (512 experts, 10 routed + 1 shared,
# hidden 2,560, 48 layers) in the "Strata: a 125B MoE at 94 tok/s" article; MTP
# verify windows of up to 3 tokens and prompt chunks in "Strata - the details".
WORKLOADS = {
    "tiny": Workload("tiny", 256, 8, 2, 256, 4, notes="all Q4_K, seed 0"),
    "sage_decode": Workload("sage_decode", 2048, 256, 8, 512, 1, layers=40,
                            notes="1 token, Q4_K gate/up/down, 40 distinct layers"),
    "mtp_window": Workload("mtp_window", 2048, 256, 8, 512, 3, layers=40,
                           notes="3 independently routed tokens through the sage_decode layer"),
    "flash_next_decode": Workload("flash_next_decode", 2560, 512, 10, 512, 1, qt_down=Q8_0,
                                  shared=True, layers=48,
                                  notes="10 routed + 1 shared, Q4_K gate/up, Q8_0 down"),
    # Q5_K experts: among the formats of the Unsloth UD-Q4_K_XL files that the
    # "Strata v0.1.31" release notes run natively; the Sage-like layer stands in
    "sage_decode_q5k": Workload("sage_decode_q5k", 2048, 256, 8, 512, 1, qt_gate=Q5_K, qt_up=Q5_K, qt_down=Q5_K,
                                layers=40, notes="the sage_decode layer with Q5_K gate/up/down"),
    "prefill_chunk_q5k": Workload("prefill_chunk_q5k", 2048, 256, 8, 512, 4096, qt_gate=Q5_K, qt_up=Q5_K,
                                  qt_down=Q5_K, zipf_s=1.1, layers=4, int8_path=True,
                                  notes="the prompt chunk with Q5_K gate/up/down"),
    # Q5_1 experts, another format of those files (32-weight blocks, scale and offset)
    "sage_decode_q51": Workload("sage_decode_q51", 2048, 256, 8, 512, 1, qt_gate=Q5_1, qt_up=Q5_1, qt_down=Q5_1,
                                layers=40, notes="the sage_decode layer with Q5_1 gate/up/down"),
    "prefill_chunk": Workload("prefill_chunk", 2048, 256, 8, 512, 4096, zipf_s=1.1, layers=4,
                              int8_path=True,
                              notes="logits N(0,1) - 1.1 ln(e+1); int8 activations"),
}
