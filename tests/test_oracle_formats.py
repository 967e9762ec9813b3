"""Pins for the oracle's block-format decoding (CPU only).

The pages name Q4_K and Q8_0 as expert formats ("Strata-Sage-A1.5-GGUF" card,
round-1 flag table; "Strata v0.1.31" release notes, Unsloth UD-Q4_K_XL bullet:
GPU dequantizers bit-exact with the reference dequantizer) but print no byte
layout and no worked block.  These tests pin the oracle to things other than
itself: numpy's own binary16 conversion over all 65,536 patterns, codec round
trips (the layout is a bijection), and hand-worked blocks whose values follow
in closed form from the fields they were built from.
"""
import numpy as np
import pytest

import oracle
from tests.golden import load_block


def test_fp16_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.fp16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_q4k_unpack_pack_roundtrip_random_bytes():
    g = np.random.default_rng(1)
    for _ in range(300):
        blk = g.integers(0, 256, 144, dtype=np.uint8)
        f = oracle.q4k_unpack(blk.tobytes())
        assert f["sc"].min() >= 0 and f["sc"].max() <= 63
        assert f["m"].min() >= 0 and f["m"].max() <= 63
        assert f["q"].min() >= 0 and f["q"].max() <= 15
        back = oracle.q4k_pack(f["d_bits"], f["dmin_bits"], f["sc"], f["m"], f["q"])
        assert np.array_equal(back, blk)


def test_q4k_pack_unpack_roundtrip_random_fields():
    g = np.random.default_rng(2)
    for _ in range(300):
        d, dm = (int(v) for v in g.integers(0, 65536, 2))
        sc = g.integers(0, 64, 8)
        m = g.integers(0, 64, 8)
        q = g.integers(0, 16, 256)
        f = oracle.q4k_unpack(oracle.q4k_pack(d, dm, sc, m, q).tobytes())
        assert f["d_bits"] == d and f["dmin_bits"] == dm
        assert np.array_equal(f["sc"], sc) and np.array_equal(f["m"], m) and np.array_equal(f["q"], q)


def test_q4k_block_a_closed_form():
    blk = load_block("q4k_block_a.txt")
    f = oracle.q4k_unpack(blk.tobytes())
    assert np.array_equal(f["sc"], np.arange(1, 9)) and np.array_equal(f["m"], np.arange(8))
    assert np.array_equal(f["q"], np.arange(256) % 16)
    w = oracle.q4k_dequant(blk)
    i = np.arange(256)
    j = i // 32
    expect = (j + 1) * (i % 16) - 0.5 * j
    assert np.array_equal(w, expect)
    assert (w[0], w[33], w[100], w[255]) == (0.0, 1.5, 14.5, 116.5)
    assert w.sum() == 8192.0


def test_q4k_block_b_high_bits():
    blk = load_block("q4k_block_b.txt")
    f = oracle.q4k_unpack(blk.tobytes())
    assert np.all(f["sc"] == 63) and np.all(f["m"] == 63) and np.all(f["q"] == 15)
    w = oracle.q4k_dequant(blk)
    assert np.all(w == 3717.0 / 4096.0)


def test_q4k_block_c_subnormal_scale():
    blk = load_block("q4k_block_c.txt")
    w = oracle.q4k_dequant(blk)
    assert np.all(w == 2.0 ** -24)


def test_q4k_single_field_sensitivity():
    """Each of the 16 scale/min fields moves only its own 32 weights (indexing pin)."""
    base_sc = np.full(8, 10)
    base_m = np.full(8, 3)
    q = np.full(256, 7)
    ref = oracle.q4k_dequant(oracle.q4k_pack(0x3C00, 0x3C00, base_sc, base_m, q))
    for j in range(8):
        sc = base_sc.copy()
        sc[j] = 50
        w = oracle.q4k_dequant(oracle.q4k_pack(0x3C00, 0x3C00, sc, base_m, q))
        diff = np.nonzero(w != ref)[0]
        assert np.array_equal(diff, np.arange(32 * j, 32 * j + 32))
        assert np.all(w[diff] - ref[diff] == 40 * 7)
        m = base_m.copy()
        m[j] = 60
        w = oracle.q4k_dequant(oracle.q4k_pack(0x3C00, 0x3C00, base_sc, m, q))
        diff = np.nonzero(w != ref)[0]
        assert np.array_equal(diff, np.arange(32 * j, 32 * j + 32))
        assert np.all(ref[diff] - w[diff] == 57)


def test_q80_block_closed_form():
    blk = load_block("q80_block.txt")
    w = oracle.q80_dequant(blk)
    assert np.array_equal(w, (np.arange(32) - 16) / 4.0)
    assert w.sum() == -4.0


def test_q80_random_vs_numpy_views():
    """Q8_0 value = fp16 scale x int8, checked through numpy's own dtype views."""
    g = np.random.default_rng(3)
    blk = g.integers(0, 256, (50, 34), dtype=np.uint8)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64)
    q = blk[:, 2:].copy().view(np.int8).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        expect = (d * q).ravel()
    got = oracle.q80_dequant(blk)
    finite = np.isfinite(expect)
    assert np.array_equal(got[finite], expect[finite])


@pytest.mark.parametrize("nb", [1, 3])
def test_q4k_dequant_exact_value(nb):
    """The oracle's fp64 weight equals d*sc*q - dmin*m evaluated exactly with fractions."""
    from fractions import Fraction
    g = np.random.default_rng(4)
    blk = g.integers(0, 256, (nb, 144), dtype=np.uint8)
    # keep scales finite
    blk[:, 1] &= 0x7B
    blk[:, 3] &= 0x7B
    w = oracle.q4k_dequant(blk)
    for b in range(nb):
        f = oracle.q4k_unpack(blk[b].tobytes())
        d = Fraction(float(np.uint16(f["d_bits"]).view(np.float16)))
        dm = Fraction(float(np.uint16(f["dmin_bits"]).view(np.float16)))
        for i in range(0, 256, 7):
            j = i // 32
            exact = d * int(f["sc"][j]) * int(f["q"][i]) - dm * int(f["m"][j])
            assert Fraction(w[256 * b + i]) == exact


def test_q4k_block_e_distinct_fields():
    blk = load_block("q4k_block_e.txt")
    sc = np.array([1, 2, 3, 4, 17, 34, 51, 60])
    m = np.array([5, 6, 7, 8, 33, 49, 20, 63])
    f = oracle.q4k_unpack(blk.tobytes())
    assert np.array_equal(f["sc"], sc) and np.array_equal(f["m"], m)
    q = np.zeros(256, np.int64)
    for c in range(4):
        for l in range(32):
            q[64 * c + l] = (c + l) % 16
            q[64 * c + 32 + l] = (3 * c + 2 * l + 1) % 16
    assert np.array_equal(f["q"], q)
    j = np.arange(256) // 32
    assert np.array_equal(oracle.q4k_dequant(blk), (sc[j] * q - m[j]).astype(np.float64))
    # and the packer reproduces the hand-worked bytes
    assert np.array_equal(oracle.q4k_pack(0x3C00, 0x3C00, sc, m, q), blk)


# ---------------------------------------------------------------------------- Q5_K
# Q5_K is among the expert formats of the Unsloth UD-Q4_K_XL files that the
# "Strata v0.1.31" release notes say run natively; its bytes follow the public
# GGUF layout (reading R-layout in the oracle).

def test_q5k_unpack_pack_roundtrip_random_bytes():
    g = np.random.default_rng(11)
    for _ in range(300):
        blk = g.integers(0, 256, 176, dtype=np.uint8)
        f = oracle.q5k_unpack(blk.tobytes())
        assert f["q"].min() >= 0 and f["q"].max() <= 31
        back = oracle.q5k_pack(f["d_bits"], f["dmin_bits"], f["sc"], f["m"], f["q"])
        assert np.array_equal(back, blk)


def test_q5k_pack_unpack_roundtrip_random_fields():
    g = np.random.default_rng(12)
    for _ in range(300):
        d, dm = (int(v) for v in g.integers(0, 65536, 2))
        sc, m, q = g.integers(0, 64, 8), g.integers(0, 64, 8), g.integers(0, 32, 256)
        f = oracle.q5k_unpack(oracle.q5k_pack(d, dm, sc, m, q).tobytes())
        assert f["d_bits"] == d and f["dmin_bits"] == dm
        assert np.array_equal(f["sc"], sc) and np.array_equal(f["m"], m) and np.array_equal(f["q"], q)


def test_q5k_block_f_closed_form():
    blk = load_block("q5k_block_f.txt")
    f = oracle.q5k_unpack(blk.tobytes())
    assert np.array_equal(f["sc"], [1, 3, 5, 7, 17, 34, 51, 62])
    assert np.array_equal(f["m"], [0, 1, 2, 3, 20, 33, 48, 63])
    i = np.arange(256)
    j = i // 32
    assert np.array_equal(f["q"], (3 * i + 5 * j) % 32)
    w = oracle.q5k_dequant(blk)
    sc = np.array([1, 3, 5, 7, 17, 34, 51, 62])[j]
    m = np.array([0, 1, 2, 3, 20, 33, 48, 63])[j]
    assert np.array_equal(w, 0.5 * sc * ((3 * i + 5 * j) % 32) - 2.0 * m)
    assert (w[0], w[33], w[200], w[255]) == (0.0, 10.0, 465.0, -126.0)
    assert w.sum() == 33760.0


def test_q5k_without_fifth_bits_is_q4k():
    """qh = 0: a Q5_K block is the Q4_K block with the same header and low nibbles."""
    g = np.random.default_rng(13)
    for _ in range(50):
        q4 = g.integers(0, 256, 144, dtype=np.uint8)
        q4[1] &= 0x3B   # finite d and dmin
        q4[3] &= 0x3B
        q5 = np.concatenate([q4[:16], np.zeros(32, np.uint8), q4[16:]])
        assert np.array_equal(oracle.q5k_dequant(q5), oracle.q4k_dequant(q4))


def test_q5k_all_fifth_bits_add_16_d_sc():
    """qh = 0xFF: every quant gains 16, so every weight gains 16*d*sc_j (exact)."""
    g = np.random.default_rng(14)
    for _ in range(50):
        q4 = g.integers(0, 256, 144, dtype=np.uint8)
        q4[1] &= 0x3B
        q4[3] &= 0x3B
        q5 = np.concatenate([q4[:16], np.full(32, 0xFF, np.uint8), q4[16:]])
        f = oracle.q4k_unpack(q4.tobytes())
        d = oracle.fp16_to_f64(np.array([f["d_bits"]], np.uint16))[0]
        bump = np.repeat(16.0 * d * f["sc"], 32)
        assert np.array_equal(oracle.q5k_dequant(q5), oracle.q4k_dequant(q4) + bump)


def test_q5k_single_bit_sensitivity():
    """Flipping qh bit b of byte l changes exactly one weight, index 32*b + l, by 16*d*sc_b."""
    blk = load_block("q5k_block_f.txt")
    base = oracle.q5k_dequant(blk)
    f = oracle.q5k_unpack(blk.tobytes())
    for l, b in [(0, 0), (5, 3), (17, 6), (31, 7)]:
        mod = blk.copy()
        mod[16 + l] ^= 1 << b
        w = oracle.q5k_dequant(mod)
        diff = np.nonzero(w != base)[0]
        assert list(diff) == [32 * b + l]
        assert abs(w[32 * b + l] - base[32 * b + l]) == 16 * 0.5 * f["sc"][b]


# ---------------------------------------------------------------------------- Q5_1
# Q5_1 is among the expert formats of the Unsloth UD-Q4_K_XL files that the
# "Strata v0.1.31" release notes say run natively: 32-weight blocks with a
# scale, an additive offset and five-bit quants (public GGUF layout, reading
# R-layout in the oracle).

def test_q51_unpack_pack_roundtrip_random_bytes():
    g = np.random.default_rng(31)
    for _ in range(300):
        blk = g.integers(0, 256, 24, dtype=np.uint8)
        f = oracle.q51_unpack(blk)
        assert f["q"].min() >= 0 and f["q"].max() <= 31
        assert np.array_equal(oracle.q51_pack(f["d_bits"], f["m_bits"], f["q"]), blk)


def test_q51_pack_unpack_roundtrip_random_fields():
    g = np.random.default_rng(32)
    for _ in range(300):
        d, m = (int(v) for v in g.integers(0, 65536, 2))
        q = g.integers(0, 32, 32)
        f = oracle.q51_unpack(oracle.q51_pack(d, m, q))
        assert f["d_bits"] == d and f["m_bits"] == m and np.array_equal(f["q"], q)


def test_q51_block_g_closed_form():
    blk = load_block("q51_block_g.txt")
    assert blk.size == 24
    f = oracle.q51_unpack(blk)
    i = np.arange(32)
    assert np.array_equal(f["q"], (11 * i + 4 * (i // 16) + 3) % 32)
    assert f["d_bits"] == 0x3400 and f["m_bits"] == 0xC200
    w = oracle.q51_dequant(blk)
    assert np.array_equal(w, 0.25 * ((11 * i + 4 * (i // 16) + 3) % 32) - 3.0)
    assert (w[0], w[5], w[16], w[31]) == (-2.25, 3.5, 2.75, 4.0)
    assert w.sum() == 28.0


def test_q51_single_bit_sensitivity():
    """Flipping bit i of qh changes weight i alone, by 16*d; flipping bit b of qs[l]
    changes weight l (b < 4) or 16+l (b >= 4) alone, by 2^(b mod 4)*d."""
    blk = load_block("q51_block_g.txt")
    base = oracle.q51_dequant(blk)
    for i in [0, 1, 7, 15, 16, 20, 31]:
        mod = blk.copy()
        mod[4 + i // 8] ^= 1 << (i % 8)
        w = oracle.q51_dequant(mod)
        assert list(np.nonzero(w != base)[0]) == [i]
        assert abs(w[i] - base[i]) == 16 * 0.25
    for l, b in [(0, 0), (3, 2), (9, 4), (15, 7)]:
        mod = blk.copy()
        mod[8 + l] ^= 1 << b
        w = oracle.q51_dequant(mod)
        idx = l if b < 4 else 16 + l
        assert list(np.nonzero(w != base)[0]) == [idx]
        assert abs(w[idx] - base[idx]) == 2 ** (b % 4) * 0.25


def test_q51_with_offset_minus_16d_is_q80():
    """m = -16*d turns a Q5_1 block into the Q8_0 block with the same d and quants
    q - 16 (in -16..15): the two formats' definitions agree value for value."""
    g = np.random.default_rng(33)
    for d_bits, m_bits in [(0x2C00, 0xBC00), (0x3400, 0xC400), (0x1E00, 0xAE00)]:   # d, -16 d
        d = oracle.fp16_to_f64(np.array([d_bits], np.uint16))[0]
        assert oracle.fp16_to_f64(np.array([m_bits], np.uint16))[0] == -16 * d
        for _ in range(20):
            q = g.integers(0, 32, 32)
            q5 = oracle.q51_pack(d_bits, m_bits, q)
            q8 = np.concatenate([np.array([d_bits & 0xFF, d_bits >> 8], np.uint8),
                                 (q - 16).astype(np.int8).view(np.uint8)])
            assert np.array_equal(oracle.q51_dequant(q5), oracle.q80_dequant(q8))


def test_q51_dequant_is_exact_at_the_extremes():
    """Largest |d*q| against the smallest offset: the sum needs 44 bits, still exact in fp64."""
    q = np.full(32, 31)
    blk = oracle.q51_pack(0x7BFF, 0x0001, q)           # d = 65504, m = 2^-24
    w = oracle.q51_dequant(blk)
    assert np.all(w == 65504.0 * 31 + 2.0 ** -24)
    assert np.all(w - 65504.0 * 31 == 2.0 ** -24)
