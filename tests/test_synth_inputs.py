"""The seeded synthetic inputs follow the stated workload shapes and value laws.

Checks, on the host generators: the five layer shapes (tiny, Sage-like decode,
3-token window, Flash-Next-like decode, 4,096-token prompt chunk); fp16 scales
drawn as |N(0,1)| * 0.01 (non-negative, finite, mean 0.01*sqrt(2/pi)); Q4_K
4-bit quants and 6-bit scales uniform over their ranges; Q8_0 codes in
-127..127 (never -128); Q5_1 offsets non-positive; the Zipf(s) logit bias
-s*ln(e+1); and that a seed fixes every byte.  CPU only.
"""
import math

import numpy as np

from quantized_moe_ffn_amd import synth


def test_workload_shapes():
    W = synth.WORKLOADS
    t = W["tiny"]
    assert (t.hidden, t.n_experts, t.top_k, t.inter, t.tokens) == (256, 8, 2, 256, 4)
    s = W["sage_decode"]
    assert (s.hidden, s.n_experts, s.top_k, s.inter, s.tokens, s.layers) == (2048, 256, 8, 512, 1, 40)
    assert (s.qt_gate, s.qt_up, s.qt_down, s.shared) == (synth.Q4_K, synth.Q4_K, synth.Q4_K, False)
    m = W["mtp_window"]
    assert (m.hidden, m.n_experts, m.top_k, m.inter, m.tokens, m.layers) == (2048, 256, 8, 512, 3, 40)
    f = W["flash_next_decode"]
    assert (f.hidden, f.n_experts, f.top_k, f.inter, f.tokens, f.layers) == (2560, 512, 10, 512, 1, 48)
    assert (f.qt_gate, f.qt_up, f.qt_down, f.shared) == (synth.Q4_K, synth.Q4_K, synth.Q8_0, True)
    p = W["prefill_chunk"]
    assert (p.hidden, p.n_experts, p.top_k, p.inter, p.tokens) == (2048, 256, 8, 512, 4096)
    assert p.int8_path and p.zipf_s == 1.1
    # bytes of one Sage-like expert: gate + up (512 rows of 8 Q4_K blocks) + down (2048 rows of 2)
    assert s.expert_bytes() == 2 * 512 * 8 * 144 + 2048 * 2 * 144 == 1_769_472
    assert f.expert_bytes() == 2 * 512 * 10 * 144 + 2560 * 16 * 34 == 2_867_200


def _f16(b, off):
    return b[:, off:off + 2].copy().view(np.float16).astype(np.float64).ravel()


def test_q4k_value_laws():
    b = synth.q4k_blocks_np(synth.rng(5), 40_000)
    assert b.shape == (40_000, 144)
    for off in (0, 2):   # d, dmin
        v = _f16(b, off)
        assert np.all(np.isfinite(v)) and np.all(v >= 0)
        assert abs(v.mean() - 0.01 * math.sqrt(2 / math.pi)) < 2e-4
    q = np.concatenate([b[:, 16:] & 15, b[:, 16:] >> 4], axis=1)
    assert q.min() == 0 and q.max() == 15 and abs(q.mean() - 7.5) < 0.02
    sc = b[:, 4:8] & 63   # the low 6 bits of the first four scale bytes: sub-block scales 0..3
    assert sc.min() == 0 and sc.max() == 63 and abs(sc.mean() - 31.5) < 0.2


def test_q80_and_q51_value_laws():
    b = synth.q80_blocks_np(synth.rng(6), 40_000)
    q = b[:, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127 and abs(q.astype(np.float64).mean()) < 0.1
    d = _f16(b, 0)
    assert np.all(np.isfinite(d)) and np.all(d >= 0)
    c = synth.q51_blocks_np(synth.rng(7), 40_000)
    assert np.all(_f16(c, 0) >= 0) and np.all(_f16(c, 2) <= 0)
    assert abs(_f16(c, 2).mean() + 0.16 * math.sqrt(2 / math.pi)) < 3e-3


def test_zipf_bias_and_logits():
    bias = synth.zipf_bias(256, 1.1)
    assert bias[0] == 0.0
    assert np.allclose(bias, -1.1 * np.log(np.arange(1, 257)), rtol=0, atol=1e-6)
    plain = synth.logits_np(synth.rng(8), 64, 256)
    skew = synth.logits_np(synth.rng(8), 64, 256, 1.1)
    assert np.allclose(skew - plain, bias[None, :], atol=1e-5)


def test_a_seed_fixes_every_byte():
    a = synth.bank_np(synth.rng(9, 1), synth.Q4_K, 2, 8, 512)
    b = synth.bank_np(synth.rng(9, 1), synth.Q4_K, 2, 8, 512)
    c = synth.bank_np(synth.rng(9, 2), synth.Q4_K, 2, 8, 512)
    assert a.shape == (2, 8, 2 * 144) and np.array_equal(a, b) and not np.array_equal(a, c)
    assert synth.seed_of(1, 2) != synth.seed_of(2, 1)
