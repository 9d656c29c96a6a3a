"""Pins for the oracle's block decoders (CPU only).

The pages name the GGUF Q4_K / Q6_K super-blocks (mojo-dllm Development plan,
"Corrections to the spec" table and "Compute design") but print no layout or
worked block; the pins below fix the decoders against values chosen first and
packed into bytes by an independent packer (tests/ggufpack.py), plus
IEEE binary16 as numpy defines it.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from ggufpack import f16_bits, f16_value, pack_q4k, pack_q6k


def test_f16_all_finite_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits[finite]])
    assert np.array_equal(got, ref[finite])


def test_q4k_hand_built_block():
    # d = 1, dmin = 0.5, sc_j = 63 - j, m_j = 32 + j (sub-blocks 4..7 use the
    # split high-bit path), u_i = i % 16.
    sc = [63 - j for j in range(8)]
    mn = [32 + j for j in range(8)]
    u = [i % 16 for i in range(256)]
    blk = pack_q4k(f16_bits(1.0), f16_bits(0.5), sc, mn, u)
    w = oracle.decode_rows(oracle.Q4_K, blk, 1, 256)[0]
    exp = np.array([(63 - i // 32) * (i % 16) - 0.5 * (32 + i // 32) for i in range(256)])
    assert np.array_equal(w, exp)


@pytest.mark.parametrize("seed", range(8))
def test_q4k_random_known_fields(seed):
    rng = np.random.default_rng(seed)
    sc = rng.integers(0, 64, 8)
    mn = rng.integers(0, 64, 8)
    u = rng.integers(0, 16, 256)  # position-unique pattern: catches index swaps
    d = float(np.float16(rng.uniform(1e-3, 1e-2)))
    dmin = float(np.float16(rng.uniform(1e-3, 1e-2)))
    blk = pack_q4k(f16_bits(d), f16_bits(dmin), sc, mn, u)
    d2, dm2, sc2, mn2, u2 = oracle.q4k_fields(blk)
    assert (d2, dm2) == (d, dmin)
    assert list(sc2) == list(sc) and list(mn2) == list(mn) and list(u2) == list(u)
    w = oracle.decode_rows(oracle.Q4_K, blk, 1, 256)[0]
    for i in range(256):
        j = i // 32
        exact = Fraction(d) * int(sc[j]) * int(u[i]) - Fraction(dmin) * int(mn[j])
        assert Fraction(w[i]) == exact


def test_q4k_scale_min_pack_bijection_exhaustive():
    u = [0] * 256
    base_sc = [5, 9, 13, 17, 21, 25, 29, 33]
    base_mn = [40, 36, 32, 28, 24, 20, 16, 12]
    for j in range(8):
        for s in range(64):
            for m in range(64):
                sc = list(base_sc); mn = list(base_mn)
                sc[j], mn[j] = s, m
                blk = pack_q4k(0x3C00, 0x3C00, sc, mn, u)
                _, _, sc2, mn2, _ = oracle.q4k_fields(blk)
                assert list(sc2) == sc and list(mn2) == mn, (j, s, m)


def test_q4k_one_hot_probes_reveal_element_positions():
    # One-hot quant at element i (all others zero), unit scales, no mins: the
    # decoded row must be the one-hot at i.
    for i in range(256):
        u = [0] * 256
        u[i] = 15
        blk = pack_q4k(0x3C00, 0, [1] * 8, [0] * 8, u)
        w = oracle.decode_rows(oracle.Q4_K, blk, 1, 256)[0]
        assert np.flatnonzero(w).tolist() == [i] and w[i] == 15.0


def test_q6k_hand_built_block():
    # d = 1, sc_g = g - 8 (negatives included), q_i = i % 64.
    sc = [g - 8 for g in range(16)]
    q = [i % 64 for i in range(256)]
    blk = pack_q6k(f16_bits(1.0), sc, q)
    w = oracle.decode_rows(oracle.Q6_K, blk, 1, 256)[0]
    exp = np.array([(i // 16 - 8) * (i % 64 - 32) for i in range(256)], np.float64)
    assert np.array_equal(w, exp)


def test_q6k_extreme_scale_minus_128():
    sc = [-128] * 16
    q = [(7 * i + 3) % 64 for i in range(256)]
    blk = pack_q6k(f16_bits(0.25), sc, q)
    w = oracle.decode_rows(oracle.Q6_K, blk, 1, 256)[0]
    assert np.array_equal(w, np.array([0.25 * -128 * (v - 32) for v in q]))


def test_q6k_every_quant_value_at_every_position():
    for shift in range(64):
        q = [(i + shift) % 64 for i in range(256)]
        sc = [(g * 37 + shift) % 256 - 128 for g in range(16)]
        blk = pack_q6k(0x3C00, sc, q)
        d, sc2, q2 = oracle.q6k_fields(blk)
        assert d == 1.0 and list(sc2) == sc and list(q2) == q


@pytest.mark.parametrize("seed", range(4))
def test_q6k_random_known_fields_exact(seed):
    rng = np.random.default_rng(100 + seed)
    sc = rng.integers(-128, 128, 16)
    q = rng.integers(0, 64, 256)
    d = float(np.float16(rng.uniform(1e-3, 1e-2)))
    blk = pack_q6k(f16_bits(d), sc, q)
    w = oracle.decode_rows(oracle.Q6_K, blk, 1, 256)[0]
    for i in range(256):
        assert Fraction(w[i]) == Fraction(d) * int(sc[i // 16]) * (int(q[i]) - 32)


def _shared_fields(rec: np.ndarray):
    D = rec[0:4].view(np.float32)[0]
    off = rec[4:68].view(np.float32)
    sc = rec[68:100].view(np.int16)
    u = rec[100:356]
    return D, off, sc, u


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
def test_shared_form_identity_on_generator_blocks(qtype):
    import synth
    rows = synth.qk_rows(qtype, 4, 1024, 7, "shared-identity").numpy()
    w = oracle.decode_rows(qtype, rows, 4, 1024)
    rec = oracle.decode_shared(qtype, rows, 16)
    for s in range(16):
        D, off, sc, u = _shared_fields(rec[s])
        n, sb = divmod(s, 4)
        for i in range(256):
            g = i // 16
            val = Fraction(float(D)) * int(sc[g]) * int(u[i]) + Fraction(float(off[g]))
            assert val == Fraction(w[n, 256 * sb + i])


def test_shared_form_known_block_q4k():
    sc = [63 - j for j in range(8)]
    mn = [32 + j for j in range(8)]
    u = [(3 * i) % 16 for i in range(256)]
    blk = pack_q4k(f16_bits(0.5), f16_bits(0.25), sc, mn, u)
    D, off, sc16, u8 = _shared_fields(oracle.decode_shared(oracle.Q4_K, blk, 1)[0])
    assert D == 0.5
    assert list(sc16) == [sc[g // 2] for g in range(16)]
    assert list(off) == [-0.25 * mn[g // 2] for g in range(16)]
    assert list(u8) == u


def test_shared_form_known_block_q6k():
    sc = [g * 16 - 128 for g in range(16)]
    q = [(5 * i) % 64 for i in range(256)]
    blk = pack_q6k(f16_bits(2.0), sc, q)
    D, off, sc16, u8 = _shared_fields(oracle.decode_shared(oracle.Q6_K, blk, 1)[0])
    assert D == 2.0
    assert list(sc16) == sc
    assert [float(v) for v in off] == [-64.0 * s for s in sc]
    assert list(u8) == q
    assert f16_value(f16_bits(2.0)) == 2.0
