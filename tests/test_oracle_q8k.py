"""Pins for the oracle's Q8_K quantizer (CPU only).

The pages fix one f32 scale per 256 values and int sums per 16 (mojo-dllm
Development plan, "Compute design", first bullet).  The rounding rule, scale
sign and tie-break are the GGUF format's own definition (a reading; the pages
are silent).  Pinned here by closed forms and invariants of that definition.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _fields(rec):
    d = rec[0:4].view(np.float32)[0]
    q = rec[4:260].view(np.int8).astype(np.int64)
    bs = rec[260:292].view(np.int16).astype(np.int64)
    return d, q, bs


def _blocks(xq, M, K):
    return xq.reshape(M * (K // 256), 292)


def test_closed_form_integer_ramp():
    # x_i = i - 128: the pivot is x_0 = -128 (first max |x|), so
    # iscale = -127/-128 = 127/128 exactly; every product is exact in f32 and
    # q_i = round-half-even(127 (i-128) / 128); d = f32(128/127).
    x = (np.arange(256) - 128).astype(np.float32)[None, :]
    d, q, bs = _fields(oracle.quantize_q8k(x)[0])
    exp = [round(Fraction(127 * (i - 128), 128)) for i in range(256)]  # half-even
    assert list(q) == exp
    assert q[0] == -127
    assert d == np.float32(1.0) / np.float32(127.0 / 128.0)
    assert list(bs) == [sum(exp[16 * g:16 * g + 16]) for g in range(16)]


def test_positive_pivot_gives_negative_scale():
    x = np.zeros((1, 256), np.float32)
    x[0, 10] = 2.0
    x[0, 11] = -1.0
    d, q, bs = _fields(oracle.quantize_q8k(x)[0])
    assert q[10] == -127 and d < 0
    assert q[11] == round(Fraction(127, 2))  # 63.5 -> 64 (half-even)
    assert q[11] == 64


def test_first_index_wins_magnitude_tie():
    x = np.zeros((1, 256), np.float32)
    x[0, 3] = -5.0
    x[0, 200] = 5.0
    d, q, _ = _fields(oracle.quantize_q8k(x)[0])
    assert q[3] == -127 and q[200] == 127 and d > 0
    x[0, 3], x[0, 200] = 5.0, -5.0
    d, q, _ = _fields(oracle.quantize_q8k(x)[0])
    assert q[3] == -127 and q[200] == 127 and d < 0


def test_all_zero_block():
    x = np.zeros((2, 512), np.float32)
    x[1, 300] = 1.0
    xq = oracle.quantize_q8k(x)
    recs = _blocks(xq, 2, 512)
    for r in (0, 1, 2):
        d, q, bs = _fields(recs[r])
        assert d == 0 and not q.any() and not bs.any()
    d, q, _ = _fields(recs[3])
    assert q[300 - 256] == -127


@pytest.mark.parametrize("seed", range(4))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    M, K = 6, 1024
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(10.0 ** rng.uniform(-3, 3))
    recs = _blocks(oracle.quantize_q8k(x), M, K)
    for r, rec in enumerate(recs):
        m, s = divmod(r, K // 256)
        xb = x[m, 256 * s:256 * s + 256].astype(np.float64)
        d, q, bs = _fields(rec)
        piv = int(np.argmax(np.abs(xb)))  # numpy argmax: first index
        assert q[piv] == -127
        assert np.abs(q).max() <= 127
        assert list(bs) == list(q.reshape(16, 16).sum(1))
        err = np.abs(xb - float(d) * q)
        # rounding of iscale, of iscale*x and of d adds at most ~2*127*2^-24 |d|
        assert err.max() <= abs(float(d)) / 2 * (1 + 2.0 ** -14)


@pytest.mark.parametrize("seed", range(3))
def test_sign_and_power_of_two_symmetry(seed):
    rng = np.random.default_rng(50 + seed)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    base = _blocks(oracle.quantize_q8k(x), 3, 512)
    neg = _blocks(oracle.quantize_q8k(-x), 3, 512)
    for k in (-7, 3, 20):
        scaled = _blocks(oracle.quantize_q8k(x * np.float32(2.0 ** k)), 3, 512)
        for a, c in zip(base, scaled):
            da, qa, ba = _fields(a)
            dc, qc, bc = _fields(c)
            assert np.array_equal(qa, qc) and np.array_equal(ba, bc)
            assert dc == np.float32(da * np.float32(2.0 ** k))
    for a, b in zip(base, neg):
        da, qa, ba = _fields(a)
        db, qb, bb = _fields(b)
        assert np.array_equal(qa, qb) and np.array_equal(ba, bb) and db == -da


def test_dequant_is_d_times_q():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 512)).astype(np.float32)
    xq = oracle.quantize_q8k(x)
    xh = oracle.dequant_q8k(xq, 2, 512)
    recs = _blocks(xq, 2, 512)
    for r, rec in enumerate(recs):
        m, s = divmod(r, 2)
        d, q, _ = _fields(rec)
        assert np.array_equal(xh[m, 256 * s:256 * s + 256], float(d) * q)
