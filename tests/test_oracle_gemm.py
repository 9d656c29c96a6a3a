"""Pins for the oracle's GEMM, per-16 partials and masked-row LM head (CPU).

What the path computes: each linear layer multiplies the per-token Q8_K
activations by Q4_K/Q6_K weight rows (mojo-dllm Development plan, "Compute
design"); the LM head only runs on the masked rows (same section; README
"How it works", "Logits only where the sampler looks").  The exact result is
y = W_hat X_hat^T of the dequantized operands.  Pinned by: exact rational
brute force from values chosen before packing, an f32 library dot product, an
integer special case, zero weights, and planted argmax rows.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from ggufpack import f16_bits, pack_q4k, pack_q6k, pack_q8k


def _rand_q4k(rng):
    sc = rng.integers(0, 64, 8); mn = rng.integers(0, 64, 8); u = rng.integers(0, 16, 256)
    d = float(np.float16(rng.uniform(1e-3, 1e-2))); dm = float(np.float16(rng.uniform(1e-3, 1e-2)))
    blk = pack_q4k(f16_bits(d), f16_bits(dm), sc, mn, u)
    vals = [Fraction(d) * int(sc[i // 32]) * int(u[i]) - Fraction(dm) * int(mn[i // 32]) for i in range(256)]
    return blk, vals, u


def _rand_q6k(rng):
    sc = rng.integers(-128, 128, 16); q = rng.integers(0, 64, 256)
    d = float(np.float16(rng.uniform(1e-3, 1e-2)))
    blk = pack_q6k(f16_bits(d), sc, q)
    vals = [Fraction(d) * int(sc[i // 16]) * (int(q[i]) - 32) for i in range(256)]
    return blk, vals, q


def _rand_q8k(rng):
    q = rng.integers(-127, 128, 256)
    d = float(np.float32(rng.uniform(-0.05, 0.05)))
    return pack_q8k(d, q), [Fraction(d) * int(v) for v in q], q


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
@pytest.mark.parametrize("seed", range(3))
def test_exact_rational_brute_force(qtype, seed):
    """N=3 rows, M=2 tokens, K=512: every output against an exact rational sum
    of values chosen before packing, within 2^-50 * sum |terms|."""
    rng = np.random.default_rng(1000 + seed)
    N, M, K = 3, 2, 512
    mk = _rand_q4k if qtype == oracle.Q4_K else _rand_q6k
    wrows, wvals = [], []
    for _ in range(N):
        bl, vl = [], []
        for _ in range(K // 256):
            b, v, _ = mk(rng); bl.append(b); vl += v
        wrows.append(np.concatenate(bl)); wvals.append(vl)
    xrows, xvals = [], []
    for _ in range(M):
        bl, vl = [], []
        for _ in range(K // 256):
            b, v, _ = _rand_q8k(rng); bl.append(b); vl += v
        xrows.append(np.concatenate(bl)); xvals.append(vl)
    y = oracle.gemm(qtype, np.stack(wrows), N, K, np.stack(xrows), M)
    # the same product with a bias per output feature (Dream-7B's QKV bias)
    bias = (rng.standard_normal(N) * 10.0).astype(np.float32)
    yb = oracle.gemm(qtype, np.stack(wrows), N, K, np.stack(xrows), M, bias=bias)
    for m in range(M):
        for n in range(N):
            terms = [a * b for a, b in zip(wvals[n], xvals[m])]
            exact = sum(terms)
            bound = sum(abs(t) for t in terms) * Fraction(1, 2 ** 50)
            assert abs(Fraction(y[m, n]) - exact) <= bound
            exact_b = exact + Fraction(float(bias[n]))
            assert abs(Fraction(yb[m, n]) - exact_b) <= bound + abs(exact_b) * Fraction(1, 2 ** 52)


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
def test_f32_library_cross_check(qtype):
    rng_seed = 77
    N, M, K = 24, 9, 1024
    w = synth.qk_rows(qtype, N, K, rng_seed, "w").numpy()
    x = synth.normal_f32((M, K), rng_seed, "x").numpy()
    xq = oracle.quantize_q8k(x)
    y64 = oracle.gemm(qtype, w, N, K, xq, M)
    wh = oracle.decode_rows(qtype, w, N, K)
    xh = oracle.dequant_q8k(xq, M, K)
    y32 = xh.astype(np.float32) @ wh.astype(np.float32).T
    absdot = np.abs(xh) @ np.abs(wh).T
    assert np.all(np.abs(y64 - y32) <= (K + 4) * 2.0 ** -24 * absdot + 1e-30)


def test_integer_special_case_q4k():
    # d = 1, dmin = 0, unit scales: weights are the 4-bit quants; activations
    # with d_x = 1 are the int8 quants, so y is an exact integer dot product.
    rng = np.random.default_rng(5)
    N, M, K = 4, 3, 512
    u = rng.integers(0, 16, (N, K)); q = rng.integers(-127, 128, (M, K))
    w = np.stack([np.concatenate([pack_q4k(0x3C00, 0, [1] * 8, [0] * 8, u[n, 256 * s:256 * s + 256])
                                  for s in range(2)]) for n in range(N)])
    xq = np.stack([np.concatenate([pack_q8k(1.0, q[m, 256 * s:256 * s + 256]) for s in range(2)])
                   for m in range(M)])
    y = oracle.gemm(oracle.Q4_K, w, N, K, xq, M)
    assert np.array_equal(y, (q @ u.T).astype(np.float64))


def test_integer_special_case_q6k():
    rng = np.random.default_rng(6)
    N, M, K = 3, 2, 256
    q6 = rng.integers(0, 64, (N, K)); q = rng.integers(-127, 128, (M, K))
    w = np.stack([pack_q6k(0x3C00, [1] * 16, q6[n]) for n in range(N)])
    xq = np.stack([pack_q8k(1.0, q[m]) for m in range(M)])
    y = oracle.gemm(oracle.Q6_K, w, N, K, xq, M)
    assert np.array_equal(y, (q @ (q6 - 32).T).astype(np.float64))


def test_zero_weights_give_zero():
    N, M, K = 5, 4, 512
    w = np.zeros((N, K // 256 * 144), np.uint8)
    x = synth.normal_f32((M, K), 1, "x").numpy()
    assert not oracle.gemm(oracle.Q4_K, w, N, K, oracle.quantize_q8k(x), M).any()


def test_zero_weights_with_bias_give_the_bias():
    """Every token's row is the bias itself, feature by feature (not a
    transposed or token-indexed bias)."""
    N, M, K = 7, 3, 256
    w = np.zeros((N, K // 256 * 210), np.uint8)
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 2, "x").numpy())
    bias = np.float32([1.5, -2.25, 3e-8, 0.0, -7e4, 0.1, 42.0])
    y = oracle.gemm(oracle.Q6_K, w, N, K, xq, M, bias=bias)
    assert np.array_equal(y, np.tile(bias.astype(np.float64), (M, 1)))
    mi = np.array([0, 2, 1, 2]); ni = np.array([6, 0, 4, 1])
    assert np.array_equal(oracle.gemm_sample(oracle.Q6_K, w, N, K, xq, M, mi, ni, bias=bias), y[mi, ni])


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
def test_gemm_sample_matches_full(qtype):
    N, M, K = 17, 5, 768
    w = synth.qk_rows(qtype, N, K, 3, "w").numpy()
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 3, "x").numpy())
    y = oracle.gemm(qtype, w, N, K, xq, M, nthreads=3)
    rng = np.random.default_rng(0)
    mi = rng.integers(0, M, 40); ni = rng.integers(0, N, 40)
    assert np.array_equal(oracle.gemm_sample(qtype, w, N, K, xq, M, mi, ni), y[mi, ni])
    assert np.array_equal(oracle.gemm(qtype, w, N, K, xq, M, nthreads=1), y)


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
def test_partials_from_known_values(qtype):
    rng = np.random.default_rng(31)
    mk = _rand_q4k if qtype == oracle.Q4_K else _rand_q6k
    wb, _, u = mk(rng)
    xb, _, q = _rand_q8k(rng)
    P = oracle.partials(qtype, wb[None], 1, 256, xb[None], 1)
    exp = (np.asarray(u).reshape(16, 16) * np.asarray(q).reshape(16, 16)).sum(1)
    assert P.shape == (1, 1, 1, 16) and list(P[0, 0, 0]) == list(exp)


@pytest.mark.parametrize("qtype", [oracle.Q4_K, oracle.Q6_K])
def test_partials_recombine_to_gemm(qtype):
    # y = sum_sb d_x * sum_g (D sc16_g P_g + off_g bsum_g): the shared-form
    # identity applied to the integer partials reproduces the f64 GEMM.
    N, M, K = 3, 2, 512
    w = synth.qk_rows(qtype, N, K, 4, "w").numpy()
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 4, "x").numpy())
    P = oracle.partials(qtype, w, N, K, xq, M)
    rec = oracle.decode_shared(qtype, w, N * 2).reshape(N, 2, 356)
    y = oracle.gemm(qtype, w, N, K, xq, M)
    xr = xq.reshape(M, 2, 292)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for s in range(2):
                D = Fraction(float(rec[n, s, 0:4].view(np.float32)[0]))
                off = rec[n, s, 4:68].view(np.float32)
                sc = rec[n, s, 68:100].view(np.int16)
                dx = Fraction(float(xr[m, s, 0:4].view(np.float32)[0]))
                bs = xr[m, s, 260:292].view(np.int16)
                for g in range(16):
                    tot += dx * (D * int(sc[g]) * int(P[m, n, s, g]) + Fraction(float(off[g])) * int(bs[g]))
            assert abs(Fraction(y[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 60)


def test_lmhead_gathers_quantizes_and_matches_gemm():
    N, M, K = 50, 12, 512
    w = synth.q6k_rows(N, K, 8, "out").numpy()
    h = synth.normal_f32((M, K), 8, "h").numpy()
    rows = np.array([7, 2, 11, 0], np.int32)
    logits, am = oracle.lmhead(oracle.Q6_K, w, N, K, h, rows)
    ref = oracle.gemm(oracle.Q6_K, w, N, K, oracle.quantize_q8k(h[rows]), rows.size)
    assert np.array_equal(logits, ref)
    assert list(am) == list(np.argmax(ref, axis=1))


def test_lmhead_planted_argmax_and_lowest_index_tie():
    N, M, K = 40, 6, 256
    rng = np.random.default_rng(12)
    q6 = rng.integers(0, 64, (N, K))
    sc = rng.integers(-8, 8, (N, 16))
    # Row 29 is a huge positive multiple of the hidden row 0 pattern; rows 13
    # and 31 are identical copies that dominate for hidden row 1, so the tie
    # must resolve to 13.
    h = rng.standard_normal((M, K)).astype(np.float32)
    xq0 = oracle.quantize_q8k(h[0:1])[0]
    q0 = xq0[4:260].view(np.int8).astype(np.int64)
    d0 = xq0[0:4].view(np.float32)[0]
    sgn = -1 if d0 < 0 else 1
    q6[29] = np.clip(32 + sgn * np.sign(q0) * 31, 0, 63)
    sc[29] = 127
    xq1 = oracle.quantize_q8k(h[1:2])[0]
    q1 = xq1[4:260].view(np.int8).astype(np.int64)
    d1 = xq1[0:4].view(np.float32)[0]
    sgn1 = -1 if d1 < 0 else 1
    q6[13] = q6[31] = np.clip(32 + sgn1 * np.sign(q1) * 31, 0, 63)
    sc[13] = sc[31] = 127
    w = np.stack([pack_q6k(f16_bits(0.01), sc[n], q6[n]) for n in range(N)])
    _, am = oracle.lmhead(oracle.Q6_K, w, N, K, h, np.array([0, 1], np.int32))
    assert am[0] == 29
    assert am[1] == 13


# ---- confidence of the greedy pick (log-sum-exp, softmax probability of the argmax)

def test_softmax_stats_closed_forms():
    """Equal logits: lse = c + ln N, p = 1/N.  One logit a above N-1 zeros:
    lse = ln(N - 1 + e^a), p = e^a / (N - 1 + e^a); below them the argmax is a
    zero and p = 1 / (N - 1 + e^a)."""
    for N, c in ((1, 0.25), (7, -3.0), (126464, 12.5)):
        lse, p = oracle.softmax_stats(np.full((1, N), c))
        assert abs(lse[0] - (c + math.log(N))) <= 1e-12 * (1 + abs(c) + math.log(N))
        assert abs(p[0] - 1.0 / N) <= 1e-12 / N
    for N, a in ((5, 2.0), (1000, 7.5), (1000, -4.0)):
        row = np.zeros(N)
        row[N // 3] = a
        lse, p = oracle.softmax_stats(row)
        z = (N - 1) + math.exp(a)
        assert abs(lse[0] - math.log(z)) <= 1e-12 * max(1.0, abs(math.log(z)))
        want = math.exp(a) / z if a > 0 else 1.0 / z
        assert abs(p[0] - want) <= 1e-12 * want


def test_softmax_stats_shift_and_large_values():
    """Adding c to every logit adds c to lse and leaves p unchanged, also for
    logits near 1000 where exp without the max shift overflows."""
    rng = np.random.default_rng(31)
    row = rng.standard_normal(4096) * 3.0
    lse0, p0 = oracle.softmax_stats(row)
    for c in (-500.0, 1000.0, 1e5):
        lse, p = oracle.softmax_stats(row + c)
        assert np.isfinite(lse[0]) and np.isfinite(p[0])
        assert abs(lse[0] - (lse0[0] + c)) <= 1e-10 * (abs(c) + abs(lse0[0]))
        assert abs(p[0] - p0[0]) <= 1e-9 * p0[0]
    lse, p = oracle.softmax_stats(np.array([[1000.0, 1001.0]]))
    assert abs(lse[0] - (1001.0 + math.log1p(math.exp(-1.0)))) <= 1e-12 * 1001.0
    assert abs(p[0] - 1.0 / (1.0 + math.exp(-1.0))) <= 1e-15


def test_softmax_stats_against_scipy():
    """scipy.special.logsumexp (an independent routine) on random rows of
    several spreads; p = exp(max - lse) from its value."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(32)
    lg = rng.standard_normal((6, 3000)) * np.array([0.01, 0.5, 1.0, 4.0, 20.0, 300.0])[:, None]
    lse, p = oracle.softmax_stats(lg)
    ref = logsumexp(lg, axis=1)
    assert np.allclose(lse, ref, rtol=1e-13, atol=1e-12)
    assert np.allclose(p, np.exp(lg.max(axis=1) - ref), rtol=1e-11, atol=0)
