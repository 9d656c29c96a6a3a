"""Pins for the oracle's fused producers of Q8_K activations (CPU only).

The pages' layer applies RMSNorm (eps 1e-5 for LLaDA) before the QKV and MLP
projections and uses a SwiGLU MLP (mojo-dllm Technical Specification,
"Transformer Execution"; Development plan, "Model facts used"), and name fused
normalization as a goal.  The oracle's definitions (a reading; the pages do not
fix the precision):
  RMSNorm -> Q8_K: codes of f32(x*g), block d times r = f32(1/sqrt(mean x^2 + eps));
  SwiGLU -> Q8_K: Q8_K of f32(gate*up/(1+exp(-gate))) evaluated in f64.
Pinned by closed forms computed at 40 digits, invariants and an independent
sigmoid (scipy's expit)."""
from decimal import Decimal, getcontext

import numpy as np

import oracle

getcontext().prec = 40


def _fields(rec):
    d = rec[0:4].view(np.float32)[0]
    q = rec[4:260].view(np.int8).astype(np.int64)
    bs = rec[260:292].view(np.int16).astype(np.int64)
    return d, q, bs


def _r_exact(x_row, eps):
    """f32 of 1/sqrt(mean(x^2) + eps) from a 40-digit evaluation."""
    ss = sum(Decimal(float(v)) ** 2 for v in x_row)
    return np.float32(float(1 / (ss / len(x_row) + Decimal(float(np.float32(eps)))).sqrt()))


# ---------------------------------------------------------------- RMSNorm ----

def test_rmsnorm_constant_row_closed_form():
    """A constant row c with g = 1: r = 1/sqrt(c^2 + eps); z = c gives codes
    -127 everywhere (pivot first, positive), d_z = 1/f32(-127/c)."""
    for c, eps, K in ((3.0, 1e-5, 512), (1e-3, 1e-5, 256), (-7.5, 1e-6, 1024)):
        x = np.full((1, K), c, np.float32)
        out, dmax = oracle.rmsnorm_quantize_q8k(x, np.ones(K, np.float32), eps)
        r = _r_exact(x[0], eps)
        iscale = np.float32(-127.0) / np.float32(c)
        dz = np.float32(1.0) / iscale
        for s in range(K // 256):
            d, q, bs = _fields(out[0, s * 292:(s + 1) * 292])
            assert list(q) == [-127] * 256
            assert list(bs) == [-127 * 16] * 16
            assert d == np.float32(r * dz)
        assert dmax[0] == abs(np.float32(r * dz))


def test_rmsnorm_codes_are_those_of_x_times_g_and_r_uses_x():
    """Codes and bsums are exactly those of quantize(f32(x*g)); g a power of
    two per block scales d_z but leaves the codes and r alone (r comes from x,
    not from x*g)."""
    rng = np.random.default_rng(41)
    M, K = 5, 1024
    x = rng.standard_normal((M, K)).astype(np.float32)
    g = rng.uniform(0.5, 2.0, K).astype(np.float32)
    out, _ = oracle.rmsnorm_quantize_q8k(x, g, 1e-5)
    plain = oracle.quantize_q8k((x * g).astype(np.float32))
    for m in range(M):
        r = _r_exact(x[m], 1e-5)
        for s in range(K // 256):
            d, q, bs = _fields(out[m, s * 292:(s + 1) * 292])
            d0, q0, bs0 = _fields(plain[m, s * 292:(s + 1) * 292])
            assert np.array_equal(q, q0) and np.array_equal(bs, bs0)
            assert d == np.float32(r * d0)
    gp = np.repeat(np.float32(2.0) ** np.arange(-1, 3, dtype=np.float32), 256)  # 1/2, 1, 2, 4 per block
    out_p, _ = oracle.rmsnorm_quantize_q8k(x, gp, 1e-5)
    out_1, _ = oracle.rmsnorm_quantize_q8k(x, np.ones(K, np.float32), 1e-5)
    for m in range(M):
        for s in range(K // 256):
            dp, qp, _ = _fields(out_p[m, s * 292:(s + 1) * 292])
            d1, q1, _ = _fields(out_1[m, s * 292:(s + 1) * 292])
            assert np.array_equal(qp, q1)
            assert dp == np.float32(d1 * gp[256 * s])


def test_rmsnorm_dequantized_matches_f64_rmsnorm():
    """d*q is within the Q8_K bound of RMSNorm(x)*g evaluated in f64 (plus the
    f32 roundings of z, r and d: a few 2^-24 relative)."""
    rng = np.random.default_rng(42)
    M, K = 4, 2048
    x = (rng.standard_normal((M, K)) * rng.uniform(0.01, 100.0, (M, 1))).astype(np.float32)
    g = rng.uniform(-2.0, 2.0, K).astype(np.float32)
    out, _ = oracle.rmsnorm_quantize_q8k(x, g, 1e-5)
    xd = x.astype(np.float64)
    y = xd / np.sqrt(np.mean(xd ** 2, axis=1, keepdims=True) + np.float64(np.float32(1e-5))) * g
    for m in range(M):
        for s in range(K // 256):
            d, q, _ = _fields(out[m, s * 292:(s + 1) * 292])
            err = np.abs(float(d) * q - y[m, s * 256:(s + 1) * 256])
            assert np.all(err <= abs(float(d)) * 0.5 * (1 + 1e-6) + 4e-7 * np.abs(y[m, s * 256:(s + 1) * 256]))


def test_rmsnorm_zero_row_and_dmax():
    K = 512
    x = np.zeros((2, K), np.float32)
    x[1, 300] = -2.0
    out, dmax = oracle.rmsnorm_quantize_q8k(x, np.ones(K, np.float32), 1e-5)
    d, q, bs = _fields(out[0, 0:292])
    assert d == 0 and not q.any() and not bs.any() and dmax[0] == 0
    d1, q1, _ = _fields(out[1, 292:584])
    assert q1[300 - 256] == -127 and d1 > 0  # negative pivot: positive d
    assert dmax[1] == abs(d1)


# ----------------------------------------------------------------- SwiGLU ----

def _act_exact(g, u):
    gd, ud = Decimal(float(g)), Decimal(float(u))
    return np.float32(float(gd * ud / (1 + (-gd).exp())))


def test_swiglu_matches_40_digit_values_then_q8k():
    """act from a 40-digit evaluation of gate*up/(1+e^-gate), rounded to f32,
    quantized by the (separately pinned) oracle quantizer: the same bytes."""
    rng = np.random.default_rng(43)
    M, F = 2, 512
    gate = rng.uniform(-20.0, 20.0, (M, F)).astype(np.float32)
    gate[0, :4] = [0.0, np.float32(np.log(3.0)), -800.0, 40.0]
    up = rng.standard_normal((M, F)).astype(np.float32)
    out, dmax = oracle.swiglu_quantize_q8k(np.concatenate([gate, up], axis=1))
    act = np.array([[_act_exact(gate[m, k], up[m, k]) for k in range(F)] for m in range(M)], np.float32)
    assert np.array_equal(out, oracle.quantize_q8k(act))
    ds = out.reshape(M, F // 256, 292)[:, :, :4].copy().view(np.float32)[..., 0]
    assert np.array_equal(dmax, np.abs(ds).max(axis=1))


def test_swiglu_gate_up_order_and_special_values():
    """silu(gate) * up, not silu(up) * gate; gate 0 or very negative gives 0;
    a large gate gives gate * up; against scipy's expit."""
    from scipy.special import expit
    F = 256
    gate = np.zeros((1, F), np.float32)
    up = np.ones((1, F), np.float32)
    gate[0, 1], up[0, 1] = 2.0, 5.0
    gate[0, 2], up[0, 2] = -1000.0, 3.0
    gate[0, 3], up[0, 3] = 60.0, 0.125
    out, _ = oracle.swiglu_quantize_q8k(np.concatenate([gate, up], axis=1))
    d, q, _ = _fields(out[0])
    deq = float(d) * q
    assert deq[0] == 0 and deq[2] == 0
    want1 = 2.0 * expit(2.0) * 5.0  # 8.807..., the block's largest: the pivot
    assert q[1] == -127 and abs(deq[1] - want1) <= abs(float(d)) * 0.5
    assert abs(deq[3] - 7.5) <= abs(float(d)) * 0.5
    swapped = 5.0 * expit(5.0) * 2.0
    assert abs(deq[1] - swapped) > abs(float(d))
