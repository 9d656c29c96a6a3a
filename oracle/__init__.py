"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The product path
(diffusion_lm_gemm_amd) never imports it.

Parity: every function here is pinned by the "not gpu" tests in
tests/test_oracle_*.py (hand-built blocks, exact rational brute force, f32
cross-checks, quantizer invariants, planted argmax).  The one thing that is
not pinned is byte-for-byte compatibility with real GGUF files: no GGUF file,
gguf package or llama.cpp is available, so the layouts follow the public
format description only ("parity unpinned" for real-file compatibility).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q4_K = 12
Q6_K = 14

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain scalar C, f64 sums)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-o",
               _LIB_PATH + ".tmp", _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_q4k_fields.restype = None
        L.oracle_q4k_fields.argtypes = [P, P, P, P, P, P]
        L.oracle_f16_round.restype = ctypes.c_double
        L.oracle_f16_round.argtypes = [ctypes.c_float]
        L.oracle_q6k_fields.restype = None
        L.oracle_q6k_fields.argtypes = [P, P, P, P]
        for name, args in {
            "oracle_decode_rows": [I, P, I64, I64, P],
            "oracle_softmax_stats": [P, I64, I64, P, P],
            "oracle_attention": [P, I64, I64, I64, I64, I64, ctypes.c_double, P],
            "oracle_rmsnorm_quantize_q8k": [P, I64, I64, I64, P, ctypes.c_float, P, P],
            "oracle_swiglu_quantize_q8k": [P, I64, I64, I64, P, P],
            "oracle_decode_shared": [I, P, I64, P],
            "oracle_quantize_q8k": [P, I64, I64, I64, P],
            "oracle_dequant_q8k": [P, I64, I64, P],
            "oracle_gemm": [I, P, I64, I64, P, I64, P, I],
            "oracle_gemm_sample": [I, P, I64, I64, P, I64, P, P, I64, P],
            "oracle_partials": [I, P, I64, I64, P, I64, P],
            "oracle_lmhead": [I, P, I64, I64, P, I64, I64, P, I64, P, P, I],
        }.items():
            fn = getattr(L, name)
            fn.restype = I
            fn.argtypes = args
        _lib = L
    return _lib


def _u8(a) -> np.ndarray:
    a = np.asarray(a)
    return np.ascontiguousarray(a.view(np.uint8) if a.dtype != np.uint8 else a)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def default_threads() -> int:
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(int(h))


def q4k_fields(block: np.ndarray):
    """(d, dmin, sc[8], min[8], u[256]) of one 144-byte Q4_K block."""
    b = _u8(block)
    assert b.size == 144
    d = np.zeros(1); dm = np.zeros(1)
    sc = np.zeros(8, np.int32); mn = np.zeros(8, np.int32); u = np.zeros(256, np.int32)
    lib().oracle_q4k_fields(_p(b), _p(d), _p(dm), _p(sc), _p(mn), _p(u))
    return float(d[0]), float(dm[0]), sc, mn, u


def q6k_fields(block: np.ndarray):
    """(d, sc[16], q[256]) of one 210-byte Q6_K block."""
    b = _u8(block)
    assert b.size == 210
    d = np.zeros(1); sc = np.zeros(16, np.int32); q = np.zeros(256, np.int32)
    lib().oracle_q6k_fields(_p(b), _p(d), _p(sc), _p(q))
    return float(d[0]), sc, q


def decode_rows(qtype: int, w, N: int, K: int) -> np.ndarray:
    """Exact f64 weights [N, K]."""
    w = _u8(w)
    out = np.zeros((N, K), np.float64)
    _check(lib().oracle_decode_rows(qtype, _p(w), N, K, _p(out)), "decode_rows")
    return out


def decode_shared(qtype: int, w, n_superblocks: int) -> np.ndarray:
    """Shared decoded form, uint8 [n_superblocks, 356]."""
    w = _u8(w)
    out = np.zeros((n_superblocks, 356), np.uint8)
    _check(lib().oracle_decode_shared(qtype, _p(w), n_superblocks, _p(out)), "decode_shared")
    return out


def quantize_q8k(x: np.ndarray) -> np.ndarray:
    """f32 [M, K] -> Q8_K bytes uint8 [M, K/256*292]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    out = np.zeros((M, K // 256 * 292), np.uint8)
    _check(lib().oracle_quantize_q8k(_p(x), M, K, K, _p(out)), "quantize_q8k")
    return out


def dequant_q8k(xq, M: int, K: int) -> np.ndarray:
    xq = _u8(xq)
    out = np.zeros((M, K), np.float64)
    _check(lib().oracle_dequant_q8k(_p(xq), M, K, _p(out)), "dequant_q8k")
    return out


def gemm(qtype: int, w, N: int, K: int, xq, M: int, nthreads: int | None = None, bias=None) -> np.ndarray:
    """f64 y [M, N] = W_hat X_hat^T, plus the f32 bias [N] of every row when
    given (the Q, K, V projections of Dream-7B, README milestones: "QKV
    bias"), added in f64."""
    w = _u8(w); xq = _u8(xq)
    y = np.zeros((M, N), np.float64)
    nt = nthreads or default_threads()
    _check(lib().oracle_gemm(qtype, _p(w), N, K, _p(xq), M, _p(y), nt), "gemm")
    if bias is not None:
        y += np.asarray(bias, np.float32).astype(np.float64)[None, :N]
    return y


def gemm_sample(qtype: int, w, N: int, K: int, xq, M: int, mi, ni, bias=None) -> np.ndarray:
    """f64 y[mi[t], ni[t]] for each t (plus bias[ni[t]] when given)."""
    w = _u8(w); xq = _u8(xq)
    mi = np.ascontiguousarray(mi, np.int64); ni = np.ascontiguousarray(ni, np.int64)
    out = np.zeros(mi.size, np.float64)
    _check(lib().oracle_gemm_sample(qtype, _p(w), N, K, _p(xq), M, _p(mi), _p(ni),
                                    mi.size, _p(out)), "gemm_sample")
    if bias is not None:
        out += np.asarray(bias, np.float32).astype(np.float64)[ni]
    return out


def partials(qtype: int, w, N: int, K: int, xq, M: int) -> np.ndarray:
    """int32 P [M, N, K/256, 16] of per-16 unsigned-quant x int8 dots."""
    w = _u8(w); xq = _u8(xq)
    P = np.zeros((M, N, K // 256, 16), np.int32)
    _check(lib().oracle_partials(qtype, _p(w), N, K, _p(xq), M, _p(P)), "partials")
    return P


def lmhead(qtype: int, w, N: int, K: int, h: np.ndarray, rows, nthreads: int | None = None):
    """(f64 logits [n_rows, N], int32 argmax [n_rows]) for the gathered rows."""
    w = _u8(w)
    h = np.ascontiguousarray(h, np.float32)
    M = h.shape[0]
    rows = np.ascontiguousarray(rows, np.int32)
    n = rows.size
    logits = np.zeros((n, N), np.float64)
    am = np.zeros(n, np.int32)
    nt = nthreads or default_threads()
    _check(lib().oracle_lmhead(qtype, _p(w), N, K, _p(h), M, h.shape[1], _p(rows), n,
                               _p(logits), _p(am), nt), "lmhead")
    return logits, am


def softmax_stats(logits: np.ndarray):
    """(f64 log-sum-exp [n_rows], f64 softmax probability of the argmax
    [n_rows]) of each row of f64 logits: the greedy pick's confidence."""
    lg = np.ascontiguousarray(logits, np.float64)
    if lg.ndim == 1:
        lg = lg[None, :]
    n, N = lg.shape
    lse = np.zeros(n, np.float64)
    p = np.zeros(n, np.float64)
    _check(lib().oracle_softmax_stats(_p(lg), n, N, _p(lse), _p(p)), "softmax_stats")
    return lse, p


def rmsnorm_quantize_q8k(x: np.ndarray, g: np.ndarray, eps: float):
    """(Q8_K records uint8 [M, K/256*292], f32 dmax [M]) of RMSNorm(x) with
    norm weight g: the codes of f32(x*g), each block's d times the row's
    f32 factor 1/sqrt(mean(x^2) + eps)."""
    x = np.ascontiguousarray(x, np.float32)
    g = np.ascontiguousarray(g, np.float32)
    M, K = x.shape
    out = np.zeros((M, K // 256 * 292), np.uint8)
    dmax = np.zeros(M, np.float32)
    _check(lib().oracle_rmsnorm_quantize_q8k(_p(x), M, K, K, _p(g), float(eps), _p(out), _p(dmax)),
           "rmsnorm_quantize_q8k")
    return out, dmax


def swiglu_quantize_q8k(gu: np.ndarray):
    """(Q8_K records uint8 [M, F/256*292], f32 dmax [M]) of silu(gate) * up,
    gate = gu[:, :F], up = gu[:, F:], evaluated in f64 and rounded once to
    f32 before quantizing."""
    gu = np.ascontiguousarray(gu, np.float32)
    M, F2 = gu.shape
    F = F2 // 2
    out = np.zeros((M, F // 256 * 292), np.uint8)
    dmax = np.zeros(M, np.float32)
    _check(lib().oracle_swiglu_quantize_q8k(_p(gu), M, F, F2, _p(out), _p(dmax)), "swiglu_quantize_q8k")
    return out, dmax


def f16_round(x: float) -> float:
    """The nearest binary16 value of an f32 (ties to even), as a float."""
    return lib().oracle_f16_round(float(x))


def attention(qkv: np.ndarray, H: int, D: int, scale: float, Hkv: int | None = None) -> np.ndarray:
    """f64 [L, H*D]: bidirectional softmax attention per head over f16-rounded
    Q, K, V taken from the rows of qkv (Q of H heads | K of Hkv heads | V of
    Hkv heads, D values per head; Hkv = H unless given).  Query head h reads
    key/value head h // (H // Hkv)."""
    Hkv = H if Hkv is None else Hkv
    qkv = np.ascontiguousarray(qkv, np.float32)
    L, ld = qkv.shape
    out = np.zeros((L, H * D), np.float64)
    _check(lib().oracle_attention(_p(qkv), L, ld, H, Hkv, D, float(scale), _p(out)), "attention")
    return out
