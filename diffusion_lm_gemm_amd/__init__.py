"""Python binding of libdllm: the per-denoising-step quantized GEMM stream of a
diffusion LM as hand-written HIP kernels for MI355X (gfx950).

Argument marshalling only: every step of the path runs in libdllm's kernels.
PyTorch supplies device memory and the current stream.  The functions keep
the C-ABI names without the ``dllm_`` prefix.  If libdllm.so is missing this
module raises on import; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

Q4_K = 12
Q6_K = 14
Q8_K = 15
QK_K = 256
Q4_K_BYTES = 144
Q6_K_BYTES = 210
Q8_K_BYTES = 292
DECODED_BYTES = 356

E_ARG, E_SHAPE, E_UNSUPPORTED, E_ALIGN, E_HIP, E_WORKSPACE = -1, -2, -3, -4, -5, -6

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdllm.so")

HEADER_EXPORTS = (
    "dllm_abi_version", "dllm_last_error", "dllm_quantize_q8k", "dllm_rmsnorm_quantize_q8k",
    "dllm_swiglu_quantize_q8k", "dllm_attention", "dllm_decode_qk",
    "dllm_qgemm_workspace_bytes", "dllm_qgemm", "dllm_qgemm_bias", "dllm_lmhead_workspace_bytes",
    "dllm_lmhead_masked", "dllm_lmhead_confidence", "dllm_qgemm_partials_i32",
    "dllm_qgemm_superblock_sums_i32", "dllm_qgemm_planned", "dllm_lmhead_planned", "dllm_qgemm_noalloc",
    "dllm_qgemm_pair_workspace_bytes", "dllm_qgemm_pair",
)

# tile configurations of dllm_qgemm_planned and the super-block sums export
TILE_CONFIGS = (1, 2, 3, 4, 5, 6, 7)


class DllmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libdllm error {code}: {message}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run diffusion_lm_gemm_amd/build.py "
                          "(or __graft_entry__.build()) first -- there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "dllm_abi_version": (I, []),
        "dllm_last_error": (ctypes.c_char_p, []),
        "dllm_quantize_q8k": (I, [P, I64, I64, I64, P, P, P]),
        "dllm_rmsnorm_quantize_q8k": (I, [P, I64, I64, I64, P, ctypes.c_float, P, P, P]),
        "dllm_swiglu_quantize_q8k": (I, [P, I64, I64, I64, P, P, P]),
        "dllm_attention": (I, [P, I64, I64, I64, I64, I64, ctypes.c_float, P, I64, P]),
        "dllm_decode_qk": (I, [I, P, I64, P, P]),
        "dllm_qgemm_workspace_bytes": (I64, [I, I64, I64, I64]),
        "dllm_qgemm": (I, [I, P, I64, I64, P, P, I64, P, I64, P, I64, P]),
        "dllm_qgemm_bias": (I, [I, P, I64, I64, P, P, I64, P, P, I64, P, I64, P]),
        "dllm_lmhead_workspace_bytes": (I64, [I, I64, I64, I64]),
        "dllm_lmhead_masked": (I, [I, P, I64, I64, P, I64, I64, P, I64, P, I64, P, P, I64, P]),
        "dllm_lmhead_confidence": (I, [I, P, I64, I64, P, I64, I64, P, I64, P, I64, P, P, P, P, I64, P]),
        "dllm_qgemm_partials_i32": (I, [I, P, I64, I64, P, I64, P, P]),
        "dllm_qgemm_superblock_sums_i32": (I, [I, P, I64, I64, P, I64, P, I, I, P]),
        "dllm_qgemm_planned": (I, [I, P, I64, I64, P, P, I64, P, P, I64, P, I64, I, I, P]),
        "dllm_lmhead_planned": (I, [I, P, I64, I64, P, I64, I64, P, I64, P, I64, P, P, P, P, I64, I, P]),
        "dllm_qgemm_noalloc": (I, [I, P, I64, I64, P, P, I64, P, P, I64, P]),
        "dllm_qgemm_pair_workspace_bytes": (I64, [I, I64, I, I64, I64, I64]),
        "dllm_qgemm_pair": (I, [I, P, I64, P, P, I64, I, P, I64, P, P, I64, I64, P, P, I64, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


def last_error() -> str:
    return lib.dllm_last_error().decode()


def abi_version() -> int:
    return lib.dllm_abi_version()


def _check(rc: int):
    if rc != 0:
        raise DllmError(rc, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("libdllm takes device tensors only")
    return t.device


def block_bytes(qtype: int) -> int:
    return {Q4_K: Q4_K_BYTES, Q6_K: Q6_K_BYTES}.get(qtype, 0)


def quantize_q8k(x: torch.Tensor, out: torch.Tensor | None = None,
                 dmax: torch.Tensor | None = None) -> torch.Tensor:
    """f32 [M, K] (row stride = ldx) -> Q8_K records uint8 [M, K/256*292].
    `dmax` (f32 [M], optional) receives each token's largest |d|, which
    qgemm takes as `x_dmax`."""
    dev = _dev(x)
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K // QK_K * Q8_K_BYTES), dtype=torch.uint8, device=dev)
    if dmax is not None:
        assert dmax.dtype == torch.float32 and dmax.is_contiguous() and dmax.numel() >= M
    _check(lib.dllm_quantize_q8k(_ptr(x), M, K, x.stride(0), _ptr(out), _ptr(dmax), _stream(dev)))
    return out


def rmsnorm_quantize_q8k(x: torch.Tensor, g: torch.Tensor, eps: float = 1e-5,
                         out: torch.Tensor | None = None,
                         dmax: torch.Tensor | None = None) -> torch.Tensor:
    """RMSNorm(x) * g -> Q8_K records uint8 [M, K/256*292] without the f32
    intermediate: the codes of x * g, each block's d times the row's factor
    1/sqrt(mean(x^2) + eps)."""
    dev = _dev(x)
    assert x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    assert g.dtype == torch.float32 and g.is_contiguous()
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K // QK_K * Q8_K_BYTES), dtype=torch.uint8, device=dev)
    if dmax is not None:
        assert dmax.dtype == torch.float32 and dmax.is_contiguous() and dmax.numel() >= M
    _check(lib.dllm_rmsnorm_quantize_q8k(_ptr(x), M, K, x.stride(0), _ptr(g), float(eps), _ptr(out), _ptr(dmax),
                                         _stream(dev)))
    return out


def swiglu_quantize_q8k(gu: torch.Tensor, out: torch.Tensor | None = None,
                        dmax: torch.Tensor | None = None) -> torch.Tensor:
    """f32 [M, 2F] (gate | up) -> the Q8_K records [M, F/256*292] of
    silu(gate) * up, evaluated in f64 and rounded once to f32."""
    dev = _dev(gu)
    assert gu.dtype == torch.float32 and gu.dim() == 2 and gu.stride(1) == 1
    M, F2 = gu.shape
    F = F2 // 2
    if out is None:
        out = torch.empty((M, F // QK_K * Q8_K_BYTES), dtype=torch.uint8, device=dev)
    if dmax is not None:
        assert dmax.dtype == torch.float32 and dmax.is_contiguous() and dmax.numel() >= M
    _check(lib.dllm_swiglu_quantize_q8k(_ptr(gu), M, F, gu.stride(0), _ptr(out), _ptr(dmax), _stream(dev)))
    return out


def attention(qkv: torch.Tensor, H: int, D: int = 128, scale: float | None = None,
              out: torch.Tensor | None = None, H_kv: int | None = None) -> torch.Tensor:
    """Bidirectional attention per query head over the rows of qkv (Q of H
    heads | K of H_kv heads | V of H_kv heads, D values per head; H_kv = H
    unless given): f32 [L, H*D]."""
    dev = _dev(qkv)
    assert qkv.dtype == torch.float32 and qkv.dim() == 2 and qkv.stride(1) == 1
    L = qkv.shape[0]
    H_kv = H if H_kv is None else H_kv
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((L, H * D), dtype=torch.float32, device=dev)
    _check(lib.dllm_attention(_ptr(qkv), L, qkv.stride(0), H, H_kv, D, float(scale), _ptr(out), out.stride(0),
                              _stream(dev)))
    return out


def decode_qk(qtype: int, w: torch.Tensor, n_superblocks: int,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """Super-blocks -> shared decoded records uint8 [n_superblocks, 356]."""
    dev = _dev(w)
    if out is None:
        out = torch.empty((n_superblocks, DECODED_BYTES), dtype=torch.uint8, device=dev)
    _check(lib.dllm_decode_qk(qtype, _ptr(w), n_superblocks, _ptr(out), _stream(dev)))
    return out


def qgemm_workspace_bytes(qtype: int, N: int, K: int, M: int) -> int:
    return int(lib.dllm_qgemm_workspace_bytes(qtype, N, K, M))


def qgemm_workspace(qtype: int, N: int, K: int, M: int, device) -> torch.Tensor:
    """A workspace for dllm_qgemm's K split at this shape (at least 256
    bytes, zero-filled)."""
    nb = max(qgemm_workspace_bytes(qtype, N, K, M), 256)
    return torch.zeros(nb, dtype=torch.uint8, device=device)


def qgemm(qtype: int, w: torch.Tensor, N: int, K: int, x_q8k: torch.Tensor, M: int,
          y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
          x_dmax: torch.Tensor | None = None, bias: torch.Tensor | None = None) -> torch.Tensor:
    """y[M, N] (f32) = dequant(x_q8k) @ dequant(w)^T (+ bias[N], f32, through
    dllm_qgemm_bias when given).  `y` may be a row-strided view; `workspace`
    (uint8, >= qgemm_workspace_bytes) enables the K split; `x_dmax` (f32 [M],
    from quantize_q8k) spares the kernel its own scan."""
    dev = _dev(w)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    assert y.dtype == torch.float32 and y.stride(1) == 1
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if x_dmax is not None:
        assert x_dmax.dtype == torch.float32 and x_dmax.is_contiguous() and x_dmax.numel() >= M
    if bias is None:
        _check(lib.dllm_qgemm(qtype, _ptr(w), N, K, _ptr(x_q8k), _ptr(x_dmax), M, _ptr(y), y.stride(0),
                              _ptr(workspace), wsb, _stream(dev)))
    else:
        assert bias.dtype == torch.float32 and bias.is_contiguous() and bias.numel() >= N
        _check(lib.dllm_qgemm_bias(qtype, _ptr(w), N, K, _ptr(x_q8k), _ptr(x_dmax), M, _ptr(bias), _ptr(y),
                                   y.stride(0), _ptr(workspace), wsb, _stream(dev)))
    return y


def qgemm_pair_workspace_bytes(qtype_a: int, N_a: int, qtype_b: int, N_b: int, K: int, M: int) -> int:
    return int(lib.dllm_qgemm_pair_workspace_bytes(qtype_a, N_a, qtype_b, N_b, K, M))


def qgemm_pair(a: tuple, b: tuple, K: int, x_q8k: torch.Tensor, M: int,
               workspace: torch.Tensor | None = None, x_dmax: torch.Tensor | None = None):
    """Two GEMMs of one activation matrix in one call (dllm_qgemm_pair).
    a and b are (qtype, w, N, y, bias) with y (f32 [M, >= N], row-strided
    views allowed) and bias (f32 [N]) optional (None); returns (y_a, y_b)."""
    outs, args = [], []
    for qtype, w, N, y, bias in (a, b):
        dev = _dev(w)
        if y is None:
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
        assert y.dtype == torch.float32 and y.stride(1) == 1
        if bias is not None:
            assert bias.dtype == torch.float32 and bias.is_contiguous() and bias.numel() >= N
        outs.append(y)
        args += [qtype, _ptr(w), N, _ptr(bias), _ptr(y), y.stride(0)]
    if x_dmax is not None:
        assert x_dmax.dtype == torch.float32 and x_dmax.is_contiguous() and x_dmax.numel() >= M
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dllm_qgemm_pair(*args, K, _ptr(x_q8k), _ptr(x_dmax), M, _ptr(workspace), wsb, _stream(_dev(x_q8k))))
    return outs[0], outs[1]


def lmhead_workspace_bytes(qtype: int, N: int, K: int, n_rows: int) -> int:
    return int(lib.dllm_lmhead_workspace_bytes(qtype, N, K, n_rows))


def lmhead_masked(qtype: int, w: torch.Tensor, N: int, K: int, h: torch.Tensor,
                  rows: torch.Tensor, logits: torch.Tensor | None = None,
                  argmax: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """Gather rows of h, quantize to Q8_K, multiply by w: (f32 logits
    [n_rows, N], int32 argmax [n_rows])."""
    dev = _dev(w)
    assert h.dtype == torch.float32 and h.stride(1) == 1 and rows.dtype == torch.int32
    M = h.shape[0]
    n = rows.numel()
    if logits is None:
        logits = torch.empty((n, N), dtype=torch.float32, device=dev)
    if argmax is None:
        argmax = torch.empty(n, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(lmhead_workspace_bytes(qtype, N, K, n), 1),
                                dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib.dllm_lmhead_masked(qtype, _ptr(w), N, K, _ptr(h), M, h.stride(0), _ptr(rows), n,
                                  _ptr(logits), logits.stride(0), _ptr(argmax), _ptr(workspace),
                                  wsb, _stream(dev)))
    return logits, argmax


def lmhead_confidence(qtype: int, w: torch.Tensor, N: int, K: int, h: torch.Tensor,
                      rows: torch.Tensor, logits: torch.Tensor | None = None,
                      argmax: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      p_argmax: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """lmhead_masked plus the greedy pick's confidence: (f32 logits [n_rows,
    N], int32 argmax [n_rows], f32 log-sum-exp [n_rows], f32 softmax
    probability of the argmax [n_rows])."""
    dev = _dev(w)
    assert h.dtype == torch.float32 and h.stride(1) == 1 and rows.dtype == torch.int32
    M = h.shape[0]
    n = rows.numel()
    if logits is None:
        logits = torch.empty((n, N), dtype=torch.float32, device=dev)
    if argmax is None:
        argmax = torch.empty(n, dtype=torch.int32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    if p_argmax is None:
        p_argmax = torch.empty(n, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(lmhead_workspace_bytes(qtype, N, K, n), 1),
                                dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib.dllm_lmhead_confidence(qtype, _ptr(w), N, K, _ptr(h), M, h.stride(0), _ptr(rows), n,
                                      _ptr(logits), logits.stride(0), _ptr(argmax), _ptr(lse),
                                      _ptr(p_argmax), _ptr(workspace), wsb, _stream(dev)))
    return logits, argmax, lse, p_argmax


def qgemm_partials_i32(qtype: int, w: torch.Tensor, N: int, K: int, x_q8k: torch.Tensor,
                       M: int) -> torch.Tensor:
    """Test export: int32 [M, N, K/256, 16] per-16 partial dots."""
    dev = _dev(w)
    P = torch.empty((M, N, K // QK_K, 16), dtype=torch.int32, device=dev)
    _check(lib.dllm_qgemm_partials_i32(qtype, _ptr(w), N, K, _ptr(x_q8k), M, _ptr(P), _stream(dev)))
    return P


def qgemm_superblock_sums_i32(qtype: int, w: torch.Tensor, N: int, K: int, x_q8k: torch.Tensor,
                              M: int, tile: int, split: int = 1) -> torch.Tensor:
    """Test export: int32 [M, N, K/256], the exact integer super-block sums
    formed by the GEMM kernel of tile configuration `tile` (TILE_CONFIGS)
    with K split `split`."""
    dev = _dev(w)
    A = torch.empty((M, N, K // QK_K), dtype=torch.int32, device=dev)
    _check(lib.dllm_qgemm_superblock_sums_i32(qtype, _ptr(w), N, K, _ptr(x_q8k), M, _ptr(A), tile, split,
                                              _stream(dev)))
    return A


def qgemm_planned(qtype: int, w: torch.Tensor, N: int, K: int, x_q8k: torch.Tensor, M: int,
                  tile: int, split: int = 1, y: torch.Tensor | None = None,
                  x_dmax: torch.Tensor | None = None, bias: torch.Tensor | None = None) -> torch.Tensor:
    """Test entry: qgemm with an explicit tile configuration (TILE_CONFIGS)
    and K split; allocates the split's workspace."""
    dev = _dev(w)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    assert y.dtype == torch.float32 and y.stride(1) == 1
    # the tile counters (64 KiB), then the partial slices; zero-filled
    ws = torch.zeros(65536 + split * M * ((N + 63) // 64 * 64) * 4, dtype=torch.uint8, device=dev)
    _check(lib.dllm_qgemm_planned(qtype, _ptr(w), N, K, _ptr(x_q8k), _ptr(x_dmax), M, _ptr(bias), _ptr(y),
                                  y.stride(0), _ptr(ws), ws.numel(), tile, split, _stream(dev)))
    return y


def lmhead_planned(qtype: int, w: torch.Tensor, N: int, K: int, h: torch.Tensor, rows: torch.Tensor,
                   path: int, confidence: bool = True, logits: torch.Tensor | None = None):
    """Test entry: the LM head on a given path (0 choose, 1 streaming, 2
    tiled): (logits, argmax, lse, p_argmax), the last two None without
    `confidence`.  `logits` (f32 [n_rows, >= N] rows, unit column stride) may
    be given."""
    dev = _dev(w)
    assert h.dtype == torch.float32 and h.stride(1) == 1 and rows.dtype == torch.int32
    M = h.shape[0]
    n = rows.numel()
    if logits is None:
        logits = torch.empty((n, N), dtype=torch.float32, device=dev)
    assert logits.dtype == torch.float32 and logits.stride(1) == 1
    argmax = torch.empty(n, dtype=torch.int32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if confidence else None
    p_am = torch.empty(n, dtype=torch.float32, device=dev) if confidence else None
    workspace = torch.empty(max(lmhead_workspace_bytes(qtype, N, K, n), 1), dtype=torch.uint8, device=dev)
    _check(lib.dllm_lmhead_planned(qtype, _ptr(w), N, K, _ptr(h), M, h.stride(0), _ptr(rows), n,
                                   _ptr(logits), logits.stride(0), _ptr(argmax), _ptr(lse), _ptr(p_am),
                                   _ptr(workspace), workspace.numel(), path, _stream(dev)))
    return logits, argmax, lse, p_am
