"""Seeded synthetic inputs for the quantized GEMM stream.

This module only draws random numbers and places them in the byte fields of
GGUF super-blocks; it holds none of the method's arithmetic (no decoding, no
quantization, no dot products).  Both the CPU oracle and the GPU path are fed
from here, so the two sides always see the same bytes.

Stand-in for the model weights and prompts of the mojo-dllm pages
("Benchmarks": LLaDA-8B-Instruct Q4_K_M), which are not available here:

* Q4_K rows (144-byte super-blocks of 256 weights): every byte uniform, so the
  6-bit scales/mins are uniform on 0..63 and the 4-bit quants uniform on 0..15;
  the two f16 fields d, dmin are then overwritten with U(1e-3, 1e-2) rounded
  to f16.
* Q6_K rows (210-byte super-blocks): low/high quant bytes uniform (6-bit quants
  uniform on 0..63), the 16 int8 sub-block scales uniform on -64..63, and the
  f16 d at the end drawn U(1e-3, 1e-2).
* Activations / hidden states: f32 N(0, 1).

Edge-case variants (for parity over the whole range the formats allow):
Q6_K scales over all of -128..127, and Q4_K d / dmin log-uniform over many
decades, down into the f16 subnormals.

Every tensor is keyed by (seed, name): the name is hashed into the generator
seed, so any tensor can be regenerated on its own.  On a CUDA/HIP device the
bytes come from torch's device generator (fast, for multi-GB weight sets); on
the CPU from torch's CPU generator.  The two do not produce the same stream for
the same key -- a test generates once and hands the same tensor to both sides.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

QK_K = 256
Q4_K_BYTES = 144
Q6_K_BYTES = 210
Q8_K_BYTES = 292

# GGUF tensor-type ids, used as the qtype tag everywhere.
GGML_TYPE_Q4_K = 12
GGML_TYPE_Q6_K = 14
GGML_TYPE_Q8_K = 15


def key_seed(seed: int, name: str) -> int:
    """64-bit generator seed for tensor `name` under master seed `seed`."""
    h = hashlib.sha256(f"{int(seed)}/{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(key_seed(seed, name))
    return g


def _f16_bytes(vals_f32: torch.Tensor) -> torch.Tensor:
    """f32 values -> their f16 (round-to-nearest-even) bit patterns as bytes."""
    return vals_f32.to(torch.float16).contiguous().view(torch.uint8).view(-1, 2)


def _uniform_f16(n: int, lo: float, hi: float, g, device, log: bool = False) -> torch.Tensor:
    """n values U(lo, hi) -- or, with `log`, log-uniform on [lo, hi] -- as f16
    bit patterns (values below 2^-14 become f16 subnormals)."""
    if log:
        u = torch.rand(n, generator=g, device=device, dtype=torch.float64)
        return _f16_bytes(torch.exp(np.log(lo) + (np.log(hi) - np.log(lo)) * u).to(torch.float32))
    u = torch.rand(n, generator=g, device=device, dtype=torch.float32)
    return _f16_bytes(lo + (hi - lo) * u)


def q4k_rows(n_rows: int, K: int, seed: int, name: str, device="cpu",
             d_range=(1e-3, 1e-2), dmin_range=(1e-3, 1e-2), log: bool = False) -> torch.Tensor:
    """uint8 tensor [n_rows, K/256*144]: seeded random Q4_K super-blocks;
    `log` draws d and dmin log-uniform over their ranges instead."""
    assert K % QK_K == 0
    sb = K // QK_K
    g = _gen(seed, name, device)
    blk = torch.randint(0, 256, (n_rows * sb, Q4_K_BYTES), generator=g,
                        device=device, dtype=torch.uint8)
    nb = n_rows * sb
    blk[:, 0:2] = _uniform_f16(nb, *d_range, g, device, log)
    blk[:, 2:4] = _uniform_f16(nb, *dmin_range, g, device, log)
    return blk.view(n_rows, sb * Q4_K_BYTES)


def q6k_rows(n_rows: int, K: int, seed: int, name: str, device="cpu",
             d_range=(1e-3, 1e-2), scale_range=(-64, 63)) -> torch.Tensor:
    """uint8 tensor [n_rows, K/256*210]: seeded random Q6_K super-blocks."""
    assert K % QK_K == 0
    sb = K // QK_K
    g = _gen(seed, name, device)
    nb = n_rows * sb
    blk = torch.randint(0, 256, (nb, Q6_K_BYTES), generator=g,
                        device=device, dtype=torch.uint8)
    lo, hi = scale_range
    sc = torch.randint(lo, hi + 1, (nb, 16), generator=g, device=device,
                       dtype=torch.int16)
    blk[:, 192:208] = sc.to(torch.int8).view(torch.uint8)
    blk[:, 208:210] = _uniform_f16(nb, *d_range, g, device)
    return blk.view(n_rows, sb * Q6_K_BYTES)


def q6k_rows_full_range(n_rows: int, K: int, seed: int, name: str) -> torch.Tensor:
    """Q6_K rows (CPU) with scales uniform on all of -128..127; in every row
    the first block has the extremes -128 and 127 planted (alternating), the
    second (when there is one) only scales in 64..127 and the third only
    -128..-65."""
    w = q6k_rows(n_rows, K, seed, name, scale_range=(-128, 127))
    blk = w.view(n_rows, K // QK_K, Q6_K_BYTES)
    sc = blk[:, :, 192:208].view(torch.int8)
    sc[:, 0, :] = torch.tensor([-128, 127] * 8, dtype=torch.int8)
    g = _gen(seed, name + "/planted", "cpu")
    if K // QK_K > 1:
        sc[:, 1, :] = torch.randint(64, 128, (n_rows, 16), generator=g).to(torch.int8)
    if K // QK_K > 2:
        sc[:, 2, :] = torch.randint(-128, -64, (n_rows, 16), generator=g).to(torch.int8)
    return w


def qk_rows(qtype: int, n_rows: int, K: int, seed: int, name: str, device="cpu"):
    if qtype == GGML_TYPE_Q4_K:
        return q4k_rows(n_rows, K, seed, name, device)
    if qtype == GGML_TYPE_Q6_K:
        return q6k_rows(n_rows, K, seed, name, device)
    raise ValueError(f"no generator for qtype {qtype}")


def normal_f32(shape, seed: int, name: str, device="cpu") -> torch.Tensor:
    """f32 N(0,1) tensor of `shape`."""
    g = _gen(seed, name, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def distinct_rows(n_rows: int, M: int, seed: int, name: str) -> torch.Tensor:
    """`n_rows` distinct row indices in [0, M), int32, CPU, in random order."""
    g = _gen(seed, name, "cpu")
    return torch.randperm(M, generator=g)[:n_rows].to(torch.int32)


def row_bytes(qtype: int, K: int) -> int:
    per = {GGML_TYPE_Q4_K: Q4_K_BYTES, GGML_TYPE_Q6_K: Q6_K_BYTES,
           GGML_TYPE_Q8_K: Q8_K_BYTES}[qtype]
    return K // QK_K * per
