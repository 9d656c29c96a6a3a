"""GPU parity on the edges of the weight formats, and the GEMM kernels' own
exact integer sums.

* Q6_K sub-block scales over all of -128..127 (GGUF stores them as int8; the
  generic draws stay in -64..63): blocks with planted -128 and 127, and blocks
  whose every scale lies in 64..127 or -128..-65, through every tile
  configuration of the GEMM and both LM-head paths.
* Q4_K d and dmin log-uniform over 1e-7..1e-1, so that about half of them are
  f16 subnormals (below 2^-14) and rows mix tiny and ordinary blocks; and
  matrices whose every d and dmin is tiny, where the whole output is tiny and
  the bound shrinks with it.
* The exact int32 super-block sums A_sb = (hi << shift) + lo that each tile
  configuration forms on the matrix cores, bit-exact against the oracle's
  per-16 partial dots combined with the blocks' integer scales (mojo-dllm
  Development plan, "Compute design": the per-16 integer scale form).
* A token's output does not depend on how many tokens share its work-group
  (the token tile): bit-identical between a small and the largest tile.
Bars as in test_gpu_parity: f32 outputs within 1e-4 * (|oracle| + rms(row))
and below 5% of that bound; integers bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _check_argmax, _check_confidence, _say, assert_close_rows

pytestmark = pytest.mark.gpu

TILES = (1, 2, 3, 4, 5, 6, 7)


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


# ------------------------------------------------------------ weights ----
def q6k_full_range(N: int, K: int, seed: int, name: str) -> torch.Tensor:
    return synth.q6k_rows_full_range(N, K, seed, name)


def q4k_log_scales(N: int, K: int, seed: int, name: str, lo: float = 1e-7, hi: float = 1e-1) -> torch.Tensor:
    return synth.q4k_rows(N, K, seed, name, d_range=(lo, hi), dmin_range=(lo, hi), log=True)


# ------------------------------------------------- exact integer sums ----
def superblock_sums_ref(qtype: int, w: np.ndarray, N: int, K: int, xq: np.ndarray, M: int) -> np.ndarray:
    """int64 A[m][n][sb] from the oracle's per-16 partials P_g = sum u q and
    the blocks' integer scales:
      Q4_K: sum_j sc_j (P_2j + P_2j+1)
      Q6_K: sum_g sc_g (P_g - 32 * sum_t q_t)   (the quants u - 32)."""
    SB = K // 256
    P = oracle.partials(qtype, w, N, K, xq, M).astype(np.int64)  # [M, N, SB, 16]
    bpb = 144 if qtype == 12 else 210
    blocks = w.reshape(N * SB, bpb)
    if qtype == 12:
        sc = np.stack([oracle.q4k_fields(blocks[i])[2] for i in range(N * SB)]).reshape(N, SB, 8).astype(np.int64)
        return (P.reshape(M, N, SB, 8, 2).sum(axis=4) * sc[None]).sum(axis=3)
    sc = np.stack([oracle.q6k_fields(blocks[i])[1] for i in range(N * SB)]).reshape(N, SB, 16).astype(np.int64)
    q = xq.reshape(M, SB, 292)[:, :, 4:260].copy().view(np.int8).astype(np.int64)  # [M, SB, 256]
    qsum = q.reshape(M, SB, 16, 16).sum(axis=3)  # [M, SB, 16]
    return ((P - 32 * qsum[:, None]) * sc[None]).sum(axis=3)


@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("tile", TILES)
def test_superblock_sums_every_tile_bitexact(dl, qtype, tile):
    """The kernels' own exact int32 super-block sums, every tile
    configuration, unsplit and with a K split whose last slice is short, on
    ragged rows and more tokens than one token tile (170); Q6_K with
    full-range scales."""
    N, K, M = 130, 1280, 170
    _say(f"superblock sums qtype={qtype} tile={tile}")
    w = q6k_full_range(N, K, 5, "sums") if qtype == 14 else synth.q4k_rows(N, K, 5, "sums")
    x = synth.normal_f32((M, K), 5, "sums-x")
    xq = oracle.quantize_q8k(x.numpy())
    ref = superblock_sums_ref(qtype, w.numpy(), N, K, xq, M)
    assert np.abs(ref).max() < 2 ** 31
    wd, xd = w.to(DEV), torch.from_numpy(xq).to(DEV)
    for split in (1, 2):
        got = dl.qgemm_superblock_sums_i32(qtype, wd, N, K, xd, M, tile=tile, split=split).cpu().numpy()
        assert np.array_equal(got.astype(np.int64), ref), f"tile {tile} split {split}"


def test_superblock_sums_extreme_planes(dl):
    """Q6_K sums at the planes' extremes: every scale -128 with every quant 0
    (s (q - 32) = 4096 = 128 * 32) and every activation quant -127 or 127."""
    N, K, M = 64, 512, 16
    w = synth.q6k_rows(N, K, 6, "extreme")
    blk = w.view(N, K // 256, 210)
    blk[:, :, :192] = 0  # q = 0 everywhere
    blk[:, :, 192:208] = torch.tensor([-128] * 16, dtype=torch.int8).view(torch.uint8)
    x = torch.where(synth.normal_f32((M, K), 6, "extreme-x") > 0, 1.0, -1.0).float()
    xq = oracle.quantize_q8k(x.numpy())
    assert set(np.unique(xq.reshape(M, K // 256, 292)[:, :, 4:260].view(np.int8))) <= {-127, 127}
    ref = superblock_sums_ref(14, w.numpy(), N, K, xq, M)
    for tile in (1, 3):
        got = dl.qgemm_superblock_sums_i32(14, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, tile=tile)
        assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


# ----------------------------------------------------- GEMM on the edges ----
@pytest.mark.parametrize("tile", TILES)
def test_qgemm_q6k_full_scale_range_every_tile(dl, tile):
    N, K, M = 200, 2048, 150
    _say(f"q6k full-range scales tile={tile}")
    w = q6k_full_range(N, K, 7, "q6-range")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 7, "q6-range-x").numpy())
    ref = oracle.gemm(14, w.numpy(), N, K, xq, M)
    wd, xd = w.to(DEV), torch.from_numpy(xq).to(DEV)
    for split in (1, 3):
        y = dl.qgemm_planned(14, wd, N, K, xd, M, tile=tile, split=split).cpu().numpy()
        assert_close_rows(y, ref, f"q6k full range tile={tile} split={split}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("lo,hi", [(1e-7, 1e-1), (1e-7, 1e-5)])
def test_qgemm_q4k_log_scales_every_tile(dl, tile, lo, hi):
    """d and dmin log-uniform on [lo, hi]: mixed within rows (1e-7..1e-1),
    and every block tiny (1e-7..1e-5, mostly f16 subnormals), where the
    whole output is tiny."""
    N, K, M = 200, 2048, 150
    _say(f"q4k log scales [{lo}, {hi}] tile={tile}")
    w = q4k_log_scales(N, K, 8, f"q4-log-{lo}-{hi}", lo, hi)
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 8, "q4-log-x").numpy())
    ref = oracle.gemm(12, w.numpy(), N, K, xq, M)
    wd, xd = w.to(DEV), torch.from_numpy(xq).to(DEV)
    for split in (1, 3):
        y = dl.qgemm_planned(12, wd, N, K, xd, M, tile=tile, split=split).cpu().numpy()
        assert_close_rows(y, ref, f"q4k log scales [{lo}, {hi}] tile={tile} split={split}")


def test_qgemm_edges_through_the_planner(dl):
    """The product entry (its own plan and K split) on both edge cases at a
    step shape (4096 x 4096, L = 148): whole oracle rows of four tokens."""
    N, K, M = 4096, 4096, 148
    toks = [0, 70, 100, 147]
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 9, "edge-step-x").numpy())
    xd = torch.from_numpy(xq).to(DEV)
    for qtype, w in ((14, q6k_full_range(N, K, 9, "edge-step-q6")), (12, q4k_log_scales(N, K, 9, "edge-step-q4"))):
        _say(f"planner edge case qtype={qtype}")
        ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
        y = dl.qgemm(qtype, w.to(DEV), N, K, xd, M, workspace=ws).cpu().numpy()
        ref = oracle.gemm(qtype, w.numpy(), N, K, xq[toks], len(toks))
        assert_close_rows(y[toks], ref, f"planner edge qtype={qtype}")


# -------------------------------------------------- LM head on the edges ----
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("case", ["q6k-range", "q4k-log", "q4k-tiny"])
def test_lmhead_edges_both_paths(dl, path, case):
    """Both LM-head paths (1 streaming, 2 tiled with the argmax epilogue) on
    the edge-case weights: logits, argmax and confidence against the oracle."""
    N, K, M, n_rows = 1000, 2048, 148, 13
    _say(f"lmhead edges case={case} path={path}")
    if case == "q6k-range":
        qtype, w = 14, q6k_full_range(N, K, 10, "lm-q6-range")
    elif case == "q4k-log":
        qtype, w = 12, q4k_log_scales(N, K, 10, "lm-q4-log")
    else:
        qtype, w = 12, q4k_log_scales(N, K, 10, "lm-q4-tiny", 1e-7, 1e-5)
    h = synth.normal_f32((M, K), 10, "lm-edge-h")
    rows = synth.distinct_rows(n_rows, M, 10, "lm-edge-rows")
    ref, ref_am = oracle.lmhead(qtype, w.numpy(), N, K, h.numpy(), rows.numpy())
    lg, am, lse, p = dl.lmhead_planned(qtype, w.to(DEV), N, K, h.to(DEV), rows.to(DEV), path=path)
    lg = lg.cpu().numpy()
    assert_close_rows(lg, ref, f"lmhead {case} path={path}")
    _check_argmax(lg, am.cpu().numpy(), ref, ref_am, f"lmhead {case} path={path}")
    _check_confidence(lg, lse.cpu().numpy().astype(np.float64), p.cpu().numpy().astype(np.float64), ref,
                      f"lmhead {case} path={path}")


# --------------------------------------------- token tile independence ----
@pytest.mark.parametrize("q,tile", [(12, 5), (12, 1), (12, 6), (14, 5), (14, 2)])
def test_token_tile_does_not_change_y(dl, q, tile):
    """37 tokens (a token tile of 3 x 16) give bit for bit the same y as the
    same 37 rows of a 160-token call (the configuration's largest tile):
    every instantiation forms and splits the same f32 values (Q4_K's min
    term in f16 halves, the per-super-block fma), unsplit and with a K
    split; activations over six decades of scale."""
    N, K, M = 333, 3072, 37
    _say(f"token tile independence q={q} tile={tile}")
    w = synth.qk_rows(q, N, K, 74, f"tt-{q}").to(DEV)
    x = synth.normal_f32((M, K), 74, "tt-x").to(DEV) * torch.logspace(-3, 3, M, device=DEV).unsqueeze(1)
    xp = torch.zeros((160, K), device=DEV)
    xp[:M] = x
    dm, dmp = torch.empty(M, device=DEV), torch.empty(160, device=DEV)
    xq, xqp = dl.quantize_q8k(x, dmax=dm), dl.quantize_q8k(xp, dmax=dmp)
    for split in (1, 3):
        a = dl.qgemm_planned(q, w, N, K, xq, M, tile=tile, split=split, x_dmax=dm)
        b = dl.qgemm_planned(q, w, N, K, xqp, 160, tile=tile, split=split, x_dmax=dmp)[:M]
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"split {split}"
