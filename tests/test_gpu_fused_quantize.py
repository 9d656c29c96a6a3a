"""Quantize and multiply in one launch (dllm_quantize_qgemm): the Q8_K records
and per-token largest |d| it writes are bit-identical to dllm_quantize_q8k's,
and its y to dllm_qgemm's (or the planned form's) on those records, for the
step's shapes, ragged shapes, every tile configuration, split and unsplit;
one workspace serves calls of different shapes and graph replays (its
counters come back to zero, its error word stays clear); whole rows match the
oracle.  (Development plan, "Compute design": every GEMM of a step is a
quantize + GEMM pair.)"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _say, _weights, assert_close_rows

pytestmark = pytest.mark.gpu

ERR_OFF = 57344


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


def _separate(dl, q, w, N, K, x, bias=None, tile=0, split=1):
    M = x.shape[0]
    dm = torch.empty(M, device=DEV)
    xq = dl.quantize_q8k(x, dmax=dm)
    if tile:
        y = dl.qgemm_planned(q, w, N, K, xq, M, tile=tile, split=split, x_dmax=dm, bias=bias)
    else:
        y = dl.qgemm(q, w, N, K, xq, M, workspace=dl.qgemm_workspace(q, N, K, M, DEV), x_dmax=dm, bias=bias)
    return y, xq, dm


CASES = [(12, 4096, 4096, 148, False), (12, 24576, 4096, 148, False), (14, 4096, 12288, 148, False),
         (12, 8192, 4096, 160, True), (14, 4096, 4096, 148, False), (12, 4096, 12288, 160, False),
         (12, 333, 3072, 37, True), (14, 200, 1024, 5, False), (12, 130, 512, 161, False)]


@pytest.mark.parametrize("q,N,K,M,with_bias", CASES)
def test_fused_equals_quantize_then_gemm(dl, q, N, K, M, with_bias):
    _say(f"fused quantize+gemm q={q} {N}x{K} M={M} bias={with_bias}")
    w = _weights(q, N, K, 71, f"fq-{q}-{N}-{K}").to(DEV)
    x = synth.normal_f32((M, K), 71, f"fq-x-{K}-{M}").to(DEV) * torch.logspace(-3, 3, M, device=DEV).unsqueeze(1)
    bias = synth.normal_f32((N,), 71, f"fq-b-{N}").to(DEV) if with_bias else None
    ws = dl.quantize_qgemm_workspace(q, N, K, M, DEV)
    y, xq, dm = dl.quantize_qgemm(q, w, N, K, x, ws, bias=bias)
    y2, xq2, dm2 = _separate(dl, q, w, N, K, x, bias)
    torch.cuda.synchronize()
    assert torch.equal(xq, xq2), "Q8_K records"
    assert torch.equal(dm, dm2), "largest |d| per token"
    assert torch.equal(y, y2), "y"
    assert int(ws[ERR_OFF:ERR_OFF + 4].view(torch.int32)[0]) == 0
    assert int(torch.count_nonzero(ws[:65536])) == 0, "counters back at zero"
    toks = [0, M // 2, M - 1]
    ref = oracle.gemm(q, w.cpu().numpy(), N, K, xq.cpu().numpy()[toks], len(toks),
                      bias=None if bias is None else bias.cpu().numpy())
    assert_close_rows(y.cpu().numpy()[toks], ref, f"fused {q} {N}x{K} M={M}")


@pytest.mark.parametrize("q", [12, 14])
@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5, 6, 7])
def test_fused_every_tile_configuration(dl, q, tile):
    N, K, M = 333, 2048, 150
    _say(f"fused planned q={q} tile={tile}")
    w = _weights(q, N, K, 72, f"fqt-{q}").to(DEV)
    x = synth.normal_f32((M, K), 72, "fqt-x").to(DEV)
    ws = torch.zeros(65536 + 3 * M * 384 * 4, dtype=torch.uint8, device=DEV)
    for split in (1, 3):
        y, xq, dm = dl.quantize_qgemm(q, w, N, K, x, ws, tile=tile, split=split)
        y2, xq2, dm2 = _separate(dl, q, w, N, K, x, tile=tile, split=split)
        torch.cuda.synchronize()
        assert torch.equal(xq, xq2) and torch.equal(dm, dm2)
        assert torch.equal(y, y2), f"tile {tile} split {split}"
    assert int(torch.count_nonzero(ws[:65536])) == 0


def test_fused_shared_workspace_and_graph_replays(dl):
    """One workspace for calls of three shapes in stream order, captured in a
    graph and replayed three times with eager work between the replays:
    every replay equals the eager result."""
    M = 148
    shapes = [(12, 4096, 4096), (14, 4096, 12288), (12, 12288, 4096)]
    nb = max(dl.lib.dllm_quantize_qgemm_workspace_bytes(q, N, K, M) for q, N, K in shapes)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    ops = []
    for i, (q, N, K) in enumerate(shapes):
        w = _weights(q, N, K, 73, f"fqg-{q}-{N}-{K}").to(DEV)
        x = synth.normal_f32((M, K), 73, f"fqg-x-{K}").to(DEV)
        y = torch.empty((M, N), device=DEV)
        xq = torch.empty((M, K // 256 * 292), dtype=torch.uint8, device=DEV)
        dm = torch.empty(M, device=DEV)
        ops.append((lambda q=q, w=w, N=N, K=K, x=x, y=y, xq=xq, dm=dm:
                    dl.quantize_qgemm(q, w, N, K, x, ws, y=y, x_q8k=xq, x_dmax=dm), y))
    for fn, _ in ops:
        fn()
    torch.cuda.synchronize()
    eager = [y.clone() for _, y in ops]
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for fn, _ in ops:
                fn()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    for rep in range(3):
        for _, y in ops:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (_, y) in enumerate(ops):
            assert torch.equal(y, eager[i]), f"replay {rep} call {i}"
        ops[rep % 3][0]()  # eager work between the replays
        torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:65536])) == 0


@pytest.mark.parametrize("q,tile", [(12, 5), (12, 1), (12, 6), (14, 5), (14, 2)])
def test_token_tile_does_not_change_y(dl, q, tile):
    """A token's y does not depend on how many tokens share its work-group:
    37 tokens (a small token tile) equal the same 37 rows of a 160-token call
    (the largest), bit for bit.  The fused entry always runs the largest
    token tile, so this is what makes it agree with the separate kernels."""
    N, K, M = 333, 3072, 37
    _say(f"token tile independence q={q} tile={tile}")
    w = _weights(q, N, K, 74, f"tt-{q}").to(DEV)
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
