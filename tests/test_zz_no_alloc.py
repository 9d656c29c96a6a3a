"""dllm_qgemm_noalloc (for callers that cannot allocate): the same bits as
dllm_qgemm_bias with its own workspace, through the C ABI, on two calls in a
row whose second is smaller, with and without a bias; and the shape limit of
its scratch is checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

DEV = "cuda:0"
SCRATCH = 24 << 20


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    return dl


def _noalloc(dl, q, w, N, K, xq, dm, M, bias, y):
    return dl.lib.dllm_qgemm_noalloc(q, dl._ptr(w), N, K, dl._ptr(xq), dl._ptr(dm), M, dl._ptr(bias), dl._ptr(y),
                                     y.stride(0), dl._stream(torch.device(DEV)))


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry(dl):
    assert torch.cuda.is_available()
    cases = [(12, 4096, 4096, 148, True), (14, 2048, 3072, 37, False), (14, 4096, 12288, 160, True)]
    for i, (q, N, K, M, with_bias) in enumerate(cases):
        print(f"noalloc call {i}: qtype={q} N={N} K={K} M={M} bias={with_bias}", flush=True)
        nb = dl.qgemm_workspace_bytes(q, N, K, M)
        assert 0 < nb <= SCRATCH, "the case must take the K split and fit the scratch"
        w = synth.qk_rows(q, N, K, 61, f"na-{q}-{N}-{K}").to(DEV)
        x = synth.normal_f32((M, K), 61, f"na-x-{K}-{M}").to(DEV)
        dm = torch.empty(M, device=DEV)
        xq = dl.quantize_q8k(x, dmax=dm)
        bias = synth.normal_f32((N,), 61, f"na-b-{N}").to(DEV) if with_bias else None
        ref = dl.qgemm(q, w, N, K, xq, M, workspace=dl.qgemm_workspace(q, N, K, M, DEV), x_dmax=dm, bias=bias)
        y = torch.full((M, N + 4), 3.0, device=DEV)
        assert _noalloc(dl, q, w, N, K, xq, dm, M, bias, y[:, :N]) == 0, dl.last_error()
        torch.cuda.synchronize()
        assert torch.equal(y[:, :N], ref), f"call {i}"
        assert torch.all(y[:, N:] == 3.0)
        # and against the oracle on a few whole rows
        toks = [0, M // 2, M - 1]
        xr = xq.cpu().numpy()
        want = oracle.gemm(q, w.cpu().numpy(), N, K, xr[toks], len(toks),
                           bias=None if bias is None else bias.cpu().numpy())
        got = y[:, :N].cpu().numpy()[toks].astype(np.float64)
        rms = np.sqrt(np.mean(want ** 2, axis=1, keepdims=True))
        assert np.all(np.abs(got - want) <= 1e-4 * (np.abs(want) + rms))


def test_noalloc_rejects_shapes_beyond_its_scratch(dl):
    """On the host, before any device call: a split that needs more than the
    24 MiB scratch is an error that names the limit."""
    q, N, K, M = 14, 4096, 12288, 400
    need = dl.qgemm_workspace_bytes(q, N, K, M)
    assert need > SCRATCH
    fake = ctypes.c_void_p(1 << 20)
    rc = dl.lib.dllm_qgemm_noalloc(q, fake, N, K, fake, None, M, None, fake, N, None)
    assert rc == dl.E_WORKSPACE
    assert "scratch" in dl.last_error() and str(SCRATCH) in dl.last_error()
