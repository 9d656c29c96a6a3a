"""GPU: two GEMMs of one activation matrix in one call (dllm_qgemm_pair),
e.g. a layer's Q + K projection in Q4_K and its V projection in Q6_K, which
read the same normalized hidden state (mojo-dllm Development plan, "Compute
design": every linear layer multiplies the L Q8_K activation rows by the
layer's weight rows).

Where the two tile plans have a grouped kernel, their work-groups share one
grid and every tile runs exactly as in its own launch, so each output must be
bit-identical to dllm_qgemm_bias alone with a full workspace: on the step's
shapes (LLaDA-8B Q + K with Q6_K V; Dream-7B's, with bias), with the roles
swapped, with no workspace (both unsplit), on shapes whose plans have no
grouped kernel (two launches in order), and on a second call over the same
workspace (the split counters are left at zero).  One direct check against
the oracle as well: |gpu - oracle| <= 1e-4 * (|oracle| + rms(row))."""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _say, _weights, assert_close_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


def _operands(dl, qa, Na, qb, Nb, K, M, bias, seed):
    wa = _weights(qa, Na, K, seed, f"pair-a-{qa}-{Na}-{K}").to(DEV)
    wb = _weights(qb, Nb, K, seed, f"pair-b-{qb}-{Nb}-{K}").to(DEV)
    x = synth.normal_f32((M, K), seed, f"pair-x-{M}-{K}", DEV)
    xq = torch.empty((M, K // 256 * 292), dtype=torch.uint8, device=DEV)
    dm = torch.empty(M, dtype=torch.float32, device=DEV)
    dl.quantize_q8k(x, xq, dm)
    ba = synth.normal_f32((Na,), seed, f"pair-ba-{Na}", DEV) if bias else None
    bb = synth.normal_f32((Nb,), seed, f"pair-bb-{Nb}", DEV) if bias else None
    return wa, wb, xq, dm, ba, bb


def _separate(dl, q, w, N, K, xq, M, dm, bias, split):
    ws = dl.qgemm_workspace(q, N, K, M, DEV) if split else None
    return dl.qgemm(q, w, N, K, xq, M, workspace=ws, x_dmax=dm, bias=bias)


CASES = [
    # (qtype_a, N_a, qtype_b, N_b, K, M, bias)
    (12, 8192, 14, 4096, 4096, 148, False),   # LLaDA-8B: Q + K with V in Q6_K (grouped)
    (12, 8192, 14, 4096, 4096, 160, False),
    (14, 4096, 12, 8192, 4096, 148, False),   # the same with A and B swapped
    (12, 4096, 14, 512, 3584, 148, True),     # Dream-7B: Q + K with V, both with bias (grouped)
    (12, 8192, 14, 4096, 4096, 37, False),    # a small canvas: no grouped kernel, two launches
    (12, 333, 14, 100, 1024, 150, True),      # ragged rows, planner-chosen plans
    (12, 2048, 12, 1024, 2048, 148, False),   # two Q4_K GEMMs: no grouped kernel, two launches
    (14, 300, 12, 500, 512, 1, True),         # one token
    # planner-chosen grouped plans whose grids are not whole groups of eight
    # and differ in size: A 132 work-groups (16.5 groups) with B 64; A 88
    # with B 128 (the larger grid's groups run after the alternation)
    (12, 2112, 14, 1000, 1024, 150, True),
    (12, 704, 14, 4096, 1024, 150, False),
]


@pytest.mark.parametrize("qa,Na,qb,Nb,K,M,bias", CASES)
def test_pair_equals_separate_calls(dl, qa, Na, qb, Nb, K, M, bias):
    _say(f"qgemm_pair {qa}:{Na} + {qb}:{Nb} K={K} M={M} bias={bias}")
    wa, wb, xq, dm, ba, bb = _operands(dl, qa, Na, qb, Nb, K, M, bias, 91)
    nb = dl.qgemm_pair_workspace_bytes(qa, Na, qb, Nb, K, M)
    assert nb >= 0
    for split in (True, False):
        ra = _separate(dl, qa, wa, Na, K, xq, M, dm, ba, split)
        rb = _separate(dl, qb, wb, Nb, K, xq, M, dm, bb, split)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=DEV) if split else None
        for call in range(2):  # the second call finds the counters the first one left
            ya, yb = dl.qgemm_pair((qa, wa, Na, None, ba), (qb, wb, Nb, None, bb), K, xq, M, workspace=ws, x_dmax=dm)
            torch.cuda.synchronize()
            assert torch.equal(ya, ra), f"A differs (split={split}, call {call})"
            assert torch.equal(yb, rb), f"B differs (split={split}, call {call})"
        if split and nb > 0:
            assert int(ws[:65536].view(torch.int32).abs().sum()) == 0, "split counters not reset"


def test_pair_row_strided_outputs_into_one_buffer(dl):
    """Both outputs as column slices of one [M, N_a + N_b] buffer (the layout
    of a fused Q|K|V activation), against the oracle on sampled tokens."""
    qa, Na, qb, Nb, K, M = 12, 8192, 14, 4096, 4096, 148
    wa, wb, xq, dm, _, _ = _operands(dl, qa, Na, qb, Nb, K, M, False, 92)
    y = torch.full((M, Na + Nb), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(dl.qgemm_pair_workspace_bytes(qa, Na, qb, Nb, K, M), 256), dtype=torch.uint8, device=DEV)
    dl.qgemm_pair((qa, wa, Na, y[:, :Na], None), (qb, wb, Nb, y[:, Na:], None), K, xq, M, workspace=ws, x_dmax=dm)
    got = y.cpu().numpy()
    assert np.all(np.isfinite(got)), "an output column was not written"
    xqh = xq.cpu().numpy()
    toks = np.array([0, 1, 63, 64, 79, 80, 131, M - 1])
    for q, w, N, c0 in ((qa, wa, Na, 0), (qb, wb, Nb, Na)):
        ref = oracle.gemm(q, w.cpu().numpy(), N, K, xqh[toks], len(toks))
        assert_close_rows(got[toks, c0:c0 + N], ref, f"pair {q}:{N} vs oracle")



def test_pair_graph_replays_match_eager(dl):
    """quantize -> the grouped Q + K / V call (V with its K split over the
    pair's workspace), captured once in a HIP graph and replayed four times
    with unrelated eager work between the replays: every replay gives the
    eager bits."""
    qa, Na, qb, Nb, K, M = 12, 8192, 14, 4096, 4096, 148
    wa, wb, xq, dm, _, _ = _operands(dl, qa, Na, qb, Nb, K, M, False, 93)
    x = synth.normal_f32((M, K), 93, "pair-graph-x", DEV)
    y = torch.empty((M, Na + Nb), dtype=torch.float32, device=DEV)
    nb = dl.qgemm_pair_workspace_bytes(qa, Na, qb, Nb, K, M)
    assert nb > 0, "V must take its K split at this shape"
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)

    def run():
        dl.quantize_q8k(x, xq, dm)
        dl.qgemm_pair((qa, wa, Na, y[:, :Na], None), (qb, wb, Nb, y[:, Na:], None), K, xq, M, workspace=ws, x_dmax=dm)

    run()
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    for k in range(4):
        y.zero_()
        junk = torch.randn(1 << 20, device=DEV) * 3.0
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {k} differs from the eager run"
        del junk
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0, "split counters not reset"
