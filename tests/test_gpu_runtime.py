"""GPU: the library as the step drives it.  Calls captured in a HIP graph
and replayed (the bench's launch mode) give the eager results bit for bit on
every replay, with unrelated eager work between replays; and calls on two
streams at once, each with its own workspace, give the sequential results
(the library keeps no state between calls); and the LM head writes through a
row-strided logits view without touching the padding."""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _weights, assert_close_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


def _layer(dl, seed):
    L, D = 148, 4096
    w = _weights(12, D, D, seed, f"rt-w-{seed}").to(DEV)
    w6 = _weights(14, 512, D, seed, f"rt-w6-{seed}").to(DEV)
    x = synth.normal_f32((L, D), seed, f"rt-x-{seed}").to(DEV)
    return L, D, w, w6, x


def test_graph_replays_match_eager(dl):
    """quantize -> Q4_K GEMM with its K split -> Q6_K GEMM with a bias ->
    masked-row LM head, captured once and replayed four times."""
    L, D, w, w6, x = _layer(dl, 91)
    bias = synth.normal_f32((512,), 91, "rt-bias").to(DEV)
    wo = _weights(14, 2048, D, 91, "rt-out").to(DEV)
    rows = torch.arange(20, 52, dtype=torch.int32, device=DEV)
    xq = torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=DEV)
    dm = torch.empty(L, dtype=torch.float32, device=DEV)
    y = torch.empty((L, D), dtype=torch.float32, device=DEV)
    y6 = torch.empty((L, 512), dtype=torch.float32, device=DEV)
    logits = torch.empty((32, 2048), dtype=torch.float32, device=DEV)
    am = torch.empty(32, dtype=torch.int32, device=DEV)
    ws = dl.qgemm_workspace(12, D, D, L, DEV)
    ws6 = dl.qgemm_workspace(14, 512, D, L, DEV)
    ws_lm = torch.empty(dl.lmhead_workspace_bytes(14, 2048, D, 32), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 256, "the Q4_K call must take its K split"

    def run():
        dl.quantize_q8k(x, xq, dm)
        dl.qgemm(12, w, D, D, xq, L, y=y, workspace=ws, x_dmax=dm)
        dl.qgemm(14, w6, 512, D, xq, L, y=y6, workspace=ws6, x_dmax=dm, bias=bias)
        dl.lmhead_masked(14, wo, 2048, D, y, rows, logits, am, ws_lm)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (xq, y, y6, logits, am)]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    for k in range(4):
        for t in (xq, y, y6, logits):
            t.zero_()
        am.fill_(-1)
        junk = torch.randn(1 << 20, device=DEV) * 3.0  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip((xq, y, y6, logits, am), eager, ("q8k", "y", "y6", "logits", "argmax")):
            assert torch.equal(a, b), f"replay {k}: {name} differs from the eager run"
        del junk
    # and the eager results are right
    ref = oracle.gemm(14, _weights(14, 512, D, 91, "rt-w6-91").numpy(), 512, D, eager[0].cpu().numpy(), L,
                      bias=bias.cpu().numpy())
    assert_close_rows(eager[2].cpu().numpy(), ref, "graph test Q6_K + bias")


def test_two_streams_at_once_match_sequential(dl):
    """Two independent GEMM chains on two streams, each with its own
    workspace, overlap on the GPU and still give the sequential results."""
    chains = [_layer(dl, 92), _layer(dl, 93)]
    outs, wss, xqs, dms = [], [], [], []
    for L, D, w, w6, x in chains:
        xqs.append(torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=DEV))
        dms.append(torch.empty(L, dtype=torch.float32, device=DEV))
        outs.append((torch.empty((L, D), dtype=torch.float32, device=DEV),
                     torch.empty((L, 512), dtype=torch.float32, device=DEV)))
        wss.append((dl.qgemm_workspace(12, D, D, L, DEV), dl.qgemm_workspace(14, 512, D, L, DEV)))

    def chain(i):
        L, D, w, w6, x = chains[i]
        for _ in range(3):
            dl.quantize_q8k(x, xqs[i], dms[i])
            dl.qgemm(12, w, D, D, xqs[i], L, y=outs[i][0], workspace=wss[i][0], x_dmax=dms[i])
            dl.qgemm(14, w6, 512, D, xqs[i], L, y=outs[i][1], workspace=wss[i][1], x_dmax=dms[i])

    for i in range(2):
        chain(i)
    torch.cuda.synchronize()
    seq = [(a.clone(), b.clone()) for a, b in outs]
    for a, b in outs:
        a.zero_(); b.zero_()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i, s in enumerate(streams):
        with torch.cuda.stream(s):
            chain(i)
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(outs[i][0], seq[i][0]) and torch.equal(outs[i][1], seq[i][1]), f"stream {i}"


@pytest.mark.parametrize("tiled", [False, True])
def test_lmhead_strided_logits(dl, tiled):
    """Logits written through a row-strided view (ldl > N) equal the
    contiguous call's, and the padding between rows is left alone, on the
    streaming and the tiled path."""
    path = 2 if tiled else 1
    N, K, L = 3000, 1024, 60
    w = _weights(14, N, K, 94, "rt-lm").to(DEV)
    h = synth.normal_f32((L, K), 94, "rt-lm-h").to(DEV)
    rows = torch.tensor([3, 59, 0, 17, 42], dtype=torch.int32, device=DEV)
    ref_lg, ref_am, _, _ = dl.lmhead_planned(14, w, N, K, h, rows, path=path, confidence=False)
    big = torch.full((rows.numel(), N + 12), -7.0, device=DEV)
    lg, am, _, _ = dl.lmhead_planned(14, w, N, K, h, rows, path=path, confidence=False, logits=big[:, :N])
    torch.cuda.synchronize()
    assert torch.equal(big[:, :N], ref_lg) and torch.equal(am, ref_am)
    assert torch.all(big[:, N:] == -7.0)


def test_split_workspace_counters_return_to_zero(dl):
    """A K-split call leaves the workspace's per-tile arrival counters (after
    the partial slices) at zero, so that the next call -- another shape, or a
    graph replay -- starts from a clean state; repeated calls on one
    workspace give the same bits."""
    M = 148
    for qtype, N, K in [(12, 4096, 4096), (14, 4096, 12288), (12, 333, 3072)]:
        nb = dl.qgemm_workspace_bytes(qtype, N, K, M)
        ldp = (N + 63) // 64 * 64
        S = (nb - 65536) // (M * ldp * 4)
        assert S > 1 and nb == 65536 + S * M * ldp * 4, "these shapes take the K split"
        off = 65536
        w = _weights(qtype, N, K, 95, f"cnt-{qtype}-{N}").to(DEV)
        xq = dl.quantize_q8k(synth.normal_f32((M, K), 95, f"cnt-x-{K}").to(DEV))
        ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
        a = dl.qgemm(qtype, w, N, K, xq, M, workspace=ws).clone()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:off])) == 0, f"counters of {qtype} {N}x{K}"
        b = dl.qgemm(qtype, w, N, K, xq, M, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
