"""GPU parity at Dream-7B's shapes and for what that model adds to the path
(mojo-dllm README, milestones: "Dream-7B (GQA, QKV bias, shifted logits, its
sampler)"; "Logits only where the sampler looks": every masked position of the
canvas, 152 064 output columns).  The layer dimensions are the model's
published configuration, which the pages do not restate: hidden 3584, 28
query and 4 key/value heads of 128, FFN 18944.  Bars as in test_gpu_parity:
|gpu - oracle| <= 1e-4 * (|oracle| + rms(row)), argmax identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _check_argmax, _check_confidence, _dmax, _say, _weights, assert_close_rows

pytestmark = pytest.mark.gpu

D_MODEL, FFN, HQ, HKV, HD, VOCAB = 3584, 18944, 28, 4, 128, 152064
L = 148


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


# ------------------------------------------------------------ QKV bias ----
def test_qgemm_bias_every_output_path(dl):
    """The bias enters once on each output path: the GEMM's own epilogue (no
    K split), the split reduction with 16-byte stores, the reduction's element
    stores (bias not 16-byte aligned), and a ragged N."""
    assert dl.qgemm_workspace_bytes(12, 4096, 4096, L) > 0, "this shape must take the K split"
    cases = [(12, 4096, 4096, L), (14, 333, 2048, 37)]
    for qtype, N, K, M in cases:
        w = _weights(qtype, N, K, 81, f"bias-w-{qtype}-{N}")
        xq = oracle.quantize_q8k(synth.normal_f32((M, K), 81, f"bias-x-{K}").numpy())
        big = synth.normal_f32((N + 1,), 81, f"bias-{N}") * 4.0
        wd, xd = w.to(DEV), torch.from_numpy(xq).to(DEV)
        ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
        for off in (0, 1):  # off = 1: 4-byte but not 16-byte aligned bias
            bias = big[off:off + N]
            ref = oracle.gemm(qtype, w.numpy(), N, K, xq, M, bias=bias.numpy())
            bd = big.to(DEV)[off:off + N]
            for workspace in (ws, None):
                _say(f"qgemm_bias qtype={qtype} {M}x{N}x{K} off={off} split={workspace is not None}")
                y = dl.qgemm(qtype, wd, N, K, xd, M, workspace=workspace, bias=bd).cpu().numpy()
                assert_close_rows(y, ref, f"qgemm_bias {qtype} {N}x{K} off={off} ws={workspace is not None}")
        # the plain entry point is unchanged by the bias path
        y0 = dl.qgemm(qtype, wd, N, K, xd, M, workspace=ws)
        y1 = dl.qgemm(qtype, wd, N, K, xd, M, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


# ------------------------------------------------------- layer shapes ----
@pytest.mark.parametrize("qtype,N,K,bias", [
    (12, D_MODEL + 2 * HKV * HD, D_MODEL, True),   # Q + K + V stacked, with their bias
    (14, HKV * HD, D_MODEL, True),                 # V alone in Q6_K, with its bias
    (12, D_MODEL, D_MODEL, False),                 # O
    (12, 2 * FFN, D_MODEL, False),                 # gate + up stacked
    (12, D_MODEL, FFN, False),                     # down, Q4_K
    (14, D_MODEL, FFN, False),                     # down, Q6_K
])
def test_dream_layer_shapes(dl, qtype, N, K, bias):
    """Every linear-layer shape of a Dream-7B layer at L = 148 (K = 3584 is
    14 super-blocks, K = 18944 is 74), in the launch configuration the step
    would use (K-split workspace and the per-token scale hint): whole oracle
    rows for five tokens over both token tiles."""
    _say(f"dream shape qtype={qtype} N={N} K={K} bias={bias}")
    w = _weights(qtype, N, K, 82, f"dream-{qtype}-{N}-{K}")
    xq = oracle.quantize_q8k(synth.normal_f32((L, K), 82, f"dream-x-{K}").numpy())
    b = synth.normal_f32((N,), 82, f"dream-b-{N}") if bias else None
    ws = dl.qgemm_workspace(qtype, N, K, L, DEV)
    dmax = torch.from_numpy(_dmax(xq, L, K)).to(DEV)
    y = dl.qgemm(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), L, workspace=ws, x_dmax=dmax,
                 bias=None if b is None else b.to(DEV)).cpu().numpy()
    toks = [0, 63, 79, 80, L - 1]
    ref = oracle.gemm(qtype, w.numpy(), N, K, xq[toks], len(toks), bias=None if b is None else b.numpy())
    assert_close_rows(y[toks], ref, f"dream shape {qtype} {N}x{K}")


# -------------------------------------------------- grouped-query attention ----
def _gqa_bound(qkv, L, H, Hkv, D, scale):
    """The bound of test_gpu_parity's attention test with each key/value head
    serving its group of query heads: P rounded to f16 (2^-11 relative), the
    scores' f32 accumulation entering through exp, and f32 sums; in units of
    sum_j P_ij |v_jd|."""
    r = qkv[:, :(H + 2 * Hkv) * D].astype(np.float16).astype(np.float64)
    q = r[:, :H * D].reshape(L, H, D)
    k = np.repeat(r[:, H * D:(H + Hkv) * D].reshape(L, Hkv, D), H // Hkv, axis=1)
    v = np.repeat(r[:, (H + Hkv) * D:].reshape(L, Hkv, D), H // Hkv, axis=1)
    s = np.einsum("ihd,jhd->hij", q, k) * scale
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    a = 130 * 2.0 ** -24 * abs(scale) * np.einsum("ihd,jhd->hij", np.abs(q), np.abs(k)).max(axis=2)
    pv = np.einsum("hij,jhd->ihd", p, np.abs(v))
    f = (2.0 ** -11 + np.expm1(2 * a).T[:, :, None] + 2.0 ** -20)
    return (pv * f).reshape(L, H * D)


@pytest.mark.parametrize("Lq,H,Hkv,spread,pad", [(L, HQ, HKV, 1.0, 0), (40, 6, 2, 2.0, 4), (17, 4, 1, 1.0, 0),
                                                 (256, 14, 2, 0.5, 8), (100, 7, 7, 3.0, 0)])
def test_gqa_attention(dl, Lq, H, Hkv, spread, pad):
    """Grouped-query attention against the oracle: Dream-7B's 28 query heads
    over 4 key/value heads at L = 148, smaller groups, one shared head, the
    longest canvas, and H_kv = H (plain multi-head) through the same entry."""
    D = HD
    _say(f"gqa attention L={Lq} H={H} Hkv={Hkv}")
    qkv = synth.normal_f32((Lq, (H + 2 * Hkv) * D + pad), 83, f"gqa-{Lq}-{H}-{Hkv}") * spread
    scale = D ** -0.5
    ref = oracle.attention(qkv[:, :(H + 2 * Hkv) * D].numpy(), H, D, scale, Hkv=Hkv)
    got = dl.attention(qkv.to(DEV), H, D, scale, H_kv=Hkv).cpu().numpy().astype(np.float64)
    bound = _gqa_bound(qkv.numpy(), Lq, H, Hkv, D, scale)
    err = np.abs(got - ref)
    _say(f"gqa attention L={Lq} H={H} Hkv={Hkv}: max err/bound = {np.max(err / bound):.3g}")
    assert np.all(err <= bound), f"gqa attention: worst err/bound {np.max(err / bound):.3g}"


def test_gqa_attention_follows_its_key_value_head(dl):
    """Changing key/value head 1 changes exactly the query heads of its group."""
    H, Hkv, D, Lq = 8, 2, HD, 60
    G = H // Hkv
    qkv = synth.normal_f32((Lq, (H + 2 * Hkv) * D), 84, "gqa-map")
    base = dl.attention(qkv.to(DEV), H, D, H_kv=Hkv).cpu()
    q2 = qkv.clone()
    q2[:, (H + Hkv + 1) * D:(H + Hkv + 2) * D] += 2.0
    got = dl.attention(q2.to(DEV), H, D, H_kv=Hkv).cpu()
    changed = [h for h in range(H) if not torch.equal(got[:, h * D:(h + 1) * D], base[:, h * D:(h + 1) * D])]
    assert changed == list(range(G, 2 * G))


# ------------------------------------------------------------- LM head ----
def test_dream_lmhead_every_masked_row(dl):
    """Dream's output projection (152 064 x 3584, Q6_K) over every masked
    position of a 148-token canvas: the 128 generated positions, whose logits
    come from the row before each (Dream's shifted logits), so rows 19..146.
    Whole logits against the oracle, the argmax, and the confidence."""
    N, K = VOCAB, D_MODEL
    rows = torch.arange(19, 147, dtype=torch.int32)
    _say(f"dream lmhead {rows.numel()} rows x {N} x {K}")
    w = _weights(14, N, K, 85, "dream-output")
    h = synth.normal_f32((L, K), 85, "dream-hidden")
    ref, ref_am = oracle.lmhead(14, w.numpy(), N, K, h.numpy(), rows.numpy())
    lg, am, lse, p = dl.lmhead_confidence(14, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    lg = lg.cpu().numpy(); am = am.cpu().numpy()
    assert_close_rows(lg, ref, "dream lmhead")
    _check_argmax(lg, am, ref, ref_am, "dream lmhead")
    _check_confidence(lg, lse.cpu().numpy().astype(np.float64), p.cpu().numpy().astype(np.float64), ref,
                      "dream lmhead confidence")


def test_dream_lmhead_block_of_32_streams(dl):
    """A block of 32 masked rows at Dream's head takes the streaming kernel
    (K = 3584 is 14 super-blocks, 152 064 rows): whole logits, argmax and
    confidence against the oracle, and the tiled path on the same rows."""
    N, K = VOCAB, D_MODEL
    rows = torch.arange(60, 92, dtype=torch.int32)
    w = _weights(14, N, K, 86, "dream-output-32")
    h = synth.normal_f32((L, K), 86, "dream-hidden-32")
    ref, ref_am = oracle.lmhead(14, w.numpy(), N, K, h.numpy(), rows.numpy())
    wd, hd, rd = w.to(DEV), h.to(DEV), rows.to(DEV)
    lg, am, lse, p = dl.lmhead_confidence(14, wd, N, K, hd, rd)
    lg = lg.cpu().numpy(); am = am.cpu().numpy()
    assert_close_rows(lg, ref, "dream lmhead 32 rows")
    _check_argmax(lg, am, ref, ref_am, "dream lmhead 32 rows")
    _check_confidence(lg, lse.cpu().numpy().astype(np.float64), p.cpu().numpy().astype(np.float64), ref,
                      "dream lmhead 32 rows confidence")
    lg_t, am_t, _, _ = dl.lmhead_planned(14, wd, N, K, hd, rd, path=2, confidence=False)
    lg_t = lg_t.cpu().numpy(); am_t = am_t.cpu().numpy()
    assert_close_rows(lg_t, ref, "dream lmhead 32 rows, tiled path")
    _check_argmax(lg_t, am_t, ref, ref_am, "dream lmhead 32 rows, tiled path")


def test_qgemm_bias_single_token_tile(dl):
    """Fewer tokens than one 16-token tile (M = 5), Q4_K and Q6_K, with the K
    split and without: the bias of every row, nothing on the padded tokens."""
    for qtype in (12, 14):
        N, K, M = 200, 3584, 5
        w = _weights(qtype, N, K, 87, f"bias-small-{qtype}")
        xq = oracle.quantize_q8k(synth.normal_f32((M, K), 87, "bias-small-x").numpy())
        bias = synth.normal_f32((N,), 87, "bias-small-b")
        ref = oracle.gemm(qtype, w.numpy(), N, K, xq, M, bias=bias.numpy())
        ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
        for workspace in (ws, None):
            big = torch.full((M + 3, N), 9.0, device=DEV)
            dl.qgemm(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, y=big[:M], workspace=workspace,
                     bias=bias.to(DEV))
            got = big.cpu().numpy()
            assert_close_rows(got[:M], ref, f"bias M=5 qtype={qtype} ws={workspace is not None}")
            assert np.all(got[M:] == 9.0)
