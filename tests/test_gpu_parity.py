"""GPU parity: libdllm's HIP kernels (through the C ABI) against the CPU oracle.

Bars (quantized GEMM stream of one denoising step; mojo-dllm Development plan,
"Compute design"):
  * Q8_K bytes, shared decoded form and per-16 int32 partials: bit-exact.
  * f32 GEMM / LM-head outputs: |gpu - oracle| <= 1e-4 * (|oracle| + rms(row)),
    rms(row) = RMS of the oracle's outputs for that token.
  * LM-head argmax: identical to the oracle's, except where the oracle's top
    two logits are closer than the tolerance (then several answers are
    correct and the GPU's pick must be one of them); and always identical to
    the argmax of the GPU's own f32 logits (same precision, lowest index).
Inputs are seeded synthetic (synth/), shaped like LLaDA-8B's layers.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return dl


def _say(*a):
    print(*a, flush=True)


# The kernels' own arithmetic (exact int32 super-block sums, f32 epilogue,
# f16 high/low pairs good to ~2^-21) stays far inside the bound on these
# inputs; above TIGHT of the bound something is wrong even if the bound holds.
TIGHT = 0.05


def assert_close_rows(y_gpu: np.ndarray, y_ref: np.ndarray, what: str, tight: bool = True):
    y_gpu = np.asarray(y_gpu, np.float64)
    assert y_gpu.shape == y_ref.shape, what
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True))
    bound = TOL * (np.abs(y_ref) + rms)
    err = np.abs(y_gpu - y_ref)
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    _say(f"{what}: max err/bound = {ratio:.3g}")
    assert np.all(np.isfinite(y_gpu)), what
    assert np.all(err <= bound), f"{what}: max err/bound {ratio}"
    if tight:
        assert ratio < TIGHT, f"{what}: max err/bound {ratio} above the {TIGHT} alarm level"


def _weights(qtype, N, K, seed, name):
    return synth.qk_rows(qtype, N, K, seed, name)


def _dmax(xq: np.ndarray, M: int, K: int) -> np.ndarray:
    """Per token, the largest |d| over its Q8_K records (f32, exact)."""
    d = np.ascontiguousarray(xq.reshape(M, K // 256, 292)[:, :, :4]).view("<f4")[..., 0]
    return np.abs(d).max(axis=1).astype(np.float32)


# ---------------------------------------------------------------- Q8_K ----
@pytest.mark.parametrize("M,K,pad", [(1, 256, 0), (17, 512, 0), (148, 4096, 0), (148, 12288, 0), (33, 1024, 64)])
def test_quantize_q8k_bitexact(dl, M, K, pad):
    _say(f"quantize M={M} K={K} pad={pad}")
    x = synth.normal_f32((M, K + pad), 11, f"q8k-{M}-{K}")
    x = x * torch.logspace(-3, 3, M).unsqueeze(1)  # spread of magnitudes
    ref = oracle.quantize_q8k(x[:, :K].numpy())
    dmax = torch.full((M,), -1.0, device=DEV)
    got = dl.quantize_q8k(x.to(DEV)[:, :K], dmax=dmax).cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(dmax.cpu().numpy(), _dmax(ref, M, K))


def test_quantize_q8k_edge_blocks(dl):
    K = 256 * 8
    x = torch.zeros((6, K))
    x[1, 5], x[1, 300] = -3.0, 3.0            # magnitude tie: first index wins
    x[2, :] = 1e-30                            # tiny values
    x[2, 777] = -2e-30
    x[3, :] = torch.linspace(-1e30, 1e30, K)   # huge values
    x[4, ::3] = 0.5                            # exact half-way products
    x[4, 1::3] = -0.25
    x[5, :] = synth.normal_f32((K,), 5, "edge")
    x[5, 256:512] = 0.0                        # an all-zero block inside a row
    ref = oracle.quantize_q8k(x.numpy())
    dmax = torch.full((6,), -1.0, device=DEV)
    got = dl.quantize_q8k(x.to(DEV), dmax=dmax).cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(dmax.cpu().numpy(), _dmax(ref, 6, K))
    assert dmax[0].item() == 0.0  # an all-zero row


# ------------------------------------------------- fused producers ----
def _split_records(xq, M, K):
    r = xq.reshape(M, K // 256, 292)
    d = np.ascontiguousarray(r[:, :, :4]).view(np.float32)[..., 0]
    return d, r[:, :, 4:]  # block scales; codes and bsums (bytes 4..292)


@pytest.mark.parametrize("M,K,pad", [(1, 256, 0), (37, 4096, 0), (148, 4096, 0), (148, 12288, 0), (9, 16384, 128)])
def test_rmsnorm_quantize_q8k(dl, M, K, pad):
    """RMSNorm -> Q8_K: codes and bsums bit-exact (those of x*g); each block
    scale within 2 ulp of the oracle's (r's f64 sum of squares runs in another
    order, which can move r by one f32 ulp); dmax exactly the largest |d|."""
    _say(f"rmsnorm quantize M={M} K={K} pad={pad}")
    x = synth.normal_f32((M, K + pad), 51, f"rms-{M}-{K}") * torch.logspace(-4, 4, M).unsqueeze(1)
    g = synth.normal_f32((K,), 51, f"rms-g-{K}")
    g[::97] = 0.0
    if M > 2:
        x[2, :] = 0.0  # an all-zero row: d = 0 everywhere
    ref, ref_dmax = oracle.rmsnorm_quantize_q8k(x[:, :K].numpy(), g.numpy(), 1e-5)
    dmax = torch.full((M,), -1.0, device=DEV)
    got = dl.rmsnorm_quantize_q8k(x.to(DEV)[:, :K], g.to(DEV), 1e-5, dmax=dmax).cpu().numpy()
    gd, gq = _split_records(got, M, K)
    rd, rq = _split_records(ref, M, K)
    assert np.array_equal(gq, rq), "codes / bsums differ"
    assert np.all(np.abs(gd - rd) <= 2 * np.spacing(np.abs(rd).astype(np.float32))), "block scales beyond 2 ulp"
    assert np.array_equal(dmax.cpu().numpy(), np.abs(gd).max(axis=1))
    assert np.all(np.abs(dmax.cpu().numpy() - ref_dmax) <= 2 * np.spacing(ref_dmax))
    _say(f"rmsnorm quantize: {np.count_nonzero(gd != rd)} of {gd.size} block scales differ from the oracle's by an ulp")


@pytest.mark.parametrize("M,F,pad", [(1, 256, 0), (37, 2048, 0), (148, 12288, 0), (5, 1024, 64)])
def test_swiglu_quantize_q8k(dl, M, F, pad):
    """SwiGLU -> Q8_K: the records of f32(silu(gate) * up) evaluated in f64,
    bit-exact, including gates of 0, +-1000 and 60; dmax exact."""
    _say(f"swiglu quantize M={M} F={F} pad={pad}")
    gu = synth.normal_f32((M, 2 * F + pad), 52, f"swiglu-{M}-{F}") * 3.0
    gu[0, :4] = torch.tensor([0.0, -1000.0, 1000.0, 60.0])
    ref, ref_dmax = oracle.swiglu_quantize_q8k(gu[:, :2 * F].numpy())
    dmax = torch.full((M,), -1.0, device=DEV)
    got = dl.swiglu_quantize_q8k(gu.to(DEV)[:, :2 * F], dmax=dmax).cpu().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(dmax.cpu().numpy(), ref_dmax)


def test_fused_producers_feed_the_gemm(dl):
    """The fused records drive dllm_qgemm like any Q8_K input: whole oracle
    rows of the down projection on SwiGLU records and of Q+K+V on RMSNorm
    records (the GEMM's parity with the oracle's own records)."""
    M, D, F = 20, 1024, 2048
    gu = synth.normal_f32((M, 2 * F), 53, "feed-gu")
    xs = synth.normal_f32((M, D), 53, "feed-x")
    g = synth.normal_f32((D,), 53, "feed-g")
    for qtype, N, K, xq_ref, xq_gpu in (
            (12, 300, F, oracle.swiglu_quantize_q8k(gu.numpy())[0], dl.swiglu_quantize_q8k(gu.to(DEV))),
            (14, 300, D, oracle.rmsnorm_quantize_q8k(xs.numpy(), g.numpy(), 1e-5)[0],
             dl.rmsnorm_quantize_q8k(xs.to(DEV), g.to(DEV), 1e-5))):
        w = _weights(qtype, N, K, 53, f"feed-w-{qtype}")
        ref = oracle.gemm(qtype, w.numpy(), N, K, xq_ref, M)
        y = dl.qgemm(qtype, w.to(DEV), N, K, xq_gpu, M).cpu().numpy()
        assert_close_rows(y, ref, f"gemm on fused records qtype={qtype}")


# --------------------------------------------------------- attention ----
def _attention_bound(qkv, L, H, D, scale):
    """Per output, what the GPU may differ from the oracle (which uses the same
    f16-rounded q, k, v): P rounded to f16 for the second product (2^-11
    relative), the scores' f32 accumulation (at most ~128 * 2^-24 * scale *
    sum|q||k|, entering the softmax weights doubled through exp), and f32
    sums and division (well below both); in units of sum_j P_ij |v_jd|."""
    r = qkv[:, :3 * H * D].astype(np.float16).astype(np.float64)
    q = r[:, :H * D].reshape(L, H, D)
    k = r[:, H * D:2 * H * D].reshape(L, H, D)
    v = r[:, 2 * H * D:].reshape(L, H, D)
    s = np.einsum("ihd,jhd->hij", q, k) * scale
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    a = 130 * 2.0 ** -24 * abs(scale) * np.einsum("ihd,jhd->hij", np.abs(q), np.abs(k)).max(axis=2)  # [h, i]
    pv = np.einsum("hij,jhd->ihd", p, np.abs(v))  # [i, h, d]
    f = (2.0 ** -11 + np.expm1(2 * a).T[:, :, None] + 2.0 ** -20)
    return (pv * f).reshape(L, H * D)


@pytest.mark.parametrize("L,H,spread,pad", [(1, 1, 1.0, 0), (17, 3, 1.0, 4), (64, 2, 3.0, 0), (80, 3, 1.0, 0),
                                            (100, 2, 2.0, 0), (148, 32, 1.0, 0), (148, 4, 4.0, 8), (176, 2, 2.0, 4),
                                            (200, 2, 0.3, 0), (256, 2, 1.0, 0)])
def test_attention(dl, L, H, spread, pad):
    """Bidirectional attention against the oracle on the same f16-rounded
    operands, within the bound of the GPU's own roundings; from the layout of
    a fused Q+K+V projection (with row padding), at soft and peaked softmaxes
    and key counts from one to 256 (every count of 32-key chunks, 1 to 8)."""
    D = 128
    _say(f"attention L={L} H={H} spread={spread} pad={pad}")
    qkv = synth.normal_f32((L, 3 * H * D + pad), 71, f"att-{L}-{H}-{pad}") * spread
    scale = D ** -0.5
    ref = oracle.attention(qkv[:, :3 * H * D].numpy(), H, D, scale)
    got = dl.attention(qkv.to(DEV), H, D, scale).cpu().numpy().astype(np.float64)
    bound = _attention_bound(qkv.numpy(), L, H, D, scale)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"attention: worst err/bound {np.max(err / bound):.3g}"
    _say(f"attention L={L} H={H}: max err/bound = {np.max(err / bound):.3g}, max rel err "
         f"{np.max(err / (np.abs(ref) + 1e-30)):.2e}")


def test_attention_strided_output_and_bidirectional(dl):
    """A strided output leaves its padding alone; query 0 follows a change in
    the last key's value (no causal mask)."""
    L, H, D = 100, 2, 128
    qkv = synth.normal_f32((L, 3 * H * D), 72, "att-strided")
    big = torch.full((L, H * D + 12), 7.0, device=DEV)
    dl.attention(qkv.to(DEV), H, D, out=big[:, :H * D])
    q2 = qkv.clone()
    q2[L - 1, 2 * H * D:] += 5.0
    o2 = dl.attention(q2.to(DEV), H, D)
    torch.cuda.synchronize()
    assert torch.all(big[:, H * D:] == 7.0)
    assert not torch.allclose(big[0, :H * D], o2[0])
    ref = oracle.attention(qkv.numpy(), H, D, D ** -0.5)
    bound = _attention_bound(qkv.numpy(), L, H, D, D ** -0.5)
    assert np.all(np.abs(big[:, :H * D].cpu().numpy() - ref) <= bound)


def test_gather_quantize_through_lmhead_equals_plain_quantize(dl):
    # the LM head's gather+quantize must feed the GEMM the same Q8_K bytes as
    # quantizing the gathered rows directly: compare logits with qgemm on them.
    N, K, M = 192, 512, 40
    w = _weights(dl.Q6_K, N, K, 21, "w").to(DEV)
    h = synth.normal_f32((M, K), 21, "h").to(DEV)
    rows = torch.tensor([39, 0, 17, 17, 5], dtype=torch.int32, device=DEV)
    logits, _ = dl.lmhead_masked(dl.Q6_K, w, N, K, h, rows)
    xq = dl.quantize_q8k(h[rows.long()].contiguous())
    y = dl.qgemm(dl.Q6_K, w, N, K, xq, rows.numel())
    torch.cuda.synchronize()
    assert torch.equal(logits, y)


# -------------------------------------------------------------- decode ----
@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("nsb", [1, 33, 1024])
def test_decode_bitexact(dl, qtype, nsb):
    _say(f"decode qtype={qtype} nsb={nsb}")
    w = _weights(qtype, nsb, 256, 3, f"dec-{nsb}")
    if qtype == 14:
        w.view(nsb, 210)[0, 192:208] = torch.tensor([-128] * 8 + [127] * 8, dtype=torch.int8).view(torch.uint8)
    ref = oracle.decode_shared(qtype, w.numpy(), nsb)
    got = dl.decode_qk(qtype, w.to(DEV), nsb).cpu().numpy()
    assert np.array_equal(got, ref)


# ------------------------------------------------------------ partials ----
@pytest.mark.parametrize("qtype", [12, 14])
def test_partials_bitexact(dl, qtype):
    N, K, M = 37, 768, 5
    w = _weights(qtype, N, K, 4, "p")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 4, "px").numpy())
    ref = oracle.partials(qtype, w.numpy(), N, K, xq, M)
    got = dl.qgemm_partials_i32(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M).cpu().numpy()
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- GEMM ----
SHAPES = [(1, 1, 256), (17, 70, 512), (148, 200, 1024), (33, 64, 2048), (161, 65, 768), (160, 128, 4096),
          (5, 300, 3072)]


@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("split", [False, True])
def test_qgemm_small_shapes(dl, qtype, M, N, K, split):
    _say(f"qgemm qtype={qtype} M={M} N={N} K={K} split={split}")
    w = _weights(qtype, N, K, 7, f"g-{N}-{K}")
    x = synth.normal_f32((M, K), 7, f"gx-{M}-{K}")
    xq = oracle.quantize_q8k(x.numpy())
    ref = oracle.gemm(qtype, w.numpy(), N, K, xq, M)
    ws = None
    if split:
        ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
    y = dl.qgemm(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, workspace=ws).cpu().numpy()
    assert_close_rows(y, ref, f"qgemm {qtype} {M}x{N}x{K} split={split}")


TILES = (1, 2, 3, 4, 5, 6, 7)


@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", [(148, 333, 2048), (37, 130, 1024), (160, 256, 512)])
def test_qgemm_every_tile_configuration(dl, qtype, tile, M, N, K):
    """Each work-group shape (64 rows as 4 waves x 16, 128 rows as 8 waves x
    16, and over at most 80 tokens 256 rows as 8 waves x 32 or 128 rows as 4
    waves x 32; 64 rows as 4 waves x 16 with one activation stage; 64 rows as
    4 waves x 16 over at most 80 tokens; 192 rows as 12 waves x 16 over at
    most 80 tokens), chosen through the test entry dllm_qgemm_planned, on
    ragged rows and tokens, split and unsplit."""
    _say(f"qgemm tile={tile} qtype={qtype} M={M} N={N} K={K}")
    w = _weights(qtype, N, K, 11, f"t-{N}-{K}")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 11, f"tx-{M}-{K}").numpy())
    ref = oracle.gemm(qtype, w.numpy(), N, K, xq, M)
    xd = torch.from_numpy(xq).to(DEV)
    wd = w.to(DEV)
    for split in (min(3, K // 256), 1):
        y = dl.qgemm_planned(qtype, wd, N, K, xd, M, tile=tile, split=split).cpu().numpy()
        assert_close_rows(y, ref, f"qgemm tile {tile} {qtype} {M}x{N}x{K} split={split}")


@pytest.mark.parametrize("qtype,N,K", [(12, 4096, 4096), (14, 4096, 12288)])
def test_qgemm_full_size_layers(dl, qtype, N, K):
    """Single LLaDA-8B linear layers at L = 148: attn_q (Q4_K 4096x4096) and
    attn_v/ffn_down-shaped Q6_K (4096x12288), in the bench's launch
    configuration (with the K-split workspace), against the full oracle."""
    M = 148
    _say(f"full-size qgemm qtype={qtype} N={N} K={K}")
    w = _weights(qtype, N, K, 42, f"layer-{qtype}-{N}-{K}")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 42, f"act-{K}").numpy())
    ref = oracle.gemm(qtype, w.numpy(), N, K, xq, M)
    ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
    y = dl.qgemm(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, workspace=ws).cpu().numpy()
    assert_close_rows(y, ref, f"full qgemm {qtype} {N}x{K}")


def test_qgemm_gate_up_shape_sampled(dl):
    """gate/up grouped (Q4_K, N = 2 x 12288, K = 4096) at L = 148: sampled
    outputs one by one, plus whole oracle rows for four tokens."""
    qtype, N, K, M = 12, 24576, 4096, 148
    w = _weights(qtype, N, K, 42, "gateup")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 42, "gateup-x").numpy())
    ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
    y = dl.qgemm(qtype, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, workspace=ws).cpu().numpy()
    toks = [0, 57, 146, 147]
    ref_rows = oracle.gemm(qtype, w.numpy(), N, K, xq[toks], len(toks))
    assert_close_rows(y[toks], ref_rows, "gate/up full rows")
    rng = np.random.default_rng(0)
    mi = rng.integers(0, M, 3000)
    ni = rng.integers(0, N, 3000)
    ref = oracle.gemm_sample(qtype, w.numpy(), N, K, xq, M, mi, ni)
    rms = float(np.sqrt(np.mean(ref_rows ** 2)))
    err = np.abs(y[mi, ni] - ref)
    assert np.all(err <= TOL * (np.abs(ref) + rms)), float(err.max())


def test_qgemm_q4k_min_term_f16_ties(dl):
    """Q4_K min term operands d_x * (bsum_2j + bsum_2j+1) that fall exactly
    half-way between two f16 values (d_x = 2^-6 -> scaled 0.5, odd sums above
    2048): the kernel's f16 high/low split must still add up exactly."""
    from ggufpack import pack_q8k
    rng = np.random.default_rng(17)
    N, M, K = 96, 24, 1024
    w = _weights(12, N, K, 17, "ties")
    recs = []
    for m in range(M):
        row = []
        for s in range(K // 256):
            q = np.zeros(256, np.int64)
            for j in range(8):
                target = int(rng.integers(1025, 2031)) * 2 + 1  # odd, in (2048, 4064)
                target *= 1 if rng.random() < 0.5 else -1
                v = np.full(32, target // 32)
                v[: target - v.sum()] += 1  # spread the remainder
                q[32 * j:32 * j + 32] = rng.permutation(v)
            assert np.abs(q).max() <= 127
            row.append(pack_q8k(2.0 ** -6, q))
        recs.append(np.concatenate(row))
    xq = np.stack(recs)
    ref = oracle.gemm(12, w.numpy(), N, K, xq, M)
    y = dl.qgemm(12, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M).cpu().numpy()
    assert_close_rows(y, ref, "q4k f16 ties")
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    assert float((np.abs(y - ref) / (TOL * (np.abs(ref) + rms))).max()) < 0.05


def test_qgemm_integer_special_case_exact(dl):
    """d = 1, dmin = 0, unit scales, d_x = 1: every partial sum is an integer
    below 2^24, so the f32 result must equal the integer dot product."""
    from ggufpack import pack_q4k, pack_q8k
    rng = np.random.default_rng(3)
    N, M, K = 64, 20, 1024
    u = rng.integers(0, 16, (N, K))
    q = rng.integers(-127, 128, (M, K))
    w = np.stack([np.concatenate([pack_q4k(0x3C00, 0, [1] * 8, [0] * 8, u[n, 256 * s:256 * s + 256])
                                  for s in range(K // 256)]) for n in range(N)])
    xq = np.stack([np.concatenate([pack_q8k(1.0, q[m, 256 * s:256 * s + 256]) for s in range(K // 256)])
                   for m in range(M)])
    y = dl.qgemm(12, torch.from_numpy(w).to(DEV), N, K, torch.from_numpy(xq).to(DEV), M).cpu().numpy()
    assert np.array_equal(y.astype(np.int64), q @ u.T)


def test_qgemm_zero_weights_and_strided_output(dl):
    N, K, M = 100, 512, 30
    w = torch.zeros((N, K // 256 * 210), dtype=torch.uint8, device=DEV)
    xq = dl.quantize_q8k(synth.normal_f32((M, K), 2, "z").to(DEV))
    big = torch.full((M, N + 28), 7.0, device=DEV)
    dl.qgemm(14, w, N, K, xq, M, y=big[:, :N])
    torch.cuda.synchronize()
    assert torch.count_nonzero(big[:, :N]) == 0
    assert torch.all(big[:, N:] == 7.0)


def test_qgemm_deterministic(dl):
    N, K, M = 4096, 4096, 148
    w = _weights(12, N, K, 9, "det").to(DEV)
    xq = dl.quantize_q8k(synth.normal_f32((M, K), 9, "detx").to(DEV))
    ws = dl.qgemm_workspace(12, N, K, M, DEV)
    a = dl.qgemm(12, w, N, K, xq, M, workspace=ws).clone()
    b = dl.qgemm(12, w, N, K, xq, M, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("M", [148, 160])
@pytest.mark.parametrize("qtype,N,K", [(12, 24576, 4096), (12, 12288, 4096), (12, 8192, 4096), (12, 4096, 4096),
                                        (14, 4096, 4096), (12, 4096, 12288), (14, 4096, 12288)])
def test_qgemm_step_shapes(dl, qtype, N, K, M):
    """Every linear-layer shape of the LLaDA-8B step at L = 148 and at L = 160
    (the canvas of 32 prompt + 128 generated tokens), in the launch
    configuration the step uses (tuned tile and K split, with workspace):
    whole oracle rows for five tokens spread over both token tiles."""
    _say(f"step shape qtype={qtype} N={N} K={K} M={M}")
    w = _weights(qtype, N, K, 21, f"step-{qtype}-{N}-{K}")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 21, f"step-x-{K}-{M}").numpy())
    ws = dl.qgemm_workspace(qtype, N, K, M, DEV)
    wd, xd = w.to(DEV), torch.from_numpy(xq).to(DEV)
    dmax = torch.from_numpy(_dmax(xq, M, K)).to(DEV)
    y = dl.qgemm(qtype, wd, N, K, xd, M, workspace=ws, x_dmax=dmax)
    toks = [0, 63, 79, 80, M - 1]
    ref = oracle.gemm(qtype, w.numpy(), N, K, xq[toks], len(toks))
    assert_close_rows(y.cpu().numpy()[toks], ref, f"step shape {qtype} {N}x{K}")
    # the per-token scale summary only spares the kernel its own scan
    y2 = dl.qgemm(qtype, wd, N, K, xd, M, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("tile", TILES)
def test_qgemm_dmax_hint_matches_scan(dl, tile):
    """Q4_K with the per-token largest |d| from dllm_quantize_q8k: the same
    bits as without it (where the kernel reads every d itself), for every
    tile configuration, split and unsplit, on ragged shapes, with magnitudes
    spread over nine decades so the power-of-two range scale differs per
    token."""
    N, K, M = 333, 3072, 150
    _say(f"dmax hint tile={tile}")
    w = _weights(12, N, K, 23, "hint").to(DEV)
    x = synth.normal_f32((M, K), 23, "hint-x") * torch.logspace(-4, 5, M).unsqueeze(1)
    dmax = torch.empty(M, device=DEV)
    xq = dl.quantize_q8k(x.to(DEV), dmax=dmax)
    ref = oracle.gemm(12, w.cpu().numpy(), N, K, xq.cpu().numpy(), M)
    for split in (4, 1):
        a = dl.qgemm_planned(12, w, N, K, xq, M, tile=tile, split=split, x_dmax=dmax)
        b = dl.qgemm_planned(12, w, N, K, xq, M, tile=tile, split=split)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        assert_close_rows(a.cpu().numpy(), ref, f"dmax hint tile {tile} split={split}")


@pytest.mark.parametrize("tile,split", [(7, 4), (6, 3), (2, 12), (4, 7), (5, 5)])
def test_qgemm_planned_splits(dl, tile, split):
    """(tile configuration, K split) pinned through dllm_qgemm_planned: the
    result stays within the bound for each plan, including splits whose last
    slice is shorter (12 super-blocks over 7 and 5 slices)."""
    N, K, M = 333, 3072, 150
    _say(f"planned tile={tile} split={split}")
    w = _weights(12, N, K, 29, "plan")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 29, "plan-x").numpy())
    ref = oracle.gemm(12, w.numpy(), N, K, xq, M)
    y = dl.qgemm_planned(12, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, tile=tile, split=split).cpu().numpy()
    assert_close_rows(y, ref, f"planned tile={tile} split={split}")


@pytest.mark.parametrize("N,pad,K,S", [(332, 0, 3072, 2), (332, 4, 3072, 3), (332, 0, 2560, 5), (332, 8, 3072, 6),
                                       (332, 0, 4096, 8), (332, 0, 3072, 12), (333, 0, 3072, 4), (332, 1, 3072, 2),
                                       (333, 3, 4096, 8), (333, 0, 2560, 5)])
def test_qgemm_split_reduce_paths(dl, N, pad, K, S):
    """The K-split sum for fixed slice counts (2, 3, 4, 6, 8) and others (run
    time), with 16-byte stores (N and the row stride multiples of four) and
    element stores (either not), into a strided output whose padding columns
    stay untouched."""
    M = 150
    _say(f"split reduce N={N} pad={pad} S={S}")
    w = _weights(12, N, K, 31, f"red-{N}")
    xq = oracle.quantize_q8k(synth.normal_f32((M, K), 31, "red-x").numpy())
    ref = oracle.gemm(12, w.numpy(), N, K, xq, M)
    big = torch.full((M, N + pad), 7.0, device=DEV)
    dl.qgemm_planned(12, w.to(DEV), N, K, torch.from_numpy(xq).to(DEV), M, tile=6, split=S, y=big[:, :N])
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == 7.0)
    assert_close_rows(big[:, :N].cpu().numpy(), ref, f"split reduce N={N} pad={pad} S={S}")


def test_qgemm_shared_workspace_across_shapes(dl):
    """One workspace, sized for the largest, serves K-split calls of
    different shapes in stream order (whole oracle rows of four tokens)."""
    M = 148
    shapes = [(12, 4096, 4096), (12, 12288, 4096), (14, 4096, 12288), (12, 4096, 4096), (14, 2048, 3072)]
    nb = max(dl.qgemm_workspace_bytes(q, N, K, M) for q, N, K in shapes)
    assert sum(dl.qgemm_workspace_bytes(q, N, K, M) > 0 for q, N, K in shapes) >= 3  # most of them split K
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    toks = [0, 31, 100, 147]
    xs = {}
    for i, (q, N, K) in enumerate(shapes):
        _say(f"shared workspace call {i}: qtype={q} N={N} K={K}")
        w = _weights(q, N, K, 13, f"ws-{q}-{N}-{K}")
        if K not in xs:
            xs[K] = oracle.quantize_q8k(synth.normal_f32((M, K), 13, f"wsx-{K}").numpy())
        y = dl.qgemm(q, w.to(DEV), N, K, torch.from_numpy(xs[K]).to(DEV), M, workspace=ws).cpu().numpy()
        ref = oracle.gemm(q, w.numpy(), N, K, xs[K][toks], len(toks))
        assert_close_rows(y[toks], ref, f"shared workspace call {i}")


# ------------------------------------------------------------- LM head ----
def _check_argmax(logits_gpu, am_gpu, ref_logits, ref_am, what):
    lg = np.asarray(logits_gpu, np.float64)
    # same precision: the kernel's pick is the argmax (lowest index) of its own f32 logits
    assert np.array_equal(am_gpu, np.argmax(np.asarray(logits_gpu), axis=1)), what
    rms = np.sqrt(np.mean(ref_logits ** 2, axis=1))
    exceptions = 0
    for r in range(ref_logits.shape[0]):
        if am_gpu[r] == ref_am[r]:
            continue
        top = np.sort(ref_logits[r])[-2:]
        tol = 2 * TOL * (abs(top[1]) + rms[r])
        assert top[1] - top[0] <= tol, f"{what}: row {r} argmax {am_gpu[r]} != {ref_am[r]}"
        assert ref_logits[r, am_gpu[r]] >= top[1] - tol
        exceptions += 1
    _say(f"{what}: argmax identical in {ref_logits.shape[0] - exceptions}/{ref_logits.shape[0]} rows")


@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("n_rows", [1, 7, 32, 40])
@pytest.mark.parametrize("K", [768, 1024, 2560])
def test_lmhead_small(dl, qtype, tiled, n_rows, K):
    """Both LM-head paths: the streaming kernel (<= 32 rows, K <= 4096) and
    the tiled GEMM (forced through dllm_lmhead_planned, and taken for 40 rows),
    on a vocabulary that is not a multiple of any tile (1000 rows) and K of
    3, 4 and 10 super-blocks (the stream's three-deep load rotation then
    meets a row-block boundary at every phase)."""
    N, M = 1000, 148
    _say(f"lmhead qtype={qtype} tiled={tiled} n_rows={n_rows} K={K}")
    w = _weights(qtype, N, K, 13, f"lm-small-{qtype}")
    h = synth.normal_f32((M, K), 13, "lm-h")
    rows = synth.distinct_rows(n_rows, M, 13, f"rows-{n_rows}")
    ref, ref_am = oracle.lmhead(qtype, w.numpy(), N, K, h.numpy(), rows.numpy())
    logits, am, _, _ = dl.lmhead_planned(qtype, w.to(DEV), N, K, h.to(DEV), rows.to(DEV), path=2 if tiled else 0,
                                         confidence=False)
    logits = logits.cpu().numpy(); am = am.cpu().numpy()
    assert_close_rows(logits, ref, f"lmhead qtype={qtype} tiled={tiled} n_rows={n_rows} K={K}")
    _check_argmax(logits, am, ref, ref_am, f"lmhead n_rows={n_rows}")


@pytest.mark.parametrize("K", [768, 1280])
def test_lmhead_q4k_and_ragged_vocab(dl, K):
    N, M = 777, 50
    w = _weights(12, N, K, 14, "lm-q4")
    h = synth.normal_f32((M, K), 14, "lm-q4h")
    rows = synth.distinct_rows(9, M, 14, "rows")
    ref, ref_am = oracle.lmhead(12, w.numpy(), N, K, h.numpy(), rows.numpy())
    logits, am = dl.lmhead_masked(12, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    assert_close_rows(logits.cpu().numpy(), ref, "lmhead q4k")
    _check_argmax(logits.cpu().numpy(), am.cpu().numpy(), ref, ref_am, "lmhead q4k")


@pytest.mark.parametrize("K", [256, 1024])
def test_lmhead_exact_tie_picks_lowest_index(dl, K):
    N, M = 300, 8
    w = _weights(14, N, K, 15, "tie")
    w[200] = w[77]
    w[250] = w[77]
    # make row 77's copies dominate for hidden row 3 by aligning h with them
    wh = oracle.decode_rows(14, w.numpy(), N, K)
    h = synth.normal_f32((M, K), 15, "tie-h")
    h[3] = torch.from_numpy(np.sign(wh[77]).astype(np.float32))
    rows = torch.tensor([3, 1], dtype=torch.int32)
    ref, ref_am = oracle.lmhead(14, w.numpy(), N, K, h.numpy(), rows.numpy())
    assert ref_am[0] == 77
    logits, am = dl.lmhead_masked(14, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    am = am.cpu().numpy()
    lg = logits.cpu().numpy()
    assert lg[0, 77] == lg[0, 200] == lg[0, 250]
    assert am[0] == 77


def _check_confidence(logits, lse, p, ref_logits, what):
    """lse and p(argmax) against (1) the f64 statistics of the GPU's own f32
    logits, which isolates the f32 reduction (exp/log rounding and the merge
    order: a few ulp per term), and (2) the oracle's, within what the logit
    bound allows: the log-sum-exp moves by at most the largest logit error
    e = max_n 1e-4 (|l_n| + rms), and log p = max - lse by at most 2e."""
    own_lse, own_p = oracle.softmax_stats(logits.astype(np.float64))
    assert np.all(np.abs(lse - own_lse) <= 4e-6 * (1.0 + np.abs(own_lse))), f"{what}: lse vs own logits"
    assert np.all(np.abs(p / own_p - 1.0) <= 4e-6 * (1.0 + np.abs(own_lse))), f"{what}: p vs own logits"
    ref_lse, ref_p = oracle.softmax_stats(ref_logits)
    rms = np.sqrt(np.mean(ref_logits ** 2, axis=1))
    e = 1e-4 * (np.abs(ref_logits).max(axis=1) + rms)
    assert np.all(np.abs(lse - ref_lse) <= e + 4e-6 * (1.0 + np.abs(ref_lse))), f"{what}: lse vs oracle"
    assert np.all(np.abs(np.log(p) - np.log(ref_p)) <= 2 * e + 4e-6 * (1.0 + np.abs(ref_lse))), f"{what}: p vs oracle"
    _say(f"{what}: lse {lse[:3]} p(argmax) {p[:3]}")


@pytest.mark.parametrize("qtype", [12, 14])
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("scale", [1.0, 0.002])
def test_lmhead_confidence(dl, qtype, tiled, scale):
    """dllm_lmhead_confidence on both LM-head paths: the same logits and
    argmax as dllm_lmhead_masked, plus the log-sum-exp and the softmax
    probability of the argmax, for peaked (scale 1) and flat (scale 0.002)
    logit rows over a ragged 1000-row vocabulary."""
    N, K, M = 1000, 2048, 148
    _say(f"lmhead confidence qtype={qtype} tiled={tiled} scale={scale}")
    w = _weights(qtype, N, K, 21, f"conf-{qtype}")
    h = synth.normal_f32((M, K), 21, "conf-h") * scale
    rows = synth.distinct_rows(13, M, 21, "conf-rows")
    ref, ref_am = oracle.lmhead(qtype, w.numpy(), N, K, h.numpy(), rows.numpy())
    wd, hd, rd = w.to(DEV), h.to(DEV), rows.to(DEV)
    path = 2 if tiled else 1
    logits, am, lse, p = dl.lmhead_planned(qtype, wd, N, K, hd, rd, path=path)
    logits2, am2, _, _ = dl.lmhead_planned(qtype, wd, N, K, hd, rd, path=path, confidence=False)
    torch.cuda.synchronize()
    assert torch.equal(logits, logits2) and torch.equal(am, am2)
    lg = logits.cpu().numpy()
    assert_close_rows(lg, ref, f"confidence logits qtype={qtype} tiled={tiled}")
    _check_argmax(lg, am.cpu().numpy(), ref, ref_am, "confidence argmax")
    _check_confidence(lg, lse.cpu().numpy().astype(np.float64), p.cpu().numpy().astype(np.float64), ref,
                      f"confidence qtype={qtype} tiled={tiled} scale={scale}")


@pytest.mark.parametrize("M,first", [(148, 20), (160, 128)])
def test_lmhead_full_size(dl, M, first):
    """Masked-row LM head: 32 masked canvas rows (20..51 of 148, or the last
    block 128..159 of a 32 + 128 canvas of 160) x LLaDA's untied 126464 x 4096
    output matrix in Q6_K, against the full oracle."""
    N, K = 126464, 4096
    _say(f"full-size lmhead M={M} rows {first}..{first + 31}")
    w = _weights(14, N, K, 42, "output")
    h = synth.normal_f32((M, K), 42, f"hidden-{M}")
    rows = torch.arange(first, first + 32, dtype=torch.int32)
    ref, ref_am = oracle.lmhead(14, w.numpy(), N, K, h.numpy(), rows.numpy())
    logits, am = dl.lmhead_masked(14, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    logits = logits.cpu().numpy(); am = am.cpu().numpy()
    assert_close_rows(logits, ref, "lmhead full")
    _check_argmax(logits, am, ref, ref_am, "lmhead full")
    # the confidence entry point on the same inputs: same logits, and the
    # statistics over all 126464 logits of each row
    lg2, am2, lse, p = dl.lmhead_confidence(14, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    assert np.array_equal(lg2.cpu().numpy(), logits) and np.array_equal(am2.cpu().numpy(), am)
    _check_confidence(logits, lse.cpu().numpy().astype(np.float64), p.cpu().numpy().astype(np.float64), ref,
                      "lmhead full confidence")


@pytest.mark.parametrize("K", [1024, 1280, 1536])
def test_lmhead_stream_phases(dl, K):
    """The streaming LM head with three 16-row blocks per wave (98304 rows
    over 2048 waves), so that its loop (six steps per iteration in the form
    for an even number of super-blocks per row, three in the other) crosses
    row-block boundaries at every phase: K = 1024 and 1536 (4 and 6
    super-blocks, the even form), K = 1280 (5, the general form); whole
    oracle rows, argmax and ties as everywhere."""
    N, M = 98304, 148
    _say(f"lmhead stream phases K={K}")
    w = _weights(14, N, K, 15, f"lm-phase-{K}")
    h = synth.normal_f32((M, K), 15, f"lm-phase-h-{K}")
    rows = synth.distinct_rows(32, M, 15, f"lm-phase-rows-{K}")
    ref, ref_am = oracle.lmhead(14, w.numpy(), N, K, h.numpy(), rows.numpy())
    logits, am = dl.lmhead_masked(14, w.to(DEV), N, K, h.to(DEV), rows.to(DEV))
    logits = logits.cpu().numpy(); am = am.cpu().numpy()
    assert_close_rows(logits, ref, f"lmhead stream phases K={K}")
    _check_argmax(logits, am, ref, ref_am, f"lmhead stream phases K={K}")
