"""Pins for the oracle's bidirectional attention (CPU only).

The pages' layer attends over the whole canvas, bidirectionally (not causal),
after the QKV projection, on f16 tensor cores with a softmax over the keys
(mojo-dllm Technical Specification, "Transformer Execution" and "Critical
difference from autoregressive execution"; README, the GPU bullet).  The
oracle's definition: f16-rounded Q, K, V (the operand format), scores, softmax
and weighted sum in f64.  Pinned by numpy's float16 rounding, closed forms,
key-permutation invariance and an independent numpy/scipy evaluation.  The
grouped-query form (Dream-7B, README milestones: "GQA") is pinned against
numpy with repeated key/value heads, against multi-head attention on heads
written out per query head, and by which query heads a key/value head feeds."""
import numpy as np
from scipy.special import softmax

import oracle


def test_f16_round_matches_numpy():
    rng = np.random.default_rng(61)
    xs = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 20000),
        np.float32([0.0, -0.0, 1.0, 65504.0, 65519.0, 65520.0, -70000.0, 6.1035156e-05, 5.9604645e-08,
                    2.9802322e-08, 2.9802326e-08, 1e-10, 0.1, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):  # the overflow to infinity is part of the rule
        want = xs.astype(np.float16).astype(np.float64)
    got = np.array([oracle.f16_round(v) for v in xs])
    assert np.array_equal(got, want)


def _numpy_attention(qkv, H, D, scale):
    L = qkv.shape[0]
    r = qkv.astype(np.float16).astype(np.float64)
    q = r[:, :H * D].reshape(L, H, D)
    k = r[:, H * D:2 * H * D].reshape(L, H, D)
    v = r[:, 2 * H * D:3 * H * D].reshape(L, H, D)
    s = np.einsum("ihd,jhd->hij", q, k) * scale
    p = softmax(s, axis=2)
    return np.einsum("hij,jhd->ihd", p, v).reshape(L, H * D)


def test_attention_against_numpy_and_scipy():
    rng = np.random.default_rng(62)
    for L, H, D in ((1, 1, 8), (7, 2, 16), (40, 3, 32)):
        qkv = rng.standard_normal((L, 3 * H * D)).astype(np.float32) * 2.0
        got = oracle.attention(qkv, H, D, D ** -0.5)
        assert np.allclose(got, _numpy_attention(qkv, H, D, D ** -0.5), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    """Equal keys: the mean of the values.  One key aligned with the query
    far more than the rest: that key's value.  L = 1: the value itself."""
    rng = np.random.default_rng(63)
    L, H, D = 9, 1, 16
    qkv = rng.standard_normal((L, 3 * D)).astype(np.float32)
    qkv[:, D:2 * D] = qkv[0, D:2 * D]  # every key the same
    got = oracle.attention(qkv, H, D, 0.25)
    v16 = qkv[:, 2 * D:].astype(np.float16).astype(np.float64)
    assert np.allclose(got, v16.mean(axis=0), rtol=1e-13, atol=1e-14)
    qkv = rng.standard_normal((L, 3 * D)).astype(np.float32)
    qkv[:, :D] = 1.0
    qkv[:, D:2 * D] = 0.0
    qkv[5, D:2 * D] = 8.0  # scores 0.25 * 16 * 8 = 32 for key 5, 0 for the rest
    got = oracle.attention(qkv, H, D, 0.25)
    v16 = qkv[:, 2 * D:].astype(np.float16).astype(np.float64)
    w = np.exp(np.float64(-32.0))
    want = (v16[5] + w * (v16.sum(axis=0) - v16[5])) / (1 + 8 * w)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)
    one = rng.standard_normal((1, 3 * D)).astype(np.float32)
    assert np.array_equal(oracle.attention(one, 1, D, 1.0)[0], one[0, 2 * D:].astype(np.float16).astype(np.float64))


def test_attention_is_bidirectional_and_permutation_invariant():
    """Permuting the keys with their values leaves every output unchanged;
    query 0 depends on the last key (no causal mask)."""
    rng = np.random.default_rng(64)
    L, H, D = 12, 2, 8
    qkv = rng.standard_normal((L, 3 * H * D)).astype(np.float32)
    base = oracle.attention(qkv, H, D, 0.5)
    perm = rng.permutation(L)
    kv = qkv[:, H * D:].copy()
    shuffled = np.concatenate([qkv[:, :H * D], kv[perm]], axis=1)
    assert np.allclose(oracle.attention(shuffled, H, D, 0.5), base, rtol=1e-12, atol=1e-14)
    changed = qkv.copy()
    changed[L - 1, 2 * H * D:] += 3.0
    assert not np.allclose(oracle.attention(changed, H, D, 0.5)[0], base[0])


def _numpy_gqa(qkv, H, Hkv, D, scale):
    """Grouped-query attention as multi-head attention on K and V repeated per
    query head (np.repeat: key/value head h // G serves query heads h)."""
    L = qkv.shape[0]
    r = qkv.astype(np.float16).astype(np.float64)
    q = r[:, :H * D].reshape(L, H, D)
    k = np.repeat(r[:, H * D:(H + Hkv) * D].reshape(L, Hkv, D), H // Hkv, axis=1)
    v = np.repeat(r[:, (H + Hkv) * D:(H + 2 * Hkv) * D].reshape(L, Hkv, D), H // Hkv, axis=1)
    s = np.einsum("ihd,jhd->hij", q, k) * scale
    p = softmax(s, axis=2)
    return np.einsum("hij,jhd->ihd", p, v).reshape(L, H * D)


def test_gqa_against_numpy_and_scipy():
    rng = np.random.default_rng(65)
    for L, H, Hkv, D in ((5, 4, 2, 8), (13, 6, 3, 16), (9, 7, 1, 8), (11, 3, 3, 16)):
        qkv = rng.standard_normal((L, (H + 2 * Hkv) * D + 3)).astype(np.float32) * 1.5
        got = oracle.attention(qkv, H, D, D ** -0.5, Hkv=Hkv)
        assert np.allclose(got, _numpy_gqa(qkv[:, :(H + 2 * Hkv) * D], H, Hkv, D, D ** -0.5), rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_on_replicated_heads():
    """GQA over Hkv heads equals plain attention over a Q+K+V row in which each
    key/value head is written out once per query head of its group."""
    rng = np.random.default_rng(66)
    L, H, Hkv, D = 10, 6, 2, 8
    G = H // Hkv
    qkv = rng.standard_normal((L, (H + 2 * Hkv) * D)).astype(np.float32)
    q = qkv[:, :H * D]
    k = qkv[:, H * D:(H + Hkv) * D].reshape(L, Hkv, D)
    v = qkv[:, (H + Hkv) * D:].reshape(L, Hkv, D)
    k_full = np.concatenate([k[:, h // G] for h in range(H)], axis=1)
    v_full = np.concatenate([v[:, h // G] for h in range(H)], axis=1)
    mha = np.concatenate([q, k_full, v_full], axis=1)
    assert np.array_equal(oracle.attention(qkv, H, D, 0.3, Hkv=Hkv), oracle.attention(mha, H, D, 0.3))


def test_gqa_group_mapping():
    """Changing key/value head 1 changes exactly the query heads G .. 2G-1."""
    rng = np.random.default_rng(67)
    L, H, Hkv, D = 8, 6, 3, 8
    G = H // Hkv
    qkv = rng.standard_normal((L, (H + 2 * Hkv) * D)).astype(np.float32)
    base = oracle.attention(qkv, H, D, 0.5, Hkv=Hkv).reshape(L, H, D)
    q2 = qkv.copy()
    q2[:, (H + Hkv + 1) * D:(H + Hkv + 2) * D] += 3.0  # V of key/value head 1
    q2[:, (H + 1) * D:(H + 2) * D] -= 1.0               # K of key/value head 1
    got = oracle.attention(q2, H, D, 0.5, Hkv=Hkv).reshape(L, H, D)
    changed = [h for h in range(H) if not np.array_equal(got[:, h], base[:, h])]
    assert changed == list(range(G, 2 * G))


def test_attention_against_torch_sdpa():
    """torch's own scaled-dot-product attention (CPU, f64, no mask, its
    grouped-query mode) on the same f16-rounded operands: an implementation
    written apart from the oracle, with the same grouping of query heads."""
    import torch
    rng = np.random.default_rng(68)
    for L, H, Hkv, D in ((9, 4, 4, 16), (23, 6, 2, 32), (31, 7, 1, 16)):
        qkv = (rng.standard_normal((L, (H + 2 * Hkv) * D)) * 1.5).astype(np.float32)
        r = torch.from_numpy(qkv.astype(np.float16).astype(np.float64))
        q = r[:, :H * D].reshape(L, H, D).permute(1, 0, 2).unsqueeze(0)
        k = r[:, H * D:(H + Hkv) * D].reshape(L, Hkv, D).permute(1, 0, 2).unsqueeze(0)
        v = r[:, (H + Hkv) * D:].reshape(L, Hkv, D).permute(1, 0, 2).unsqueeze(0)
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=D ** -0.5, enable_gqa=True)
        want = want.squeeze(0).permute(1, 0, 2).reshape(L, H * D).numpy()
        got = oracle.attention(qkv, H, D, D ** -0.5, Hkv=Hkv)
        assert np.allclose(got, want, rtol=1e-11, atol=1e-12)
