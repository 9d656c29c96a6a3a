"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before anything is
enqueued (technical specification, error-handling section: explicit,
actionable messages; unsupported types fail with no fallback)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm.h")


@pytest.fixture(scope="module")
def dl():
    import diffusion_lm_gemm_amd as dl
    return dl


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dllm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_header_function(dl):
    names = _header_functions()
    assert len(names) == 20
    lib = ctypes.CDLL(dl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(dl.HEADER_EXPORTS) == names


def test_abi_version_matches_header(dl):
    v = int(re.search(r"#define DLLM_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert dl.abi_version() == v


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation


def test_unsupported_type_message(dl):
    rc = dl.lib.dllm_qgemm(8, FAKE, 64, 256, FAKE, None, 4, FAKE, 64, None, 0, None)
    assert rc == dl.E_UNSUPPORTED
    msg = dl.last_error()
    assert "Q8_0" in msg and "Q4_K and Q6_K" in msg


@pytest.mark.parametrize("K", [0, 100, 257, -256])
def test_k_must_be_multiple_of_256(dl, K):
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 64, K, FAKE, None, 4, FAKE, 64, None, 0, None) == dl.E_SHAPE
    assert dl.lib.dllm_quantize_q8k(FAKE, 4, K, max(K, 1), FAKE, None, None) == dl.E_SHAPE


def test_null_pointers(dl):
    assert dl.lib.dllm_qgemm(dl.Q4_K, None, 64, 256, FAKE, None, 4, FAKE, 64, None, 0, None) == dl.E_ARG
    assert "null" in dl.last_error()
    assert dl.lib.dllm_qgemm(dl.Q6_K, FAKE, 64, 256, FAKE, None, 4, None, 64, None, 0, None) == dl.E_ARG
    assert dl.lib.dllm_quantize_q8k(None, 4, 256, 256, FAKE, None, None) == dl.E_ARG
    assert dl.lib.dllm_decode_qk(dl.Q4_K, None, 1, FAKE, None) == dl.E_ARG


def test_bad_shapes_and_leading_dims(dl):
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 0, 256, FAKE, None, 4, FAKE, 64, None, 0, None) == dl.E_SHAPE
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 64, 256, FAKE, None, 0, FAKE, 64, None, 0, None) == dl.E_SHAPE
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 64, 256, FAKE, None, 4, FAKE, 63, None, 0, None) == dl.E_ARG
    assert dl.lib.dllm_quantize_q8k(FAKE, 4, 512, 500, FAKE, None, None) == dl.E_ARG
    assert dl.lib.dllm_decode_qk(dl.Q6_K, FAKE, 0, FAKE, None) == dl.E_SHAPE


def test_alignment(dl):
    odd = ctypes.c_void_p((1 << 20) + 8)  # 8-byte aligned, not 16
    assert dl.lib.dllm_qgemm(dl.Q4_K, odd, 64, 256, FAKE, None, 4, FAKE, 64, None, 0, None) == dl.E_ALIGN
    two = ctypes.c_void_p((1 << 20) + 2)
    assert dl.lib.dllm_qgemm(dl.Q6_K, two, 64, 256, FAKE, None, 4, FAKE, 64, None, 0, None) == dl.E_ALIGN
    assert dl.lib.dllm_quantize_q8k(two, 4, 256, 256, FAKE, None, None) == dl.E_ALIGN
    # the optional per-token scale summary must be 4-byte aligned too
    assert dl.lib.dllm_quantize_q8k(FAKE, 4, 256, 256, FAKE, two, None) == dl.E_ALIGN
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 64, 256, FAKE, two, 4, FAKE, 64, None, 0, None) == dl.E_ALIGN


def test_oversized_operands_rejected(dl):
    # 2 GiB of Q4_K weights: the kernels address operands with 32-bit offsets
    assert dl.lib.dllm_qgemm(dl.Q4_K, FAKE, 1 << 20, 4096 * 4, FAKE, None, 4, FAKE, 1 << 20, None, 0, None) == dl.E_SHAPE
    assert "2 GiB" in dl.last_error()


def test_lmhead_argument_errors(dl):
    L = dl.lib
    ok_ws = dl.lmhead_workspace_bytes(dl.Q6_K, 1000, 512, 4)
    assert ok_ws > 0
    ws = ctypes.c_void_p(1 << 24)
    # n_rows outside [1, M]
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 3, 512, FAKE, 4, FAKE, 1000, FAKE, ws, ok_ws, None) == dl.E_SHAPE
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 3, 512, FAKE, 0, FAKE, 1000, FAKE, ws, ok_ws, None) == dl.E_SHAPE
    # workspace too small, or missing
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE, ws, ok_ws - 1, None) == dl.E_WORKSPACE
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE, None, ok_ws, None) == dl.E_ARG
    # ldl < N, ldh < K, unaligned workspace
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 999, FAKE, ws, ok_ws, None) == dl.E_ARG
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 256, FAKE, 4, FAKE, 1000, FAKE, ws, ok_ws, None) == dl.E_ARG
    assert L.dllm_lmhead_masked(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE,
                                ctypes.c_void_p((1 << 24) + 16), ok_ws, None) == dl.E_ALIGN


def test_lmhead_confidence_argument_errors(dl):
    L = dl.lib
    ok_ws = dl.lmhead_workspace_bytes(dl.Q6_K, 1000, 512, 4)
    ws = ctypes.c_void_p(1 << 24)
    # lse and p_argmax are required, and 4-byte aligned
    assert L.dllm_lmhead_confidence(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE,
                                    None, FAKE, ws, ok_ws, None) == dl.E_ARG
    assert "lse" in dl.last_error()
    assert L.dllm_lmhead_confidence(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE,
                                    FAKE, None, ws, ok_ws, None) == dl.E_ARG
    assert L.dllm_lmhead_confidence(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE,
                                    ctypes.c_void_p((1 << 20) + 2), FAKE, ws, ok_ws, None) == dl.E_ALIGN
    # the shared checks name this entry point
    assert L.dllm_lmhead_confidence(dl.Q6_K, FAKE, 1000, 512, FAKE, 3, 512, FAKE, 4, FAKE, 1000, FAKE,
                                    FAKE, FAKE, ws, ok_ws, None) == dl.E_SHAPE
    assert "dllm_lmhead_confidence" in dl.last_error()
    assert L.dllm_lmhead_confidence(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE,
                                    FAKE, FAKE, ws, ok_ws - 1, None) == dl.E_WORKSPACE


def test_fused_producer_argument_errors(dl):
    L = dl.lib
    y = FAKE
    # RMSNorm: K a multiple of 256 and at most 16384, ldx >= K, eps in [0, 1], g required
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 300, 300, FAKE, 1e-5, y, None, None) == dl.E_SHAPE
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 16640, 16640, FAKE, 1e-5, y, None, None) == dl.E_SHAPE
    assert "16384" in dl.last_error()
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 512, 256, FAKE, 1e-5, y, None, None) == dl.E_ARG
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 512, 512, None, 1e-5, y, None, None) == dl.E_ARG
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 512, 512, FAKE, -1.0, y, None, None) == dl.E_ARG
    assert L.dllm_rmsnorm_quantize_q8k(FAKE, 4, 512, 512, FAKE, float("nan"), y, None, None) == dl.E_ARG
    assert L.dllm_rmsnorm_quantize_q8k(ctypes.c_void_p((1 << 20) + 2), 4, 512, 512, FAKE, 1e-5, y, None,
                                       None) == dl.E_ALIGN
    # SwiGLU: F a multiple of 256, the row holds gate and up (ldgu >= 2F)
    assert L.dllm_swiglu_quantize_q8k(FAKE, 4, 100, 200, y, None, None) == dl.E_SHAPE
    assert L.dllm_swiglu_quantize_q8k(FAKE, 4, 256, 511, y, None, None) == dl.E_ARG
    assert "ldgu" in dl.last_error()
    assert L.dllm_swiglu_quantize_q8k(None, 4, 256, 512, y, None, None) == dl.E_ARG
    assert L.dllm_swiglu_quantize_q8k(FAKE, 0, 256, 512, y, None, None) == dl.E_SHAPE


def test_attention_argument_errors(dl):
    L = dl.lib
    A = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never dereferenced
    assert L.dllm_attention(A, 148, 3 * 4096, 32, 32, 64, 0.1, A, 4096, None) == dl.E_SHAPE  # D != 128
    assert "128" in dl.last_error()
    assert L.dllm_attention(A, 257, 3 * 4096, 32, 32, 128, 0.1, A, 4096, None) == dl.E_SHAPE  # L > 256
    assert L.dllm_attention(A, 0, 3 * 4096, 32, 32, 128, 0.1, A, 4096, None) == dl.E_SHAPE
    assert L.dllm_attention(A, 148, 3 * 4096 - 4, 32, 32, 128, 0.1, A, 4096, None) == dl.E_ARG
    assert L.dllm_attention(A, 148, 3 * 4096, 32, 32, 128, 0.1, A, 4092, None) == dl.E_ARG
    assert L.dllm_attention(A, 148, 3 * 4096, 32, 32, 128, float("inf"), A, 4096, None) == dl.E_ARG
    assert L.dllm_attention(ctypes.c_void_p((1 << 20) + 4), 148, 3 * 4096, 32, 32, 128, 0.1, A, 4096,
                            None) == dl.E_ALIGN
    assert L.dllm_attention(A, 148, 3 * 4096 + 2, 32, 32, 128, 0.1, A, 4096, None) == dl.E_ALIGN
    assert L.dllm_attention(None, 148, 3 * 4096, 32, 32, 128, 0.1, A, 4096, None) == dl.E_ARG
    # grouped-query attention: H_kv must divide H; the row holds Q of H heads
    # and K, V of H_kv heads (Dream-7B: 28 and 4, (28 + 8) * 128 = 4608)
    assert L.dllm_attention(A, 148, 4608, 28, 5, 128, 0.1, A, 3584, None) == dl.E_SHAPE
    assert "H_kv" in dl.last_error()
    assert L.dllm_attention(A, 148, 4608, 28, 0, 128, 0.1, A, 3584, None) == dl.E_SHAPE
    assert L.dllm_attention(A, 148, 4604, 28, 4, 128, 0.1, A, 3584, None) == dl.E_ARG
    assert L.dllm_attention(A, 148, 4608, 28, 4, 128, 0.1, A, 3580, None) == dl.E_ARG


def test_qgemm_bias_argument_errors(dl):
    L = dl.lib
    FAKE = ctypes.c_void_p(1 << 20)
    # a bias must be 4-byte aligned; the rest are dllm_qgemm's checks
    assert L.dllm_qgemm_bias(dl.Q4_K, FAKE, 64, 256, FAKE, None, 4, ctypes.c_void_p((1 << 20) + 2), FAKE, 64,
                             None, 0, None) == dl.E_ALIGN
    assert "bias" in dl.last_error()
    assert L.dllm_qgemm_bias(dl.Q4_K, FAKE, 64, 300, FAKE, None, 4, FAKE, FAKE, 64, None, 0, None) == dl.E_SHAPE
    assert L.dllm_qgemm_bias(8, FAKE, 64, 256, FAKE, None, 4, FAKE, FAKE, 64, None, 0, None) == dl.E_UNSUPPORTED
    assert L.dllm_qgemm_bias(dl.Q6_K, FAKE, 64, 256, FAKE, None, 4, FAKE, None, 64, None, 0, None) == dl.E_ARG
    assert "dllm_qgemm_bias" in dl.last_error()


def test_workspace_queries(dl):
    # 4096 x 4096 at 148 tokens is split along K; a 126464-row LM head is not.
    assert dl.qgemm_workspace_bytes(dl.Q4_K, 4096, 4096, 148) > 0
    assert dl.qgemm_workspace_bytes(dl.Q6_K, 126464, 4096, 32) == 0
    assert dl.qgemm_workspace_bytes(99, 4096, 4096, 148) == -1
    assert dl.lmhead_workspace_bytes(dl.Q6_K, 126464, 4096, 32) >= 32 * 16 * 292


def test_test_entry_argument_errors(dl):
    """The test-only entry points validate their explicit kernel choice on
    the host: tile configuration 1..7, K split 1..K/256, LM-head path 0..2
    (the streaming path only where it applies), a workspace for a split."""
    L = dl.lib
    big = 1 << 30
    for tile in (0, 8, 32):
        assert L.dllm_qgemm_planned(dl.Q4_K, FAKE, 64, 1024, FAKE, None, 4, None, FAKE, 64, FAKE, big, tile, 1,
                                    None) == dl.E_ARG
        assert "tile" in dl.last_error()
        assert L.dllm_qgemm_superblock_sums_i32(dl.Q6_K, FAKE, 64, 1024, FAKE, 4, FAKE, tile, 1, None) == dl.E_ARG
    for split in (0, 5):
        assert L.dllm_qgemm_planned(dl.Q4_K, FAKE, 64, 1024, FAKE, None, 4, None, FAKE, 64, FAKE, big, 1, split,
                                    None) == dl.E_ARG
        assert "split" in dl.last_error()
        assert L.dllm_qgemm_superblock_sums_i32(dl.Q4_K, FAKE, 64, 1024, FAKE, 4, FAKE, 1, split, None) == dl.E_ARG
    # a split needs a 16-byte aligned workspace of S * M * N * 4 bytes
    assert L.dllm_qgemm_planned(dl.Q4_K, FAKE, 64, 1024, FAKE, None, 4, None, FAKE, 64, None, 0, 1, 2,
                                None) == dl.E_WORKSPACE
    assert L.dllm_qgemm_planned(dl.Q4_K, FAKE, 64, 1024, FAKE, None, 4, None, FAKE, 64, FAKE, 2 * 4 * 64 * 4 - 1, 1,
                                2, None) == dl.E_WORKSPACE
    ok_ws = dl.lmhead_workspace_bytes(dl.Q6_K, 1000, 512, 4)
    ws = ctypes.c_void_p(1 << 24)
    for path in (-1, 3):
        assert L.dllm_lmhead_planned(dl.Q6_K, FAKE, 1000, 512, FAKE, 8, 512, FAKE, 4, FAKE, 1000, FAKE, None, None,
                                     ws, ok_ws, path, None) == dl.E_ARG
        assert "path" in dl.last_error()
    # the streaming kernel takes K <= 4096 and at most 32 rows
    ok_ws = dl.lmhead_workspace_bytes(dl.Q6_K, 1000, 8192, 4)
    assert L.dllm_lmhead_planned(dl.Q6_K, FAKE, 1000, 8192, FAKE, 8, 8192, FAKE, 4, FAKE, 1000, FAKE, None, None,
                                 ws, ok_ws, 1, None) == dl.E_SHAPE
    ok_ws = dl.lmhead_workspace_bytes(dl.Q6_K, 1000, 512, 40)
    assert L.dllm_lmhead_planned(dl.Q6_K, FAKE, 1000, 512, FAKE, 48, 512, FAKE, 40, FAKE, 1000, FAKE, None, None,
                                 ws, ok_ws, 1, None) == dl.E_SHAPE


def test_no_environment_reads_in_the_library():
    """Kernel choice is made by arguments and compiled tables only: the
    library sources read no environment variables."""
    csrc = os.path.join(ROOT, "diffusion_lm_gemm_amd", "csrc")
    for name in os.listdir(csrc):
        if name.endswith((".hip", ".hpp", ".h", ".cpp")):
            assert "getenv" not in open(os.path.join(csrc, name)).read(), name


def test_pair_checks_both_gemms_before_launching(dl):
    """dllm_qgemm_pair reports an error in either GEMM's arguments (or the
    shared ones) before anything is enqueued; its workspace query rejects
    invalid shapes with -1."""
    L = dl.lib
    ok = (dl.Q4_K, FAKE, 64, None, FAKE, 64)
    assert L.dllm_qgemm_pair(*ok, 13, FAKE, 64, None, FAKE, 64, 256, FAKE, None, 1, None, 0, None) == dl.E_UNSUPPORTED
    assert L.dllm_qgemm_pair(8, FAKE, 64, None, FAKE, 64, *ok, 256, FAKE, None, 1, None, 0, None) == dl.E_UNSUPPORTED
    assert L.dllm_qgemm_pair(*ok, dl.Q6_K, FAKE, 64, None, None, 64, 256, FAKE, None, 1, None, 0, None) == dl.E_ARG
    assert L.dllm_qgemm_pair(*ok, dl.Q6_K, None, 64, None, FAKE, 64, 256, FAKE, None, 1, None, 0, None) == dl.E_ARG
    assert L.dllm_qgemm_pair(dl.Q4_K, FAKE, 64, None, FAKE, 63, dl.Q6_K, FAKE, 64, None, FAKE, 64, 256, FAKE, None, 1,
                             None, 0, None) == dl.E_ARG
    assert L.dllm_qgemm_pair(*ok, dl.Q6_K, FAKE, 0, None, FAKE, 64, 256, FAKE, None, 1, None, 0, None) == dl.E_SHAPE
    assert L.dllm_qgemm_pair(*ok, dl.Q6_K, FAKE, 64, None, FAKE, 64, 300, FAKE, None, 1, None, 0, None) == dl.E_SHAPE
    two = ctypes.c_void_p((1 << 20) + 2)
    assert L.dllm_qgemm_pair(*ok, dl.Q6_K, FAKE, 64, two, FAKE, 64, 256, FAKE, None, 1, None, 0, None) == dl.E_ALIGN
    assert dl.qgemm_pair_workspace_bytes(dl.Q4_K, 64, dl.Q6_K, 64, 300, 1) == -1
    assert dl.qgemm_pair_workspace_bytes(dl.Q4_K, 64, 8, 64, 256, 1) == -1
    assert dl.qgemm_pair_workspace_bytes(dl.Q4_K, 8192, dl.Q6_K, 4096, 4096, 148) == (
        dl.qgemm_workspace_bytes(dl.Q6_K, 4096, 4096, 148))  # only V splits: its slices after the counters
