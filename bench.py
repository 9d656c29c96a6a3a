"""Benchmark: one denoising step's quantized GEMM stream on one MI355X.

Workload (the whole-step stream of LLaDA-8B Q4_K_M at canvas L = 148; mojo-dllm
Development plan, "Model facts used" and "Compute design"): 32 layers, each
  quantize(x_norm) -> Q,K,V (4096x4096 each) -> quantize(attn) -> O (4096x4096)
  -> quantize(h_norm) -> gate, up (12288x4096 each) -> quantize(act) -> down (4096x12288)
with Q4_K weights except attn_v and ffn_down in Q6_K in the even layers (a
reading of "half the layers"), then the masked-row LM head (32 masked rows
20..51 of the canvas, 126464x4096 Q6_K, f32 logits + argmax).  Q,K,V share an
input and run as one GEMM over their stacked rows when they share a type
(K and V stacked likewise for gate/up); the arithmetic is unchanged.
Weights and activations are seeded synthetic (synth/), resident in HBM before
timing; every layer has its own weights (4.6 GB) and its own f32 inputs.

A step is one replay of a HIP graph holding the whole stream.  Prints ONE
JSON line (rank 0).  `value` is ms per step (lower is better).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per denoising-step GEMM stream (L=148) + int8 TOPS and % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
D, FFN, LAYERS, VOCAB = 4096, 12288, 32, 126464
MASKED = 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--L", type=int, default=148, help="canvas tokens")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dream", action="store_true", help="skip the Dream-7B-shaped step (a reported extra)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    ap.add_argument("--profile-dominant", action="store_true",
                    help="for hardware-counter runs: a 256 MiB device copy (the counters' calibration), then "
                         "--steps launches of the step's dominant GEMM (one layer's gate/up), then exit")
    ap.add_argument("--profile-kernel", choices=("lmhead", "attention", "rmsnorm", "swiglu"), default=None,
                    help="for hardware-counter runs: the same calibration copy, then --steps launches of the masked-row "
                         "LM head (32 rows x 126464 x 4096, Q6_K), of attention (L tokens, 32 heads x 128) or of a fused "
                         "producer (RMSNorm -> Q8_K over 4096 values, SwiGLU -> Q8_K over 2 x 12288), then exit")
    return ap.parse_args()


DOMINANT = ("qgemm_q4k", 2 * FFN, D)  # gate/up: the call that takes most of the step


# Dream-7B's layer dimensions (the model's published configuration; the pages
# name the model, its GQA, QKV bias and 152 064-column output projection)
DREAM = {"D": 3584, "FFN": 18944, "HQ": 28, "HKV": 4, "HD": 128, "LAYERS": 28, "VOCAB": 152064}


def dream_step(dl, synth, torch, dev, L, seed, graph_node_ms):
    """The same step for Dream-7B's shapes (a reported extra, not `value`):
    28 layers of Q+K+V (with their bias; V in Q6_K in even layers), O, gate+up
    and down (Q6_K in even layers), each after a quantize, then the LM head
    over every masked position (the 128 generated rows, logits from the row
    before each).  Captured as one graph, the median of 5 replays; also the
    grouped-query attention of one layer.  Weights are freed afterwards."""
    Q4, Q6 = dl.Q4_K, dl.Q6_K
    D, FFN, HQ, HKV, HD, NL, VOC = (DREAM[k] for k in ("D", "FFN", "HQ", "HKV", "HD", "LAYERS", "VOCAB"))
    NQKV = (HQ + 2 * HKV) * HD
    masked = L - 20
    lay = []
    for l in range(NL):
        even = l % 2 == 0
        lw = {"even": even, "bias": synth.normal_f32((NQKV,), seed, f"D{l:02d}.qkv_bias", dev)}
        if even:
            lw["qk"] = synth.q4k_rows(NQKV - HKV * HD, D, seed, f"D{l:02d}.attn_qk", dev)
            lw["v"] = synth.q6k_rows(HKV * HD, D, seed, f"D{l:02d}.attn_v", dev)
            lw["down"] = synth.q6k_rows(D, FFN, seed, f"D{l:02d}.ffn_down", dev)
        else:
            lw["qkv"] = synth.q4k_rows(NQKV, D, seed, f"D{l:02d}.attn_qkv", dev)
            lw["down"] = synth.q4k_rows(D, FFN, seed, f"D{l:02d}.ffn_down", dev)
        lw["o"] = synth.q4k_rows(D, D, seed, f"D{l:02d}.attn_output", dev)
        lw["gu"] = synth.q4k_rows(2 * FFN, D, seed, f"D{l:02d}.ffn_gate_up", dev)
        lay.append(lw)
    x_d = synth.normal_f32((L, D), seed, "D.x", dev)
    x_f = synth.normal_f32((L, FFN), seed, "D.act", dev)
    w_out = synth.q6k_rows(VOC, D, seed, "D.output", dev)
    hidden = synth.normal_f32((L, D), seed, "D.hidden", dev)
    rows = torch.arange(19, 19 + masked, dtype=torch.int32, device=dev)
    xq_d = torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=dev)
    xq_f = torch.empty((L, FFN // 256 * 292), dtype=torch.uint8, device=dev)
    dm_d = torch.empty(L, dtype=torch.float32, device=dev)
    dm_f = torch.empty(L, dtype=torch.float32, device=dev)
    y_qkv = torch.empty((L, NQKV), dtype=torch.float32, device=dev)
    y_o = torch.empty((L, D), dtype=torch.float32, device=dev)
    y_gu = torch.empty((L, 2 * FFN), dtype=torch.float32, device=dev)
    y_dn = torch.empty((L, D), dtype=torch.float32, device=dev)
    logits = torch.empty((masked, VOC), dtype=torch.float32, device=dev)
    amax = torch.empty(masked, dtype=torch.int32, device=dev)
    shapes = [(Q4, NQKV - HKV * HD, D), (Q6, HKV * HD, D), (Q4, NQKV, D), (Q4, D, D), (Q4, 2 * FFN, D),
              (Q4, D, FFN), (Q6, D, FFN)]
    ws = torch.zeros(max(256, max(dl.qgemm_workspace_bytes(q, n, k, L) for q, n, k in shapes)),
                     dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(dl.lmhead_workspace_bytes(Q6, VOC, D, masked), dtype=torch.uint8, device=dev)
    fns, byts, ops = [], 0, 0

    def quant(x, out, dm):
        nonlocal byts
        fns.append(lambda: dl.quantize_q8k(x, out, dm))
        byts += x.numel() * 4 + x.numel() // 256 * 292

    def gemm(q, w, N, K, xq, dm, y, bias=None):
        nonlocal byts, ops
        fns.append(lambda: dl.qgemm(q, w, N, K, xq, L, y=y, workspace=ws, x_dmax=dm, bias=bias))
        byts += N * K // 256 * dl.block_bytes(q) + L * K // 256 * 292 + L * N * 4
        ops += 2 * L * N * K

    for lw in lay:
        quant(x_d, xq_d, dm_d)
        if lw["even"]:
            nqk = NQKV - HKV * HD
            gemm(Q4, lw["qk"], nqk, D, xq_d, dm_d, y_qkv[:, :nqk], lw["bias"][:nqk])
            gemm(Q6, lw["v"], HKV * HD, D, xq_d, dm_d, y_qkv[:, nqk:], lw["bias"][nqk:])
        else:
            gemm(Q4, lw["qkv"], NQKV, D, xq_d, dm_d, y_qkv, lw["bias"])
        quant(x_d, xq_d, dm_d)
        gemm(Q4, lw["o"], D, D, xq_d, dm_d, y_o)
        quant(x_d, xq_d, dm_d)
        gemm(Q4, lw["gu"], 2 * FFN, D, xq_d, dm_d, y_gu)
        quant(x_f, xq_f, dm_f)
        gemm(Q6 if lw["even"] else Q4, lw["down"], D, FFN, xq_f, dm_f, y_dn)
    fns.append(lambda: dl.lmhead_masked(Q6, w_out, VOC, D, hidden, rows, logits, amax, ws_lm))
    byts += masked * D * 4 + masked * D // 256 * 292 + VOC * D // 256 * dl.block_bytes(Q6) + masked * VOC * 4
    ops += 2 * masked * VOC * D
    step_ms = graph_node_ms(fns) * len(fns)
    attn_out = torch.empty((L, HQ * HD), dtype=torch.float32, device=dev)
    a_ms = graph_node_ms([lambda: dl.attention(y_qkv, HQ, HD, None, attn_out, H_kv=HKV)] * 20)
    out = {"ms_per_step": round(step_ms, 4), "int8_TOPS": round(ops / (step_ms * 1e-3) / 1e12, 2),
           "GBps": round(byts / (step_ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(byts / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "calls_per_step": len(fns), "step_algorithmic_bytes": byts,
           "attention_gqa": {"avg_ms": round(a_ms, 5), "shape": f"L={L}, {HQ} query / {HKV} key-value heads x {HD}",
                             "in_step": False},
           "workload": f"Dream-7B Q4_K_M shapes, L={L}: {NL} layers (Q+K+V {NQKV}x{D} with bias, O {D}x{D}, "
                       f"gate+up {2 * FFN}x{D}, down {D}x{FFN}; attn_v/ffn_down Q6_K in even layers) + LM head "
                       f"{masked}x{VOC}x{D} Q6_K over every masked row",
           "timing": "one graph of the step's calls, median of 5 replays"}
    del lay, w_out
    torch.cuda.empty_cache()
    return out


def profile_dominant(args):
    """A known-size copy kernel (FETCH_SIZE / WRITE_SIZE of it calibrate the
    counters), then the dominant GEMM call alone, as in the step."""
    import torch
    import diffusion_lm_gemm_amd as dl
    import synth
    dev = torch.device("cuda:0")
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    _, N, K = DOMINANT
    L = args.L
    w = synth.q4k_rows(N, K, args.seed, "L01.ffn_gate_up", dev)
    dmax = torch.empty(L, dtype=torch.float32, device=dev)
    xq = dl.quantize_q8k(synth.normal_f32((L, K), args.seed, "L01.h_norm", dev), dmax=dmax)
    y = torch.empty((L, N), dtype=torch.float32, device=dev)
    ws = dl.qgemm_workspace(dl.Q4_K, N, K, L, dev)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        dl.qgemm(dl.Q4_K, w, N, K, xq, L, y=y, workspace=ws, x_dmax=dmax)
    torch.cuda.synchronize()
    print(f"[profile-dominant] copy of {a.numel() * 4} bytes, then {args.steps} x qgemm Q4_K N={N} K={K} M={L}",
          flush=True)


def profile_kernel(args):
    """The calibration copy of profile_dominant, then --steps launches of one
    other call of the path: the masked-row LM head or bidirectional attention,
    on inputs of the step's shapes."""
    import torch
    import diffusion_lm_gemm_amd as dl
    import synth
    dev = torch.device("cuda:0")
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    L = args.L
    if args.profile_kernel == "lmhead":
        w = synth.q6k_rows(VOCAB, D, args.seed, "output", dev)
        hidden = synth.normal_f32((L, D), args.seed, "hidden", dev)
        rows = torch.arange(20, 20 + MASKED, dtype=torch.int32, device=dev)
        logits = torch.empty((MASKED, VOCAB), dtype=torch.float32, device=dev)
        amax = torch.empty(MASKED, dtype=torch.int32, device=dev)
        ws = torch.empty(dl.lmhead_workspace_bytes(dl.Q6_K, VOCAB, D, MASKED), dtype=torch.uint8, device=dev)
        fn = lambda: dl.lmhead_masked(dl.Q6_K, w, VOCAB, D, hidden, rows, logits, amax, ws)
        what = f"lmhead_masked Q6_K N={VOCAB} K={D} rows={MASKED} of M={L}"
    elif args.profile_kernel == "attention":
        qkv = synth.normal_f32((L, 3 * D), args.seed, "qkv", dev)
        out = torch.empty((L, D), dtype=torch.float32, device=dev)
        fn = lambda: dl.attention(qkv, 32, 128, None, out)
        what = f"attention L={L} H=32 D=128"
    elif args.profile_kernel == "rmsnorm":
        x = synth.normal_f32((L, D), args.seed, "x_norm", dev)
        g = synth.normal_f32((D,), args.seed, "norm_weight", dev)
        xq = torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=dev)
        dm = torch.empty(L, dtype=torch.float32, device=dev)
        fn = lambda: dl.rmsnorm_quantize_q8k(x, g, 1e-5, xq, dm)
        what = f"rmsnorm_quantize_q8k M={L} K={D}"
    else:
        gu = synth.normal_f32((L, 2 * FFN), args.seed, "gate_up", dev)
        xq = torch.empty((L, FFN // 256 * 292), dtype=torch.uint8, device=dev)
        dm = torch.empty(L, dtype=torch.float32, device=dev)
        fn = lambda: dl.swiglu_quantize_q8k(gu, xq, dm)
        what = f"swiglu_quantize_q8k M={L} F={FFN}"
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    print(f"[profile-kernel] copy of {a.numel() * 4} bytes, then {args.steps} x {what}", flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py runs on one GPU only: this build has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    if args.profile_dominant:
        profile_dominant(args)
        return
    if args.profile_kernel:
        profile_kernel(args)
        return

    import torch
    import diffusion_lm_gemm_amd as dl
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, seed = args.L, args.seed
    Q4, Q6 = dl.Q4_K, dl.Q6_K

    def bb(q):
        return dl.block_bytes(q)

    # ---------------- weights and inputs (resident before timing) ----------
    t_setup = time.time()
    layers = []
    for l in range(LAYERS):
        even = (l % 2 == 0)
        lw = {"even": even}
        if even:  # V is Q6_K: Q and K stacked, V alone
            lw["qk"] = synth.q4k_rows(2 * D, D, seed, f"L{l:02d}.attn_qk", dev)
            lw["v"] = synth.q6k_rows(D, D, seed, f"L{l:02d}.attn_v", dev)
            lw["down"] = synth.q6k_rows(D, FFN, seed, f"L{l:02d}.ffn_down", dev)
        else:
            lw["qkv"] = synth.q4k_rows(3 * D, D, seed, f"L{l:02d}.attn_qkv", dev)
            lw["down"] = synth.q4k_rows(D, FFN, seed, f"L{l:02d}.ffn_down", dev)
        lw["o"] = synth.q4k_rows(D, D, seed, f"L{l:02d}.attn_output", dev)
        lw["gu"] = synth.q4k_rows(2 * FFN, D, seed, f"L{l:02d}.ffn_gate_up", dev)
        lw["x_norm"] = synth.normal_f32((L, D), seed, f"L{l:02d}.x_norm", dev)
        lw["attn"] = synth.normal_f32((L, D), seed, f"L{l:02d}.attn", dev)
        lw["h_norm"] = synth.normal_f32((L, D), seed, f"L{l:02d}.h_norm", dev)
        lw["act"] = synth.normal_f32((L, FFN), seed, f"L{l:02d}.act", dev)
        layers.append(lw)
    w_out = synth.q6k_rows(VOCAB, D, seed, "output", dev)
    hidden = synth.normal_f32((L, D), seed, "hidden", dev)
    rows = torch.arange(20, 20 + MASKED, dtype=torch.int32, device=dev)

    xq_d = torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=dev)
    xq_f = torch.empty((L, FFN // 256 * 292), dtype=torch.uint8, device=dev)
    dmax_d = torch.empty(L, dtype=torch.float32, device=dev)  # per-token largest |d|
    dmax_f = torch.empty(L, dtype=torch.float32, device=dev)
    y_qkv = torch.empty((L, 3 * D), dtype=torch.float32, device=dev)
    y_o = torch.empty((L, D), dtype=torch.float32, device=dev)
    y_gu = torch.empty((L, 2 * FFN), dtype=torch.float32, device=dev)
    y_down = torch.empty((L, D), dtype=torch.float32, device=dev)
    logits = torch.empty((MASKED, VOCAB), dtype=torch.float32, device=dev)
    amax = torch.empty(MASKED, dtype=torch.int32, device=dev)
    ws_bytes = max(dl.qgemm_workspace_bytes(q, n, k, L) for q, n, k in
                   [(Q4, 3 * D, D), (Q4, 2 * D, D), (Q6, D, D), (Q4, D, D), (Q4, 2 * FFN, D),
                    (Q4, D, FFN), (Q6, D, FFN)])
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    ws_lm = torch.empty(dl.lmhead_workspace_bytes(Q6, VOCAB, D, MASKED), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # ---------------- the step as a list of calls --------------------------
    calls = []  # (kind, fn, algorithmic bytes, int8 ops)

    def add_quant(x, out, dmax):
        M, K = x.shape
        calls.append(("quantize_q8k", lambda: dl.quantize_q8k(x, out, dmax),
                      M * K * 4 + M * K // 256 * 292 + M * 4, 0, ("quantize_q8k", M, K)))

    def add_gemm(q, w, N, K, xq, dmax, y):
        byts = N * K // 256 * bb(q) + L * K // 256 * 292 + L * N * 4
        kind = "qgemm_q4k" if q == Q4 else "qgemm_q6k"
        calls.append((kind, lambda: dl.qgemm(q, w, N, K, xq, L, y=y, workspace=ws, x_dmax=dmax), byts,
                      2 * L * N * K, (kind, N, K)))

    for lw in layers:
        add_quant(lw["x_norm"], xq_d, dmax_d)
        if lw["even"]:
            add_gemm(Q4, lw["qk"], 2 * D, D, xq_d, dmax_d, y_qkv[:, :2 * D])
            add_gemm(Q6, lw["v"], D, D, xq_d, dmax_d, y_qkv[:, 2 * D:])
        else:
            add_gemm(Q4, lw["qkv"], 3 * D, D, xq_d, dmax_d, y_qkv)
        add_quant(lw["attn"], xq_d, dmax_d)
        add_gemm(Q4, lw["o"], D, D, xq_d, dmax_d, y_o)
        add_quant(lw["h_norm"], xq_d, dmax_d)
        add_gemm(Q4, lw["gu"], 2 * FFN, D, xq_d, dmax_d, y_gu)
        add_quant(lw["act"], xq_f, dmax_f)
        add_gemm(Q6 if lw["even"] else Q4, lw["down"], D, FFN, xq_f, dmax_f, y_down)
    lm_bytes = (MASKED * D * 4 + MASKED * D // 256 * 292 + VOCAB * D // 256 * bb(Q6)
                + MASKED * VOCAB * 4 + MASKED * 4)
    calls.append(("lmhead_q6k", lambda: dl.lmhead_masked(Q6, w_out, VOCAB, D, hidden, rows, logits, amax, ws_lm),
                  lm_bytes, 2 * MASKED * VOCAB * D, ("lmhead_q6k", VOCAB, D)))
    step_bytes = sum(c[2] for c in calls)
    step_ops = sum(c[3] for c in calls)

    def run_step():
        for c in calls:
            c[1]()

    # ---------------- graph capture and timed replays ----------------------
    run_step()  # eager warm-up (also loads every code object)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run_step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] setup {t_setup:.1f}s; {len(calls)} calls/step; graph: {ms_step:.4f} ms/step "
          f"(wall {1e3 * wall / args.steps:.4f} ms/step)", file=sys.stderr, flush=True)

    # ---------------- per-call durations (eager, HIP events on the launch stream)
    # Every call is bracketed by events on the stream it is launched on; calls
    # are grouped by kind and by shape.
    reps = 3
    per = {}
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
    for _ in range(reps):
        for (a, b), c in zip(evs, calls):
            a.record()
            c[1]()
            b.record()
        torch.cuda.synchronize()
        for (a, b), c in zip(evs, calls):
            for key in (c[0], c[4]):
                k = per.setdefault(key, [0.0, 0, 0, 0])
                k[0] += a.elapsed_time(b)
                k[1] += 1
                k[2] += c[2]
                k[3] += c[3]

    def stats(key):
        ms, n, byts, ops = per[key]
        return {"launches_per_step": n // reps, "avg_ms": ms / n, "GBps": byts / (ms * 1e-3) / 1e9,
                "TOPS": ops / (ms * 1e-3) / 1e12 if ops else 0.0}
    kind_keys = [k for k in per if isinstance(k, str)]
    shape_keys = [k for k in per if isinstance(k, tuple)]
    tot = sum(per[k][0] for k in kind_keys)
    kinds = {k: dict(stats(k), share_of_eager_time=per[k][0] / tot) for k in kind_keys}
    shapes = {f"{k[0]} {k[1]}x{k[2]}": dict(stats(k), share_of_eager_time=per[k][0] / tot) for k in shape_keys}
    def graph_node_ms(fns, replays=5):
        """Per call, as the nodes of a replayed graph of the given calls in
        order (captured and replayed like the step), between HIP events on the
        stream the graph runs on; median of the replays."""
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        fg = torch.cuda.CUDAGraph()
        fs = torch.cuda.Stream()
        fs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(fs):
            with torch.cuda.graph(fg, stream=fs):
                for fn in fns:
                    fn()
        torch.cuda.current_stream().wait_stream(fs)
        fg.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fg.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / len(fns))
        return sorted(times)[replays // 2]

    # the dominant kind of call: its calls in the eager pass above, in step
    # order, each between HIP events on its launch stream (the events also
    # hold the dispatch of the call between them)
    dom = max(shape_keys, key=lambda k: per[k][0])
    dms, dn, dbytes, dops = per[dom]
    dom_call_ms = dms / dn
    dom_bytes, dom_ops = dbytes // dn, dops // dn  # per call
    dom_name = f"{dom[0]}_{dom[1]}x{dom[2]}"
    achieved = dom_bytes / (dom_call_ms * 1e-3) / 1e9
    # the LM head with the greedy pick's confidence (log-sum-exp and softmax
    # probability of the argmax per masked row; not part of the step), timed
    # the same way on the same inputs
    lse = torch.empty(MASKED, dtype=torch.float32, device=dev)
    p_am = torch.empty(MASKED, dtype=torch.float32, device=dev)
    conf = lambda: dl.lmhead_confidence(Q6, w_out, VOCAB, D, hidden, rows, logits, amax, lse, p_am, ws_lm)
    conf()
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in cev:
        a.record()
        conf()
        b.record()
    torch.cuda.synchronize()
    conf_ms = sum(a.elapsed_time(b) for a, b in cev) / reps

    # the fused producers of the quantized activations (not part of the step):
    # RMSNorm -> Q8_K on a layer input, SwiGLU -> Q8_K on the gate/up output,
    # against the plain quantizer on the f32 tensors they replace
    g_norm = synth.normal_f32((D,), seed, "norm_weight", dev)
    fused = {
        "rmsnorm_quantize_q8k": (lambda: dl.rmsnorm_quantize_q8k(layers[0]["x_norm"], g_norm, 1e-5, xq_d, dmax_d),
                                 L * D * 4 + D * 4 + L * D // 256 * 292),
        "quantize_q8k_after_rmsnorm": (lambda: dl.quantize_q8k(layers[0]["x_norm"], xq_d, dmax_d),
                                       L * D * 4 + L * D // 256 * 292),
        "swiglu_quantize_q8k": (lambda: dl.swiglu_quantize_q8k(y_gu, xq_f, dmax_f),
                                L * 2 * FFN * 4 + L * FFN // 256 * 292),
        "quantize_q8k_after_swiglu": (lambda: dl.quantize_q8k(layers[0]["act"], xq_f, dmax_f),
                                      L * FFN * 4 + L * FFN // 256 * 292),
    }

    fused_out = {}
    for name, (fn, byts) in fused.items():
        fms = graph_node_ms([fn] * 20)
        fused_out[name] = {"avg_ms": round(fms, 5), "GBps": round(byts / (fms * 1e-3) / 1e9, 1)}

    # bidirectional attention on the Q+K+V projection's output (not part of
    # the step): 32 heads of 128 over the L-token canvas
    attn_out = torch.empty((L, D), dtype=torch.float32, device=dev)
    a_ms = graph_node_ms([lambda: dl.attention(y_qkv, 32, 128, None, attn_out)] * 20)
    a_flops = 4 * L * L * D
    attention = {"avg_ms": round(a_ms, 5), "TFLOPs": round(a_flops / (a_ms * 1e-3) / 1e12, 2),
                 "GBps": round((L * 3 * D * 4 + L * D * 4) / (a_ms * 1e-3) / 1e9, 1),
                 "shape": f"L={L}, 32 heads x 128, f16 operands", "in_step": False}
    dream = None if args.no_dream else dream_step(dl, synth, torch, dev, L, seed, graph_node_ms)
    if dream:
        print(f"[bench] dream-7B step: {dream['ms_per_step']} ms", file=sys.stderr, flush=True)
    print(f"[bench] per-call kinds: " + json.dumps(kinds), file=sys.stderr, flush=True)
    print(f"[bench] per-call shapes: " + json.dumps(shapes), file=sys.stderr, flush=True)

    # ---------------- HBM traffic from committed counter summaries ---------
    # FETCH_SIZE + WRITE_SIZE of the dominant call's kernel, scaled by the
    # same counters on a copy of known size; valid only for the kernel
    # sources it was measured on.
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{dom_name}_L{L}.txt")
    if os.path.exists(tpath):
        kv = dict(l.split("=", 1) for l in open(tpath).read().split() if "=" in l)
        src_hash = _kernel_hash()
        if kv.get("kernel_sha") == src_hash and "bytes_per_call" in kv:
            traffic = float(kv["bytes_per_call"])

    # ---------------- CPU oracle baseline (bounded sample) -----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, step_ops // 2)

    step_s = ms_step * 1e-3
    out = {
        "metric": METRIC,
        "value": round(ms_step, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"whole denoising-step GEMM stream, LLaDA-8B Q4_K_M shapes, L={L}: "
                               f"32 layers (Q,K,V,O 4096x4096; gate,up 12288x4096; down 4096x12288; "
                               f"attn_v/ffn_down Q6_K in even layers) + masked LM head 32x126464x4096 Q6_K",
                   "L": L, "layers": LAYERS, "masked_rows": MASKED, "calls_per_step": len(calls),
                   "launch": "one HIP graph replay per step"},
        "step_int8_TOPS": round(step_ops / step_s / 1e12, 2),
        "step_GBps": round(step_bytes / step_s / 1e9, 1),
        "step_frac_hbm": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_frac_mfma": round(step_ops / step_s / 1e12 / INT8_PEAK_TOPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "step_int8_ops": step_ops,
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_call_ms": round(dom_call_ms, 5), "calls_per_step": dn // reps,
                     "timing": "each call of one eager step pass between HIP events on its launch stream",
                     "algorithmic_bytes_per_call": dom_bytes,
                     "int8_TOPS": round(dom_ops / (dom_call_ms * 1e-3) / 1e12, 2),
                     "frac_mfma": round(dom_ops / (dom_call_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)},
        "per_call_kind": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                          for k, v in kinds.items()},
        "per_call_shape": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                           for k, v in shapes.items()},
        "lmhead_confidence": {"avg_ms": round(conf_ms, 5), "GBps": round(lm_bytes / (conf_ms * 1e-3) / 1e9, 1),
                              "outputs": "logits, argmax, log-sum-exp and p(argmax) per masked row",
                              "in_step": False},
        "fused_producers": dict(fused_out, in_step=False),
        "attention": attention,
        "dream_step": dream,
        "cpu_baseline": cpu,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


def _kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("common.hpp", "kernels.hpp", "unpack.hpp", "qgemm.hip", "quantize.hip", "abi.hip"):
        h.update(open(os.path.join(ROOT, "diffusion_lm_gemm_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(args, step_macs: int):
    """The oracle (plain f64 C, threads over output rows) on a bounded sample of
    the step: Q4_K layers of 4096 x 4096 and Q6_K 4096 x 12288 rows at L
    tokens, grown until about --cpu-seconds of CPU work, then scaled to ms per
    step by the step's MAC count."""
    import numpy as np
    import oracle
    import synth
    L = args.L
    nt = oracle.default_threads()
    x4 = oracle.quantize_q8k(synth.normal_f32((L, D), 1, "cpu-x4").numpy())
    x12 = oracle.quantize_q8k(synth.normal_f32((L, FFN), 1, "cpu-x12").numpy())
    # one Q4_K 4096 x 4096 layer and one Q6_K 4096 x 12288 layer at L tokens,
    # repeated until about --cpu-seconds have passed
    w4 = synth.q4k_rows(D, D, 1, "cpu-w4").numpy()
    w6 = synth.q6k_rows(D, FFN, 1, "cpu-w6").numpy()
    macs, secs, reps = 0, 0.0, 0
    t0 = time.perf_counter()
    while secs < args.cpu_seconds:
        oracle.gemm(12, w4, D, D, x4, L, nt)
        oracle.gemm(14, w6, D, FFN, x12, L, nt)
        reps += 1
        macs += D * L * (D + FFN)
        secs = time.perf_counter() - t0
    rate = macs / secs
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(step_macs / rate * 1e3, 1), "unit": "ms", "cores": nt, "kind": "oracle",
            "sample": f"{reps} x (oracle f64 GEMM of a Q4_K 4096x4096 layer + a Q6_K 4096x12288 layer at {L} tokens): "
                      f"{macs / 1e9:.1f} G MAC in {secs:.2f} s = {rate / 1e9:.2f} GMAC/s, scaled to the step's "
                      f"{step_macs / 1e12:.3f} T MAC",
            "cpu": cpu_model or platform.processor()}


if __name__ == "__main__":
    main()
