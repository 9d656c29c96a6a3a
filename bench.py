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
    ap.add_argument("--no-l160", action="store_true", help="skip the L=160 step (a reported extra)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"), default=None,
                    help="write profiles/OUT from the rocprofv3 --kernel-trace --stats output in DIR (libdllm "
                         "kernels: calls, average and share per kernel and launch shape), then exit")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("TARGET", "DIR_PREFIX", "OUT"), default=None,
                    help="write profiles/OUT from FETCH_SIZE and WRITE_SIZE passes DIR_PREFIX_FETCH_SIZE and "
                         "DIR_PREFIX_WRITE_SIZE of a --profile-kernel TARGET run (or --profile-dominant for TARGET "
                         "dominant), scaled by the same counters on the run's 256 MiB copy, then exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("TARGET", "DIR_PREFIX"), default=None,
                    help="write profiles/mfma_<kernel>.txt from the counter passes DIR_PREFIX_{A,B,C} of a "
                         "--profile-kernel TARGET run (rocprofv3 --pmc ... --output-format csv), then exit")
    ap.add_argument("--profile-dominant", action="store_true",
                    help="for hardware-counter runs: a 256 MiB device copy (the counters' calibration), then "
                         "--steps launches of the step's dominant GEMM (one layer's gate/up), then exit")
    ap.add_argument("--profile-kernel", choices=("lmhead", "attention", "rmsnorm", "swiglu", "pair") + tuple(STEP_CALLS),
                    default=None,
                    help="for hardware-counter runs: the same calibration copy, then --steps launches of one call of "
                         "the step as the step makes it (" + ", ".join(f"{k}: {v[3]}" for k, v in STEP_CALLS.items()) +
                         "), of the masked-row LM head (32 rows x 126464 x 4096, Q6_K), of attention (L tokens, 32 "
                         "heads x 128) or of a fused producer (RMSNorm -> Q8_K over 4096 values, SwiGLU -> Q8_K over "
                         "2 x 12288), then exit")
    return ap.parse_args()


DOMINANT = ("qgemm_q4k", 2 * FFN, D)  # gate/up: the call that takes most of the step

# Hardware-counter passes (each a separate rocprofv3 --pmc run of
# `bench.py --profile-kernel TARGET --steps 5`; at most 8 SQ and 2 GRBM
# counters per pass) and the summary file each target's figures go to.
PMC_PASSES = {
    "A": "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_LDS SQ_INSTS_VMEM SQ_INSTS_SALU "
         "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
    "B": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
         "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "C": "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_SCA SQ_VALU_MFMA_COEXEC_CYCLES SQ_INST_LEVEL_LDS "
         "SQ_LEVEL_WAVES SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_CYCLES GRBM_GUI_ACTIVE",
}
PMC_TARGETS = {
    "gateup": "qgemm_q4k_24576x4096_L148", "o": "qgemm_q4k_4096x4096_L148", "down6": "qgemm_q6k_4096x12288_L148",
    "v6": "qgemm_q6k_4096x4096_L148", "quant4096": "quantize_q8k_148x4096", "lmhead": "lmhead_q6k_126464x4096_rows32",
    "pair": "qgemm_pair_q4k8192_q6k4096x4096_L148",
}
CUS, SIMDS, XCDS = 256, 4, 8  # MI355X

# The step's calls by name: (kind, N, K, description); kind 12 / 14 is a GEMM
# of that weight type, 0 the quantizer over K values per token.
STEP_CALLS = {
    "gateup": (12, 2 * FFN, D, "gate+up Q4_K 24576x4096"),
    "qkv": (12, 3 * D, D, "Q+K+V Q4_K 12288x4096"),
    "qk": (12, 2 * D, D, "Q+K Q4_K 8192x4096"),
    "o": (12, D, D, "O Q4_K 4096x4096"),
    "v6": (14, D, D, "V Q6_K 4096x4096"),
    "down4": (12, D, FFN, "down Q4_K 4096x12288"),
    "down6": (14, D, FFN, "down Q6_K 4096x12288"),
    "quant4096": (0, 0, D, "quantize_q8k Lx4096"),
    "quant12288": (0, 0, FFN, "quantize_q8k Lx12288"),
}


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
    nqk = NQKV - HKV * HD
    ws = torch.zeros(max(256, max(dl.qgemm_workspace_bytes(q, n, k, L) for q, n, k in shapes),
                         dl.qgemm_pair_workspace_bytes(Q4, nqk, Q6, HKV * HD, D, L)), dtype=torch.uint8, device=dev)
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
        if lw["even"]:  # Q + K (Q4_K) and V (Q6_K) in one launch
            fns.append(lambda lw=lw: dl.qgemm_pair((Q4, lw["qk"], nqk, y_qkv[:, :nqk], lw["bias"][:nqk]),
                                                   (Q6, lw["v"], HKV * HD, y_qkv[:, nqk:], lw["bias"][nqk:]), D,
                                                   xq_d, L, workspace=ws, x_dmax=dm_d))
            byts += (nqk * D // 256 * dl.block_bytes(Q4) + HKV * HD * D // 256 * dl.block_bytes(Q6)
                     + L * D // 256 * 292 + L * NQKV * 4)
            ops += 2 * L * NQKV * D
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
    if args.profile_kernel in STEP_CALLS:
        q, N, K, what = STEP_CALLS[args.profile_kernel]
        x = synth.normal_f32((L, K), args.seed, f"prof-x-{K}", dev)
        xq = torch.empty((L, K // 256 * 292), dtype=torch.uint8, device=dev)
        dm = torch.empty(L, dtype=torch.float32, device=dev)
        dl.quantize_q8k(x, xq, dm)
        if q == 0:
            fn = lambda: dl.quantize_q8k(x, xq, dm)
        else:
            w = (synth.q4k_rows if q == dl.Q4_K else synth.q6k_rows)(N, K, args.seed, f"prof-w-{q}-{N}-{K}", dev)
            y = torch.empty((L, N), dtype=torch.float32, device=dev)
            ws = dl.qgemm_workspace(q, N, K, L, dev)
            fn = lambda: dl.qgemm(q, w, N, K, xq, L, y=y, workspace=ws, x_dmax=dm)
        what = f"{what}, L={L}"
    elif args.profile_kernel == "pair":
        # an even layer's Q + K (Q4_K) and V (Q6_K) projections, one launch
        x = synth.normal_f32((L, D), args.seed, f"prof-x-{D}", dev)
        xq = torch.empty((L, D // 256 * 292), dtype=torch.uint8, device=dev)
        dm = torch.empty(L, dtype=torch.float32, device=dev)
        dl.quantize_q8k(x, xq, dm)
        wa = synth.q4k_rows(2 * D, D, args.seed, f"prof-w-12-{2 * D}-{D}", dev)
        wb = synth.q6k_rows(D, D, args.seed, f"prof-w-14-{D}-{D}", dev)
        y = torch.empty((L, 3 * D), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(256, dl.qgemm_pair_workspace_bytes(dl.Q4_K, 2 * D, dl.Q6_K, D, D, L)),
                         dtype=torch.uint8, device=dev)
        fn = lambda: dl.qgemm_pair((dl.Q4_K, wa, 2 * D, y[:, :2 * D], None), (dl.Q6_K, wb, D, y[:, 2 * D:], None), D,
                                   xq, L, workspace=ws, x_dmax=dm)
        what = f"qgemm_pair Q+K Q4_K {2 * D}x{D} with V Q6_K {D}x{D}, L={L}"
    elif args.profile_kernel == "lmhead":
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


def capture(torch, fns):
    """One HIP graph of the calls in order (each run once eagerly first, which
    also loads every code object)."""
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for fn in fns:
                fn()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    return g


def time_replays(torch, g, n_total, batches):
    """n_total replays of graph g in `batches` batches, each batch between HIP
    events on the stream the replays run on: ms per replay of each batch."""
    sizes = [n_total // batches + (1 if b < n_total % batches else 0) for b in range(batches)]
    out = []
    for n in sizes:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / n)
    return out


def med(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def counter_summary(name: str):
    """Hardware-counter figures of a kernel from profiles/mfma_<name>.txt, if
    they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"mfma_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = dict(l.split("=", 1) for l in open(path).read().split() if "=" in l)
    if kv.get("kernel_sha") != _kernel_hash():
        return {"stale": True, "file": os.path.relpath(path, ROOT)}
    keep = ("mfma_util", "valu_per_mfma", "valu_active", "wait_any", "lds_bank_conflict_frac", "counter_TOPS_i8")
    return {k: float(kv[k]) for k in keep if k in kv} | {"file": os.path.relpath(path, ROOT)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py runs on one GPU only: this build has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
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
    GiB = 1 << 30

    def bb(q):
        return dl.block_bytes(q)

    # ---------------- weights (resident before timing) ---------------------
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
        layers.append(lw)
    w_out = synth.q6k_rows(VOCAB, D, seed, "output", dev)

    def build_step(Lc):
        """The step's calls at a canvas of Lc tokens, each layer with its own
        f32 inputs: [(kind, fn, algorithmic bytes, int8 ops, shape key)]."""
        xq_d = torch.empty((Lc, D // 256 * 292), dtype=torch.uint8, device=dev)
        xq_f = torch.empty((Lc, FFN // 256 * 292), dtype=torch.uint8, device=dev)
        dmax_d = torch.empty(Lc, dtype=torch.float32, device=dev)  # per-token largest |d|
        dmax_f = torch.empty(Lc, dtype=torch.float32, device=dev)
        y_qkv = torch.empty((Lc, 3 * D), dtype=torch.float32, device=dev)
        y_o = torch.empty((Lc, D), dtype=torch.float32, device=dev)
        y_gu = torch.empty((Lc, 2 * FFN), dtype=torch.float32, device=dev)
        y_down = torch.empty((Lc, D), dtype=torch.float32, device=dev)
        logits = torch.empty((MASKED, VOCAB), dtype=torch.float32, device=dev)
        amax = torch.empty(MASKED, dtype=torch.int32, device=dev)
        ws_bytes = max([dl.qgemm_workspace_bytes(q, n, k, Lc) for q, n, k in
                        [(Q4, 3 * D, D), (Q4, D, D), (Q4, 2 * FFN, D), (Q4, D, FFN), (Q6, D, FFN)]]
                       + [dl.qgemm_pair_workspace_bytes(Q4, 2 * D, Q6, D, D, Lc)])
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        ws_lm = torch.empty(dl.lmhead_workspace_bytes(Q6, VOCAB, D, MASKED), dtype=torch.uint8, device=dev)
        hidden = synth.normal_f32((Lc, D), seed, f"hidden-{Lc}", dev)
        first = 20 if Lc == L else Lc - MASKED  # the masked rows: 20..51, or the last block of the canvas
        rows = torch.arange(first, first + MASKED, dtype=torch.int32, device=dev)
        calls = []

        def add_quant(x, out, dmax):
            M, K = x.shape
            calls.append(("quantize_q8k", lambda: dl.quantize_q8k(x, out, dmax),
                          M * K * 4 + M * K // 256 * 292 + M * 4, 0, ("quantize_q8k", M, K)))

        def add_gemm(q, w, N, K, xq, dmax, y):
            byts = N * K // 256 * bb(q) + Lc * K // 256 * 292 + Lc * N * 4
            kind = "qgemm_q4k" if q == Q4 else "qgemm_q6k"
            calls.append((kind, lambda: dl.qgemm(q, w, N, K, xq, Lc, y=y, workspace=ws, x_dmax=dmax), byts,
                          2 * Lc * N * K, (kind, N, K)))

        def add_pair(qa, wa, Na, ya, qb, wb, Nb, yb, K, xq, dmax):
            """Two GEMMs of one input in one launch (dllm_qgemm_pair)."""
            byts = (Na * K // 256 * bb(qa) + Nb * K // 256 * bb(qb) + Lc * K // 256 * 292 + Lc * (Na + Nb) * 4)
            calls.append(("qgemm_pair", lambda: dl.qgemm_pair((qa, wa, Na, ya, None), (qb, wb, Nb, yb, None), K, xq,
                                                              Lc, workspace=ws, x_dmax=dmax),
                          byts, 2 * Lc * (Na + Nb) * K, ("qgemm_pair", f"{Na}+{Nb}", K)))

        for l, lw in enumerate(layers):
            x_norm = synth.normal_f32((Lc, D), seed, f"L{l:02d}.x_norm-{Lc}", dev)
            attn = synth.normal_f32((Lc, D), seed, f"L{l:02d}.attn-{Lc}", dev)
            h_norm = synth.normal_f32((Lc, D), seed, f"L{l:02d}.h_norm-{Lc}", dev)
            act = synth.normal_f32((Lc, FFN), seed, f"L{l:02d}.act-{Lc}", dev)
            add_quant(x_norm, xq_d, dmax_d)
            if lw["even"]:  # Q + K (Q4_K) and V (Q6_K) in one launch
                add_pair(Q4, lw["qk"], 2 * D, y_qkv[:, :2 * D], Q6, lw["v"], D, y_qkv[:, 2 * D:], D, xq_d, dmax_d)
            else:
                add_gemm(Q4, lw["qkv"], 3 * D, D, xq_d, dmax_d, y_qkv)
            add_quant(attn, xq_d, dmax_d)
            add_gemm(Q4, lw["o"], D, D, xq_d, dmax_d, y_o)
            add_quant(h_norm, xq_d, dmax_d)
            add_gemm(Q4, lw["gu"], 2 * FFN, D, xq_d, dmax_d, y_gu)
            add_quant(act, xq_f, dmax_f)
            add_gemm(Q6 if lw["even"] else Q4, lw["down"], D, FFN, xq_f, dmax_f, y_down)
        lm_bytes = (MASKED * D * 4 + MASKED * D // 256 * 292 + VOCAB * D // 256 * bb(Q6)
                    + MASKED * VOCAB * 4 + MASKED * 4)
        calls.append(("lmhead_q6k", lambda: dl.lmhead_masked(Q6, w_out, VOCAB, D, hidden, rows, logits, amax, ws_lm),
                      lm_bytes, 2 * MASKED * VOCAB * D, ("lmhead_q6k", VOCAB, D)))
        bufs = dict(y_qkv=y_qkv, y_gu=y_gu, xq_d=xq_d, xq_f=xq_f, dmax_d=dmax_d, dmax_f=dmax_f, ws=ws,
                    ws_lm=ws_lm, hidden=hidden, rows=rows, logits=logits, amax=amax, lm_bytes=lm_bytes)
        return calls, bufs

    calls, B = build_step(L)
    n_calls = len(calls)
    step_bytes = sum(c[2] for c in calls)
    step_ops = sum(c[3] for c in calls)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # ---------------- the step: graph capture and timed replays -------------
    # W untimed replays, then exactly K timed replays in up to 5 batches
    # (median of the batches' ms per step, with their min and max)
    g = capture(torch, [c[1] for c in calls])
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per_batch = time_replays(torch, g, args.steps, max(1, min(5, args.steps)))
    wall = time.perf_counter() - t0
    ms_step = med(per_batch)
    print(f"[bench] setup {t_setup:.1f}s; {len(calls)} calls/step; graph: {ms_step:.4f} ms/step "
          f"(batches {[round(x, 4) for x in per_batch]}, wall {1e3 * wall / args.steps:.4f} ms/step)",
          file=sys.stderr, flush=True)
    del g

    # ---------------- per-call durations (eager, HIP events on the launch stream)
    # Every call is bracketed by events on the stream it is launched on; calls
    # are grouped by kind and by shape (context: the events also hold each
    # call's dispatch).
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
        fg = capture(torch, fns)
        fg.replay()
        torch.cuda.synchronize()
        return med(time_replays(torch, fg, replays, replays)) / len(fns)

    # ---------------- stand-alone configurations ---------------------------
    # R >= 100 calls per graph, cycling through >= 1 GiB of distinct weight
    # copies (the step's own layers where they are enough), so that every
    # call streams its weights from HBM; 5 replays, median per call.
    def standalone(make, weights, per_call_bytes, per_call_ops, what):
        wlist = list(weights)
        nbytes = sum(w.numel() for w in wlist)
        k = 0
        while nbytes < GiB:  # copies of the given weights until >= 1 GiB
            c = wlist[k % len(weights)].clone()
            wlist.append(c)
            nbytes += c.numel()
            k += 1
        R = max(100, len(wlist))
        fns = [make(wlist[i % len(wlist)]) for i in range(R)]
        fg = capture(torch, fns)
        fg.replay()
        torch.cuda.synchronize()
        pb = [x / R for x in time_replays(torch, fg, 5, 5)]
        ms = med(pb)
        del fg, fns, wlist
        torch.cuda.empty_cache()
        return {"avg_ms": round(ms, 5), "min_ms": round(min(pb), 5), "max_ms": round(max(pb), 5),
                "GBps": round(per_call_bytes / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(per_call_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "int8_TOPS": round(per_call_ops / (ms * 1e-3) / 1e12, 2),
                "frac_mfma": round(per_call_ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                "algorithmic_bytes": per_call_bytes, "int8_ops": per_call_ops,
                "calls_per_replay": R, "weight_bytes_cycled": nbytes, "workload": what,
                "timing": "one graph of R calls cycling the weight copies, median of 5 replays (min, max)"}

    xq_d, dm_d, xq_f, dm_f, ws = B["xq_d"], B["dmax_d"], B["xq_f"], B["dmax_f"], B["ws"]
    dl.quantize_q8k(synth.normal_f32((L, D), seed, "cfg-x4", dev), xq_d, dm_d)
    dl.quantize_q8k(synth.normal_f32((L, FFN), seed, "cfg-x12", dev), xq_f, dm_f)
    y_d = torch.empty((L, D), dtype=torch.float32, device=dev)
    y_gu = B["y_gu"]
    gbytes = lambda q, N, K: N * K // 256 * bb(q) + L * K // 256 * 292 + L * N * 4
    configs = {}
    configs["1_q4k_4096x4096"] = standalone(
        lambda w: (lambda: dl.qgemm(Q4, w, D, D, xq_d, L, y=y_d, workspace=ws, x_dmax=dm_d)),
        [lw["o"] for lw in layers], gbytes(Q4, D, D), 2 * L * D * D,
        f"config 1: Q4_K {D}x{D} GEMM at L={L} (the O projection's plan)")
    configs["2_q6k_4096x12288"] = standalone(
        lambda w: (lambda: dl.qgemm(Q6, w, D, FFN, xq_f, L, y=y_d, workspace=ws, x_dmax=dm_f)),
        [lw["down"] for lw in layers if lw["even"]], gbytes(Q6, D, FFN), 2 * L * D * FFN,
        f"config 2: Q6_K {D}x{FFN} GEMM at L={L} (ffn_down)")
    lm = lambda w: (lambda: dl.lmhead_masked(Q6, w, VOCAB, D, B["hidden"], B["rows"], B["logits"], B["amax"],
                                              B["ws_lm"]))
    configs["4_lmhead_q6k"] = standalone(lm, [w_out], B["lm_bytes"], 2 * MASKED * VOCAB * D,
                                         f"config 4: masked LM head, {MASKED} of {L} rows x {VOCAB}x{D} Q6_K")
    # config 3: one even layer's stream (4 quantizes, Q+K with V, O, gate+up,
    # down in Q4_K / Q6_K as in the step), cycling the step's 16 even layers
    layer_calls = []
    ci = 0
    for lw in layers:
        n = 8  # quantize, Q+K+V (one call: QKV, or the Q+K / V pair), quantize, O, quantize, gate/up, quantize, down
        if lw["even"]:
            layer_calls.append(calls[ci:ci + n])
        ci += n
    l_bytes = sum(c[2] for c in layer_calls[0])
    l_ops = sum(c[3] for c in layer_calls[0])
    R3 = 6 * len(layer_calls)
    fns3 = [c[1] for i in range(R3) for c in layer_calls[i % len(layer_calls)]]
    g3 = capture(torch, fns3)
    g3.replay()
    torch.cuda.synchronize()
    pb3 = [x / R3 for x in time_replays(torch, g3, 5, 5)]
    del g3, fns3
    ms3 = med(pb3)
    configs["3_layer_L148"] = {
        "avg_ms": round(ms3, 5), "min_ms": round(min(pb3), 5), "max_ms": round(max(pb3), 5),
        "GBps": round(l_bytes / (ms3 * 1e-3) / 1e9, 1), "frac_hbm": round(l_bytes / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "int8_TOPS": round(l_ops / (ms3 * 1e-3) / 1e12, 2), "algorithmic_bytes": l_bytes, "int8_ops": l_ops,
        "calls_per_layer": len(layer_calls[0]), "layers_per_replay": R3,
        "weight_bytes_cycled": sum(c[2] for lc in layer_calls for c in lc),
        "workload": f"config 3: one layer's stream at L={L} (4 quantizes; Q+K, O, gate+up Q4_K; V, down Q6_K; "
                    f"Q+K and V in one launch)",
        "timing": f"one graph of {R3} layer passes cycling the step's {len(layer_calls)} even layers, median of 5 replays"}

    # the dominant call (gate/up, a third of the step) stand-alone: the
    # roofline figure of the step's dominant kernel
    dom = ("qgemm_q4k", 2 * FFN, D)
    dom_name = f"{dom[0]}_{dom[1]}x{dom[2]}"
    dom_cfg = standalone(
        lambda w: (lambda: dl.qgemm(Q4, w, 2 * FFN, D, xq_d, L, y=y_gu, workspace=ws, x_dmax=dm_d)),
        [lw["gu"] for lw in layers], gbytes(Q4, 2 * FFN, D), 2 * L * 2 * FFN * D,
        f"gate+up Q4_K {2 * FFN}x{D} at L={L}")
    for k_, v_ in configs.items():
        print(f"[bench] {k_}: {v_['avg_ms'] * 1e3:.2f} us, {v_['GBps']} GB/s", file=sys.stderr, flush=True)
    print(f"[bench] dominant {dom_name}: {dom_cfg['avg_ms'] * 1e3:.2f} us, {dom_cfg['GBps']} GB/s",
          file=sys.stderr, flush=True)

    # ---------------- the step at L = 160 (a reported extra) ----------------
    step160 = None
    if L != 160 and not args.no_l160:
        del calls
        torch.cuda.empty_cache()
        calls160, B160 = build_step(160)
        b160 = sum(c[2] for c in calls160)
        o160 = sum(c[3] for c in calls160)
        g160 = capture(torch, [c[1] for c in calls160])
        for _ in range(args.warmup):
            g160.replay()
        torch.cuda.synchronize()
        pb160 = time_replays(torch, g160, args.steps, max(1, min(5, args.steps)))
        del g160
        ms160 = med(pb160)
        step160 = {"ms_per_step": round(ms160, 5), "min_ms": round(min(pb160), 5), "max_ms": round(max(pb160), 5),
                   "step_algorithmic_bytes": b160, "step_int8_ops": o160,
                   "GBps": round(b160 / (ms160 * 1e-3) / 1e9, 1),
                   "frac_hbm": round(b160 / (ms160 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "int8_TOPS": round(o160 / (ms160 * 1e-3) / 1e12, 2),
                   "frac_mfma": round(o160 / (ms160 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                   "workload": "config 5 text: the whole step at L=160 (32 prompt + 128 generated), LM head on "
                               "the last block's 32 masked rows (128..159)",
                   "timing": f"{args.steps} replays in {len(pb160)} batches, median (min, max)"}
        print(f"[bench] L=160 step: {ms160:.4f} ms", file=sys.stderr, flush=True)
        del calls160, B160
        torch.cuda.empty_cache()

    # the LM head with the greedy pick's confidence (log-sum-exp and softmax
    # probability of the argmax per masked row; not part of the step)
    lse = torch.empty(MASKED, dtype=torch.float32, device=dev)
    p_am = torch.empty(MASKED, dtype=torch.float32, device=dev)
    conf = lambda: dl.lmhead_confidence(Q6, w_out, VOCAB, D, B["hidden"], B["rows"], B["logits"], B["amax"], lse, p_am,
                                        B["ws_lm"])
    conf_ms = graph_node_ms([conf] * 5)

    # the fused producers of the quantized activations (not part of the step):
    # RMSNorm -> Q8_K on a layer input, SwiGLU -> Q8_K on the gate/up output,
    # against the plain quantizer on the f32 tensors they replace
    g_norm = synth.normal_f32((D,), seed, "norm_weight", dev)
    x_in = synth.normal_f32((L, D), seed, "fused-x", dev)
    act_in = synth.normal_f32((L, FFN), seed, "fused-act", dev)
    fused = {
        "rmsnorm_quantize_q8k": (lambda: dl.rmsnorm_quantize_q8k(x_in, g_norm, 1e-5, xq_d, dm_d),
                                 L * D * 4 + D * 4 + L * D // 256 * 292),
        "quantize_q8k_after_rmsnorm": (lambda: dl.quantize_q8k(x_in, xq_d, dm_d),
                                       L * D * 4 + L * D // 256 * 292),
        "swiglu_quantize_q8k": (lambda: dl.swiglu_quantize_q8k(y_gu, xq_f, dm_f),
                                L * 2 * FFN * 4 + L * FFN // 256 * 292),
        "quantize_q8k_after_swiglu": (lambda: dl.quantize_q8k(act_in, xq_f, dm_f),
                                      L * FFN * 4 + L * FFN // 256 * 292),
    }
    fused_out = {}
    for name, (fn, byts) in fused.items():
        fms = graph_node_ms([fn] * 20)
        fused_out[name] = {"avg_ms": round(fms, 5), "GBps": round(byts / (fms * 1e-3) / 1e9, 1)}

    # bidirectional attention on the Q+K+V projection's output (not part of
    # the step): 32 heads of 128 over the L-token canvas
    attn_out = torch.empty((L, D), dtype=torch.float32, device=dev)
    a_ms = graph_node_ms([lambda: dl.attention(B["y_qkv"], 32, 128, None, attn_out)] * 20)
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
        if kv.get("kernel_sha") == _kernel_hash() and "bytes_per_call" in kv:
            traffic = float(kv["bytes_per_call"])
    counters = {n_: counter_summary(n_) for n_ in PMC_TARGETS.values()}
    counters = {k_: v_ for k_, v_ in counters.items() if v_ is not None}

    # ---------------- CPU oracle baseline (bounded sample) -----------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, step_ops // 2)

    step_s = ms_step * 1e-3
    dom_ms = dom_cfg["avg_ms"]
    dom_bytes, dom_ops = dom_cfg["algorithmic_bytes"], dom_cfg["int8_ops"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
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
                   "L": L, "layers": LAYERS, "masked_rows": MASKED, "calls_per_step": n_calls,
                   "launch": "one HIP graph replay per step"},
        "step_timing": {"batches_ms": [round(x, 5) for x in per_batch], "median_ms": round(ms_step, 5),
                        "min_ms": round(min(per_batch), 5), "max_ms": round(max(per_batch), 5),
                        "how": f"{args.steps} timed replays in {len(per_batch)} batches between HIP events"},
        "step_int8_TOPS": round(step_ops / step_s / 1e12, 2),
        "step_GBps": round(step_bytes / step_s / 1e9, 1),
        "step_frac_hbm": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_frac_mfma": round(step_ops / step_s / 1e12 / INT8_PEAK_TOPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "step_int8_ops": step_ops,
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_call_ms": round(dom_ms, 5), "calls_per_step": LAYERS,
                     "timing": dom_cfg["timing"] + ", HIP events on the replay stream",
                     "algorithmic_bytes_per_call": dom_bytes,
                     "int8_TOPS": round(dom_ops / (dom_ms * 1e-3) / 1e12, 2),
                     "frac_mfma": round(dom_ops / (dom_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "counters": counters.get(PMC_TARGETS["gateup"])},
        "configs_standalone": configs,
        "step_L160": step160,
        "hardware_counters": counters,
        "per_call_kind": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                          for k, v in kinds.items()},
        "per_call_shape": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                           for k, v in shapes.items()},
        "lmhead_confidence": {"avg_ms": round(conf_ms, 5), "GBps": round(B["lm_bytes"] / (conf_ms * 1e-3) / 1e9, 1),
                              "outputs": "logits, argmax, log-sum-exp and p(argmax) per masked row",
                              "in_step": False},
        "fused_producers": dict(fused_out, in_step=False),
        "attention": attention,
        "dream_step": dream,
        "cpu_baseline": cpu,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


def summarize_pmc(spec):
    """profiles/mfma_<kernel>.txt from three counter passes of one
    --profile-kernel target: per dispatch of the target's kernel (the last
    dispatches of the run), averaged.  MFMA utilisation is the busy cycles of
    the matrix units over the SIMD cycles of the kernel: SQ_VALU_MFMA_BUSY_CYCLES
    / (GRBM_GUI_ACTIVE / XCDs x CUs x SIMDs), GRBM_GUI_ACTIVE being summed over
    the XCDs."""
    import csv
    target, prefix = spec
    name = PMC_TARGETS[target]
    pick = {"lmhead": "k_lmhead", "quant4096": "k_quantize"}.get(target, "k_qgemm")
    vals, kname, dur = {}, None, []
    for p in PMC_PASSES:
        rows = list(csv.DictReader(open(os.path.join(f"{prefix}_{p}", "run_counter_collection.csv"))))
        per = {}
        for r in rows:
            if pick not in r["Kernel_Name"]:
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            kname = r["Kernel_Name"]
        # the first dispatch of a pass is left out: its counter window also
        # holds the code object's first load (GRBM_GUI_ACTIVE several times
        # the kernel's own)
        ids = sorted(per)
        for i in (ids[1:] if len(ids) > 1 else ids):
            for k, v in per[i].items():
                vals.setdefault(k, []).append(v)
    m = {k: sum(v) / len(v) for k, v in vals.items()}
    n_disp = len(vals["SQ_WAVES"])
    simd_cycles = m["GRBM_GUI_ACTIVE"] / XCDS * CUS * SIMDS
    wc = m["SQ_WAVE_CYCLES"]
    fig = {
        "mfma_util": m["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles,
        "valu_per_mfma": m["SQ_INSTS_VALU"] / max(m["SQ_INSTS_MFMA"], 1.0),
        "valu_active": m["SQ_ACTIVE_INST_VALU"] / wc,
        "mfma_valu_coexec": m["SQ_VALU_MFMA_COEXEC_CYCLES"] / wc,
        "wait_any": m["SQ_WAIT_ANY"] / wc,
        "wait_inst_any": m["SQ_WAIT_INST_ANY"] / wc,
        "lds_bank_conflict_frac": m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_INSTS_LDS"], 1.0),
        "counter_TOPS_i8": m["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512 / (m["_ns"] * 1e-9) / 1e12,
        "kernel_us": m["_ns"] / 1e3,
        "insts_per_wave_valu": m["SQ_INSTS_VALU"] / m["SQ_WAVES"],
        "insts_per_wave_mfma": m["SQ_INSTS_MFMA"] / m["SQ_WAVES"],
        "insts_per_wave_lds": m["SQ_INSTS_LDS"] / m["SQ_WAVES"],
    }
    lines = [f"# hardware counters of {STEP_CALLS.get(target, (0, 0, 0, target))[3]} at L=148 (bench.py --profile-kernel {target})",
             f"# kernel: {kname}",
             "# commands (one pass each; run from /tmp with TMPDIR=/tmp):"]
    for p, cs in PMC_PASSES.items():
        lines.append(f"#   rocprofv3 --pmc {cs} --output-format csv -d {prefix}_{p} -o run -- "
                     f"python3 bench.py --profile-kernel {target} --steps 5")
    lines.append(f"#   python3 bench.py --summarize-pmc {target} {prefix}")
    lines.append(f"# {n_disp} dispatches of the kernel over the passes (each pass's first left out), averaged")
    lines.append("# mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs x 4 SIMDs)")
    lines.append("# valu_per_mfma = SQ_INSTS_VALU / SQ_INSTS_MFMA; valu_active, mfma_valu_coexec, wait_any,"
                 " wait_inst_any = SQ_ACTIVE_INST_VALU, SQ_VALU_MFMA_COEXEC_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY"
                 " / SQ_WAVE_CYCLES")
    lines.append("# counter_TOPS_i8 = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 / kernel duration (issued int8 work,"
                 " both planes, padded tokens)")
    lines.append("# raw means per dispatch: " + " ".join(f"{k}={v:.6g}" for k, v in sorted(m.items()) if k != "_ns"))
    lines.append("# kernel_sha: hash of the kernel sources the counters were taken on")
    lines.append(f"kernel_sha={_kernel_hash()}")
    lines += [f"{k}={v:.5g}" for k, v in fig.items()]
    path = os.path.join(ROOT, "profiles", f"mfma_{name}.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(f"[summarize-pmc] wrote {path}: mfma_util {fig['mfma_util']:.3f}, valu/mfma {fig['valu_per_mfma']:.2f}")


def _short_kernel(name: str) -> str:
    """k_qgemm<12, 5, 12, 1, false, 2, false> from a demangled or plain name."""
    n = name.split("(")[0].replace("void ", "").replace("dllm::", "")
    return n.strip()


def summarize_trace(d, out):
    """profiles/<out>: libdllm kernels of a rocprofv3 --kernel-trace run
    (per kernel and per kernel + grid)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_trace.csv"))))
    per, per_grid = {}, {}
    for r in rows:
        kn = _short_kernel(r["Kernel_Name"])
        if not kn.startswith("k_"):
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        wg = [int(r[f"Workgroup_Size_{a}"]) for a in "XYZ"]
        grid = tuple(int(r[f"Grid_Size_{a}"]) // w for a, w in zip("XYZ", wg))
        per.setdefault(kn, []).append(us)
        per_grid.setdefault((kn, grid), []).append(us)
    tot = sum(sum(v) for v in per.values())
    lines = [f"# libdllm kernels of one rocprofv3 --kernel-trace --stats run; durations in microseconds",
             f"# source: {os.path.basename(os.path.normpath(d))}/run_kernel_trace.csv; summary: "
             f"python3 bench.py --summarize-trace <dir> {out}",
             f"# kernel_sha={_kernel_hash()}", "",
             f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'total_us':>11s} {'share':>6s}"]
    for kn, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{kn:44s} {len(v):6d} {sum(v) / len(v):9.2f} {sum(v):11.1f} {100 * sum(v) / tot:5.1f}%")
    lines += ["", f"{'kernel (grid x,y,z in work-groups)':56s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for (kn, g), v in sorted(per_grid.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{kn + ' (' + ','.join(map(str, g)) + ')':56s} {len(v):6d} {sum(v) / len(v):9.2f} "
                     f"{min(v):9.2f} {max(v):9.2f}")
    path = os.path.join(ROOT, "profiles", out)
    open(path, "w").write("\n".join(lines) + "\n")
    print(f"[summarize-trace] wrote {path}")


def summarize_traffic(target, prefix, out):
    """profiles/<out>: HBM bytes per call of a target's kernel from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
    reads for the run's 256 MiB device copy."""
    import csv
    pick = {"lmhead": "k_lmhead", "quant4096": "k_quantize", "quant12288": "k_quantize", "rmsnorm": "k_quantize",
            "swiglu": "k_quantize", "attention": "k_attention"}.get(target, "k_qgemm")
    res = {}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = list(csv.DictReader(open(os.path.join(f"{prefix}_{cn}", "run_counter_collection.csv"))))
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == cn]
        kern = [(float(r["Counter_Value"]), r["Kernel_Name"]) for r in rows
                if pick in r["Kernel_Name"] and r["Counter_Name"] == cn]
        copy_bytes = 256 << 20  # read and written once by the copy
        per_kib = copy_bytes / copy[0]
        res[cn] = (sum(v for v, _ in kern) / len(kern), per_kib, len(kern), kern[0][1])
    f_kib, f_scale, n, kname = res["FETCH_SIZE"]
    w_kib, w_scale, _, _ = res["WRITE_SIZE"]
    rd, wr = f_kib * f_scale, w_kib * w_scale
    L = 148
    other = {  # (what, algorithmic bytes per call) of the calls outside STEP_CALLS
        "lmhead": ("the masked-row LM head, 32 rows x 126464 x 4096 Q6_K (streaming kernel)",
                   VOCAB * D // 256 * 210 + MASKED * D // 256 * 292 + MASKED * VOCAB * 4),
        "rmsnorm": (f"RMSNorm -> Q8_K, {L} x {D}", L * D * 4 + D * 4 + L * D // 256 * 292 + L * 4),
        "swiglu": (f"SwiGLU -> Q8_K, {L} x 2 x {FFN}", L * 2 * FFN * 4 + L * FFN // 256 * 292 + L * 4),
        "attention": (f"bidirectional attention, L={L}, 32 heads x 128 (f32 Q+K+V rows in, f32 out)",
                      L * 3 * D * 4 + L * D * 4),
        "pair": (f"Q+K Q4_K {2 * D}x{D} with V Q6_K {D}x{D} in one launch",
                 2 * D * D // 256 * 144 + D * D // 256 * 210 + L * D // 256 * 292 + L * 3 * D * 4),
    }
    if target == "dominant":
        q, N, K, what = 12, 2 * FFN, D, "gate+up Q4_K 24576x4096"
    elif target in STEP_CALLS:
        q, N, K, what = STEP_CALLS[target]
    else:
        q, (what, alg) = -1, other[target]
    if q == -1:
        pass
    elif q == 0:
        alg = L * K * 4 + L * K // 256 * 292 + L * 4
    else:
        alg = N * K // 256 * (144 if q == 12 else 210) + L * K // 256 * 292 + L * N * 4
    cmd = "--profile-dominant" if target == "dominant" else f"--profile-kernel {target}"
    lines = [f"# HBM traffic of {what} at L={L} (bench.py {cmd})",
             f"# kernel: {_short_kernel(kname)}",
             "# commands (each counter in its own pass; run from /tmp with TMPDIR=/tmp):",
             f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {prefix}_FETCH_SIZE -o run -- python3 bench.py {cmd} --steps 5",
             f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {prefix}_WRITE_SIZE -o run -- python3 bench.py {cmd} --steps 5",
             f"#   python3 bench.py --summarize-traffic {target} {prefix} {out}",
             f"# calibration: the same counters on the 256 MiB device copy the run makes first:",
             f"#   FETCH_SIZE -> {f_scale:.2f} bytes per counted KiB, WRITE_SIZE -> {w_scale:.2f} bytes per counted KiB",
             f"# kernel, mean of {n} dispatches: FETCH_SIZE {f_kib:.2f} KiB, WRITE_SIZE {w_kib:.2f} KiB",
             f"# -> read {rd / 1e6:.2f} MB + written {wr / 1e6:.2f} MB per call; algorithmic bytes per call "
             f"{alg / 1e6:.2f} MB (ratio {(rd + wr) / alg:.3f})",
             "# kernel_sha: hash of the kernel sources the counters were taken on",
             f"kernel_sha={_kernel_hash()}",
             f"bytes_per_call={int(rd + wr)}", f"read_bytes_per_call={int(rd)}", f"write_bytes_per_call={int(wr)}",
             f"algorithmic_bytes_per_call={alg}"]
    path = os.path.join(ROOT, "profiles", out)
    open(path, "w").write("\n".join(lines) + "\n")
    print(f"[summarize-traffic] wrote {path}: read {rd / 1e6:.2f} MB, written {wr / 1e6:.2f} MB, alg {alg / 1e6:.2f} MB")


def _kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("common.hpp", "kernels.hpp", "unpack.hpp", "qgemm.hip", "quantize.hip", "abi.hip", "lmhead.hip",
              "attention.hip"):
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
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "vendor_id", "cpu family", "model", "stepping", "cpu MHz", "cache size") \
                    and k not in info:
                info[k] = v.strip()
    except OSError:
        pass
    cpu_model = (f"{info.get('model name', platform.processor())} ({info.get('vendor_id', '?')} family "
                 f"{info.get('cpu family', '?')} model {info.get('model', '?')} stepping {info.get('stepping', '?')}, "
                 f"{info.get('cpu MHz', '?')} MHz, cache {info.get('cache size', '?')}; {os.cpu_count()} logical CPUs "
                 f"on the host, {nt} in this process's affinity set)")
    return {"value": round(step_macs / rate * 1e3, 1), "unit": "ms", "cores": nt, "kind": "oracle",
            "sample": f"{reps} x (oracle f64 GEMM of a Q4_K 4096x4096 layer + a Q6_K 4096x12288 layer at {L} tokens): "
                      f"{macs / 1e9:.1f} G MAC in {secs:.2f} s = {rate / 1e9:.2f} GMAC/s, scaled to the step's "
                      f"{step_macs / 1e12:.3f} T MAC",
            "cpu": cpu_model}


if __name__ == "__main__":
    main()
