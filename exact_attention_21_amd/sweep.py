"""Sequence-length sweep of the forward kernel on one GPU.

The trend the pages describe for FlashAttention-2 (utilisation grows with N,
most clearly with the causal mask; d = 128 runs faster than d = 64) is
measured here over N = 512 .. 16384.  Each point holds the tokens per call
(B * N = 16384) and the model width (H * d = 2048) fixed, so every point moves
the same number of Q/K/V/O bytes and the FLOPs grow with N.  Inputs are seeded
N(0, 1) fp16 (or bf16) tensors made on the GPU.

    python exact_attention_21_amd/sweep.py [--dims 64,128,256] [--dtype fp16]

prints one markdown table row per (d, causal, N): time per call and TFLOP/s
(4 B H N^2 d, halved for causal) as a share of the 2516.6 TFLOP/s dense
fp16/bf16 MFMA peak.  ``--pass bwd`` sweeps the backward (fa2_bwd on the
forward's O and LSE and a seeded dO; 10 B H N^2 d FLOPs, halved for causal).
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6
TOKENS = 16384
WIDTH = 2048
NS = (512, 1024, 2048, 4096, 8192, 16384)


def time_call(fn, stream, settle_ms: float = 300.0, iters: int = 50) -> float:
    """Mean milliseconds per call after `settle_ms` of untimed back-to-back calls."""
    import torch
    spent = 0.0
    while spent < settle_ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            fn()
        e1.record(stream)
        e1.synchronize()
        spent += e0.elapsed_time(e1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--dims", default="64,128,256")
    ap.add_argument("--dtype", default="fp16", choices=("fp16", "bf16"))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd")
    args = ap.parse_args()

    import torch
    from exact_attention_21_amd import backward, forward

    dev = torch.device("cuda:0")
    dt = torch.float16 if args.dtype == "fp16" else torch.bfloat16
    stream = torch.cuda.current_stream(dev)
    print(f"| d | causal | N | B | H | ms per call | TFLOP/s | % of peak |", flush=True)
    print("|---|---|---|---|---|---|---|---|", flush=True)
    for d in (int(x) for x in args.dims.split(",")):
        H = WIDTH // d
        for causal in (False, True):
            for N in NS:
                B = TOKENS // N
                g = torch.Generator(device=dev).manual_seed(args.seed)
                q, k, v = (torch.randn(B, H, N, d, generator=g, device=dev).to(dt) for _ in range(3))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
                scale = d ** -0.5
                flops = 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)
                if args.pass_ == "bwd":
                    forward(q, k, v, scale=scale, causal=causal, out=o, lse=lse)
                    do = torch.randn(B, H, N, d, generator=g, device=dev).to(dt)
                    grads = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
                    ws = torch.empty((2, B, H, N), dtype=torch.float32, device=dev)
                    ms = time_call(lambda: backward(q, k, v, o, lse, do, scale=scale, causal=causal, workspace=ws,
                                                    out=grads), stream)
                    flops *= 2.5
                    del do, grads, ws
                else:
                    ms = time_call(lambda: forward(q, k, v, scale=scale, causal=causal, out=o, lse=lse), stream)
                tf = flops / ms / 1e9
                print(f"| {d} | {causal} | {N} | {B} | {H} | {ms:.4f} | {tf:.1f} | {100 * tf / PEAK_TFLOPS:.1f} |",
                      flush=True)
                del q, k, v, o, lse
    return 0


if __name__ == "__main__":
    sys.exit(main())
