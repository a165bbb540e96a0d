"""Driver for hardware-counter runs: a few fa2_fwd launches on one seeded
workload (``--pass bwd``: one fa2_fwd launch, then a few fa2_bwd calls), then
one plain device-to-device copy of known size.

The copy gives the factor that turns the FETCH_SIZE / WRITE_SIZE counters into
bytes (it moves exactly ``copy_mb`` MiB each way).  Usage (from any directory):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT -- \
      python3 REPO/exact_attention_21_amd/profile_run.py --workload NAME
"""
from __future__ import annotations

import argparse
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="headline_b1h8n8192d64_fp16")
    ap.add_argument("--launches", type=int, default=3)
    ap.add_argument("--copy-mb", type=int, default=256)
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd")
    args = ap.parse_args()

    import torch

    from exact_attention_21_amd import backward, forward, library
    from exact_attention_21_amd import workloads as wl

    library()
    w = {x.name: x for x in wl.ALL_WORKLOADS}[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = wl.make_inputs(w, seed=0)

    def to_dev(x):
        t = torch.from_numpy(x) if w.dtype == wl.FP16 else \
            torch.from_numpy(x.view("int16")).view(torch.bfloat16)
        return t.to(dev)

    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    out = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    mask_kw = {}
    if w.window is not None:
        mask_kw["window"] = w.window
    if w.key_lens is not None:
        mask_kw["key_lens"] = torch.tensor(w.key_lens, dtype=torch.int32, device=dev)
    if args.pass_ == "bwd":
        forward(tq, tk, tv, scale=w.softmax_scale(), causal=w.causal, out=out, lse=lse, **mask_kw)
        tdo = to_dev(wl.make_grad_output(w, seed=0))
        grads = (torch.empty_like(tq), torch.empty_like(tq), torch.empty_like(tq))
        ws = torch.empty((2, w.B, w.H, w.N), dtype=torch.float32, device=dev)
        for _ in range(args.launches):
            backward(tq, tk, tv, out, lse, tdo, scale=w.softmax_scale(), causal=w.causal, workspace=ws, out=grads,
                     **mask_kw)
    else:
        for _ in range(args.launches):
            forward(tq, tk, tv, scale=w.softmax_scale(), causal=w.causal, out=out, lse=lse, **mask_kw)
    torch.cuda.synchronize(dev)
    n = args.copy_mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(f"profile_run: {args.launches} {args.pass_} launches of {w.name}, copy of {args.copy_mb} MiB", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
