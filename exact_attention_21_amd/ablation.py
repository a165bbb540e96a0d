"""Design ablations of the forward kernel on one workload.

Each row is a build of the library with one design switch flipped (the
switches are listed at the top of csrc/fa2_kernel.hpp; the default build is
the shipped design).  All builds are loaded into one process and timed in
alternation, round after round, so clock drift and box-to-box differences
affect every row alike; a row's time is the median over the rounds.  Each
variant's output is compared with the shipped build's on the same inputs
(layout-only switches must give identical bits; the others change the
summation order or the exponent base and must stay within 1e-3).

Two PyTorch rows give context, as the ablation table on the MMA notes page
does: attention in three steps (S = Q K^T into HBM, the mask, softmax, P V),
and torch's scaled_dot_product_attention (fp16 unmasked or causal only, and
never its math backend).  Masked workloads run fa2_fwd_masked.

    python exact_attention_21_amd/ablation.py --build        # compile the variant builds (no GPU needed)
    python exact_attention_21_amd/ablation.py [--workload NAME] [--rounds 5]
    python exact_attention_21_amd/ablation.py --only NAME    # a few launches of one build, for counter runs
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 2516.6

# (name, design switches, what changes against the shipped design)
VARIANTS = [
    ("shipped", None, "the library as built"),
    ("no_kv_swizzle", {"FA2_KV_SWIZZLE": 0}, "K and V tiles stored row-major in LDS (no chunk permutation)"),
    ("checked_only", {"FA2_UNCHECKED_RUN": 0}, "every tile's row sums checked; no fixed-base unchecked run"),
    ("no_split_kv", {"FA2_SPLIT_KV": 0}, "4 waves per workgroup with one K/V stream (no split-KV wave groups)"),
    ("deep_ring", {"FA2_KV_SLOTS": 8}, "8-slot K/V rings, one barrier per 4 tiles (instead of 4 slots, per 2)"),
    ("two_slot_ring", {"FA2_KV_SLOTS": 2},
     "2-slot K/V rings, one barrier per tile: the nearest form of the single K and V buffer"),
    ("padded_rows", {"FA2_KV_PAD": 1},
     "K/V rows padded in LDS (K +16 B, V +64 B), filled through VGPRs; no swizzle, no direct-to-LDS loads"),
    ("no_xcd_groups", {"FA2_XCD_GROUPS": 0}, "work order over all heads at once (no XCD-sized head groups)"),
    ("no_w4_bound", {"FA2_W4_TWO_PER_SIMD": 0},
     "d = 64 4-wave form without the two-waves-per-SIMD register bound"),
]
# Switches that only move data in LDS, change the barrier cadence, the order
# of the workgroups or the register budget: the arithmetic is the same, so the
# output must be bit-identical.
LAYOUT_ONLY = {"no_kv_swizzle", "deep_ring", "two_slot_ring", "padded_rows", "no_xcd_groups", "no_w4_bound"}


def lib_path(name: str) -> str:
    from exact_attention_21_amd._build import LIB_PATH, variant_path
    return LIB_PATH if name == "shipped" else variant_path(name)


# Head dims the variant builds compile (FA2_DIMS bit mask: d = 64 and 128,
# those of the ablation workloads), which keeps each build short.
VARIANT_DIMS = 0x0A


def build_all() -> None:
    from concurrent.futures import ThreadPoolExecutor

    from exact_attention_21_amd._build import build_variant
    todo = [(name, {**defines, "FA2_DIMS": VARIANT_DIMS}) for name, defines, _ in VARIANTS if defines is not None]
    with ThreadPoolExecutor(4) as ex:
        for path in ex.map(lambda t: build_variant(t[0], t[1]), todo):
            print(path, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true", help="compile the variant builds and exit")
    ap.add_argument("--workload", default="headline_b1h8n8192d64_fp16")
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--iters", type=int, default=30)
    ap.add_argument("--only", default=None, help="run a few launches of one build and exit")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--no-torch", action="store_true", help="skip the PyTorch context rows")
    args = ap.parse_args()
    if args.build:
        build_all()
        return 0

    import torch

    from exact_attention_21_amd import _binding as bd
    from exact_attention_21_amd import workloads as wl

    w = {x.name: x for x in wl.ALL_WORKLOADS}[args.workload]
    dev = torch.device("cuda:0")
    q, k, v = wl.make_inputs(w, seed=0)

    def to_dev(x):
        t = torch.from_numpy(x) if w.dtype == wl.FP16 else \
            torch.from_numpy(x.view("int16")).view(torch.bfloat16)
        return t.to(dev)

    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    stream = torch.cuda.current_stream(dev)
    dt = bd.FA2_DTYPE_FP16 if w.dtype == wl.FP16 else bd.FA2_DTYPE_BF16
    scale = w.softmax_scale()
    names = [n for n, _, _ in VARIANTS] if args.only is None else [args.only]
    for n in names:
        if n not in {x for x, _, _ in VARIANTS}:
            print(f"unknown variant {n!r}", file=sys.stderr)
            return 2
        if not os.path.exists(lib_path(n)):
            print(f"{lib_path(n)} is not built (run with --build)", file=sys.stderr)
            return 1
    libs = {n: bd.open_library(lib_path(n)) for n in names}
    outs = {n: (torch.empty_like(tq), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev))
            for n in names}

    # Masked workloads: fa2_fwd_masked with the workload's window and lengths.
    left, right = w.window if w.window is not None else (-1, -1)
    if w.causal:
        right = 0 if right < 0 else min(right, 0)
    lens = torch.tensor(w.key_lens, dtype=torch.int32, device=dev) if w.key_lens is not None else None

    def launcher(n):
        lib, (o, lse) = libs[n], outs[n]
        if w.masked:
            args_ = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.N, w.d, scale, left, right, lens.data_ptr() if lens is not None else None, dt,
                     stream.cuda_stream)
            fn, fname = lib.fa2_fwd_masked, "fa2_fwd_masked"
        else:
            args_ = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.N, w.d, scale, int(w.causal), dt, stream.cuda_stream)
            fn, fname = lib.fa2_fwd, "fa2_fwd"

        def run():
            st = fn(*args_)
            if st != bd.FA2_OK:
                raise bd.Fa2Error(st, f"{fname} ({n})")
        return run

    runs = {n: launcher(n) for n in names}
    if args.only is not None:
        for _ in range(args.launches):
            runs[args.only]()
        torch.cuda.synchronize(dev)
        print(f"{args.only}: {args.launches} launches on {w.name}", flush=True)
        return 0

    # Context rows from PyTorch.
    if not args.no_torch:
        kt = tk.transpose(-1, -2).contiguous()

        hidden = None
        if w.causal or w.masked:
            i = torch.arange(w.N, device=dev)[:, None]
            j = torch.arange(w.N, device=dev)[None, :]
            hidden = torch.zeros(w.N, w.N, dtype=torch.bool, device=dev)
            if right >= 0:
                hidden |= j > i + right
            if left >= 0:
                hidden |= j < i - left
            hidden = hidden[None, None]
            if lens is not None:
                hidden = hidden | (j[None, None] >= lens[:, None, None, None])

        def unfused():
            s = torch.matmul(tq, kt) * scale
            if hidden is not None:
                s = s.masked_fill(hidden, float("-inf"))
            p = torch.softmax(s.float(), dim=-1).to(tq.dtype)
            return torch.matmul(p, tv)
        runs["torch_unfused"] = unfused
        if w.dtype == wl.FP16 and not w.masked:
            from torch.nn.attention import SDPBackend, sdpa_kernel
            import torch.nn.functional as F

            def sdpa():
                with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=w.causal, scale=scale)
            try:
                sdpa()
                torch.cuda.synchronize(dev)
                runs["torch_sdpa"] = sdpa
            except RuntimeError as e:  # no fused backend for this shape
                print(f"torch_sdpa skipped: {e}", flush=True)

    # Parity of each build against the shipped one.
    for n in names:
        runs[n]()
    torch.cuda.synchronize(dev)
    o0, l0 = outs["shipped"]
    parity = {}
    for n in names:
        o, lse = outs[n]
        do = (o.float() - o0.float()).abs().max().item()
        dl = (lse - l0).abs().max().item()
        same = bool(torch.equal(o, o0) and torch.equal(lse, l0))
        ok = same if n in LAYOUT_ONLY else (do <= 1e-3 and dl <= 1e-3)
        parity[n] = (same, do, dl, ok)
        print(f"parity {n}: identical={same} max|dO|={do:.2e} max|dLSE|={dl:.2e} {'ok' if ok else 'MISMATCH'}",
              flush=True)

    def timed(fn, iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / iters

    order = list(runs)
    samples = {n: [] for n in order}
    for r in range(args.rounds):
        rot = order[r % len(order):] + order[:r % len(order)]
        for n in rot:
            iters = args.iters if not n.startswith("torch") else max(3, args.iters // 6)
            spent = 0.0
            while spent < 300.0:  # sustained load before each timed block
                spent += timed(runs[n], iters) * iters
            samples[n].append(timed(runs[n], iters))
        print(f"round {r + 1}/{args.rounds}: " + ", ".join(f"{n} {samples[n][-1]:.4f} ms" for n in order), flush=True)

    flops = w.flops()
    base = statistics.median(samples["shipped"])
    desc = {n: d for n, _, d in VARIANTS}
    desc["torch_unfused"] = "PyTorch: S = Q K^T (N x N in HBM), softmax in fp32, P V (K^T made contiguous outside the timing)"
    desc["torch_sdpa"] = "PyTorch scaled_dot_product_attention (flash or memory-efficient backend)"
    print(f"\n{w.name}: median of {args.rounds} rounds, {args.iters} launches each (PyTorch rows: "
          f"{max(3, args.iters // 6)})\n", flush=True)
    print("| build | what changes | ms | TFLOP/s | % of peak | time vs shipped | output vs shipped |")
    print("|---|---|---|---|---|---|---|")
    for n in order:
        ms = statistics.median(samples[n])
        tf = flops / ms / 1e9
        if n in parity:
            same, do, dl, ok = parity[n]
            pt = "identical" if same else f"max abs dO {do:.1e}, dLSE {dl:.1e}"
        else:
            pt = "-"
        print(f"| {n} | {desc[n]} | {ms:.4f} | {tf:.1f} | {100 * tf / PEAK_TFLOPS:.1f} | {ms / base:.3f}x | {pt} |")
    return 0 if all(p[3] for p in parity.values()) else 3


if __name__ == "__main__":
    sys.exit(main())
