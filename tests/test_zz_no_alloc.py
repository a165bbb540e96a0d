"""fa2_bwd_noalloc, the allocation-free backward entry point, through the C
ABI: two calls in a row (the second on a smaller problem, so the scratch
array still holds the first call's Delta), each bit-identical to fa2_bwd on
the same inputs with a caller-allocated workspace, and the first also within
the oracle's rounding bound."""
import numpy as np
import pytest
import torch

from exact_attention_21_amd import FA2_OK, fa2_bwd, fa2_bwd_noalloc
from exact_attention_21_amd import _binding as bd
from exact_attention_21_amd import workloads as wl
from tests import bwd_helpers as bh
from tests.gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, dtype, causal, device, seed):
    w, q, k, v, do = bh.make_case(B, H, N, d, dtype, seed, causal=causal)
    q64, k64, v64 = (wl.to_float64(x, dtype) for x in (q, k, v))
    o_in, lse_in = bh.forward_inputs(q64, k64, v64, w.softmax_scale(), causal, dtype)
    ts = [to_device(x, dtype, device) for x in (q, k, v, o_in, do)]
    return w, (q, k, v, do), ts, torch.from_numpy(lse_in).to(device)


def _grads(ts, lse, w, device, workspace):
    tq, tk, tv, to, tdo = ts
    outs = [torch.full_like(tq, float("nan")) for _ in range(3)]
    ptrs = [t.data_ptr() for t in (tq, tk, tv, to, tdo)] + [lse.data_ptr()] + [t.data_ptr() for t in outs]
    stream = torch.cuda.current_stream(device).cuda_stream
    dt = 1 if w.dtype == wl.BF16 else 0
    if workspace is None:
        st = fa2_bwd_noalloc(*ptrs, w.B, w.H, w.N, w.d, w.softmax_scale(), int(w.causal), dt, stream)
    else:
        st = fa2_bwd(*ptrs, workspace.data_ptr(), w.B, w.H, w.N, w.d, w.softmax_scale(), int(w.causal), dt,
                     stream)
    assert st == FA2_OK, st
    torch.cuda.synchronize(device)
    return outs


def test_noalloc_matches_fa2_bwd_on_two_calls(gpu_device):
    for i, (B, H, N, d, dtype, causal) in enumerate([(2, 4, 1000, 128, wl.BF16, True),
                                                     (1, 2, 300, 64, wl.FP16, False)]):
        print(f"call {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
        w, host, ts, lse = _inputs(B, H, N, d, dtype, causal, gpu_device, seed=11 + i)
        ws = torch.empty((2, B, H, N), dtype=torch.float32, device=gpu_device)
        ref = _grads(ts, lse, w, gpu_device, ws)
        got = _grads(ts, lse, w, gpu_device, None)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i} {name} differs from fa2_bwd"
        if i == 0:
            q64, k64, v64, do64 = (wl.to_float64(x, dtype) for x in host)
            refs, bounds = bh.grad_bounds(q64, k64, v64, do64, bh.to_np(ts[3]), lse.cpu().numpy().astype(np.float64),
                                          w.softmax_scale(), causal, dtype)
            gotn = {n: bh.to_np(t).reshape(refs[n].shape) for n, t in zip(("dq", "dk", "dv"), got)}
            bh.assert_grads_within(gotn, refs, bounds, "fa2_bwd_noalloc")


def test_noalloc_rejects_more_than_its_scratch(gpu_device):
    n = (1 << 21) // 64 + 1  # B * H * N = 2^21 + 64
    # Never dereferenced: the call is rejected before anything is enqueued
    # (4 GiB apart, so that the size check, not the overlap check, decides).
    ptrs = [(i + 1) << 32 for i in range(9)]
    st = fa2_bwd_noalloc(*ptrs, 1, 64, n, 64, 0.125, 0, 0, 0)
    assert st == bd.FA2_ERR_TOO_LARGE
