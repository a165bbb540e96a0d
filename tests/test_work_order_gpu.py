"""Grids whose workgroups take their (slice, query tile) in groups of slices.

A launch takes the batch*head slices in groups whose query tiles fill one
round of an XCD's resident workgroups (8 XCDs); with no mask or a window
bounded on both sides whenever the grid has more slices than one group, under
other masks only when the plain order would run at most 2 query tiles of a
slice at once per XCD (slices >= 4 x resident per XCD).  The last group may hold fewer slices than the others.  With one
workgroup per compute unit (32 resident per XCD) these shapes give: 21 slices
of 16 query tiles at d = 128, no mask (groups of 16 and 5); 36 slices of 8 at
d = 64, no mask (32 and 4); 136 causal slices of 4 at d = 64 (64, 64, 8); 132
padded causal slices of 5 at d = 96 (48, 48, 36); 36 slices of 8 at d = 64
under a window bounded on both sides, which is grouped like no mask (32 and
4).

Causal grids of more than one round of resident workgroups and at most two
(one workgroup per compute unit: 256 < grid <= 512), whose second round
takes the short query tiles: 20 slices of 16 tiles at d = 128, 40 of 8 at
d = 64 (split-KV), 17 of 17 at d = 128 (an odd count), 14 of 22 at d = 256
and 5 of 63 at d = 1024.

O and LSE start as NaN, so a tile that no workgroup writes fails, and every
element is compared with the fp64 oracle.
"""
import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from oracle import attention_ref, attention_ref_masked
from tests.gpu_helpers import assert_close, assert_close_masked, to_device

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype, causal, (window_left, window_right, key_lens) or None)
CASES = [
    (3, 7, 4096, 128, wl.BF16, False, None),
    (4, 9, 2048, 64, wl.FP16, False, None),
    (8, 17, 1024, 64, wl.BF16, True, None),
    (4, 33, 640, 96, wl.FP16, False, (-1, 0, [640, 401, 77, 639])),
    (4, 9, 2048, 64, wl.FP16, False, (100, 20, None)),
    (1, 20, 4096, 128, wl.BF16, True, None),
    (1, 40, 2048, 64, wl.FP16, True, None),
    (1, 17, 4300, 128, wl.BF16, True, None),
    (1, 14, 2800, 256, wl.FP16, True, None),
    (1, 5, 4000, 1024, wl.BF16, True, None),
]


@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}h{c[1]}n{c[2]}d{c[3]}" for c in CASES])
def test_grouped_order_writes_every_tile(gpu_device, case):
    import torch
    from exact_attention_21_amd import forward
    B, H, N, d, dtype, causal, mask = case
    w = wl.Workload("g", B, H, N, d, dtype, causal)
    q, k, v = wl.make_inputs(w, seed=5)
    tq, tk, tv = (to_device(x, dtype, gpu_device) for x in (q, k, v))
    out = torch.full_like(tq, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=gpu_device)
    kw = {}
    if mask is not None:
        kw = dict(window=mask[:2])
        if mask[2] is not None:
            kw["key_lens"] = torch.tensor(mask[2], dtype=torch.int32, device=gpu_device)
    forward(tq, tk, tv, scale=w.softmax_scale(), causal=causal, out=out, lse=lse, **kw)
    torch.cuda.synchronize(gpu_device)
    o = out.float().cpu().numpy().astype(np.float64)
    l64 = lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(o).any() and not np.isnan(l64).any(), "some query tile was never written"
    f64 = [wl.to_float64(x, dtype) for x in (q, k, v)]
    label = f"B={B} H={H} N={N} d={d} {dtype}"
    if mask is None:
        o_ref, lse_ref = attention_ref(*f64, w.softmax_scale(), causal)
        assert_close(o, l64, o_ref, lse_ref, dtype, label)
    else:
        o_ref, lse_ref = attention_ref_masked(*f64, w.softmax_scale(), *mask)
        assert_close_masked(o, l64, o_ref, lse_ref, dtype, label)
