"""Parity of fa2_fwd_masked (sliding window, key padding) with the fp64
oracle's attention_ref_masked, through the C ABI on the GPU.

Tolerances are those of the unmasked tests (fp16 2e-3 on O and 1e-3 on LSE,
bf16 4e-3 and 2e-3; seeded N(0,1) inputs); rows with no visible key must give
O = 0 and LSE = +inf exactly.
"""
import math

import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from oracle import attention_ref_masked
from tests.gpu_helpers import (assert_close_masked, assert_close_stress, p_rounding_bound, run_gpu,
                               spiky_inputs)

pytestmark = pytest.mark.gpu

# (window_left, window_right, key_lens for B = 2); a negative bound is none.
MASKS = [
    (256, 0, None),          # causal sliding window
    (100, 37, None),         # two-sided window, not tile aligned
    (0, 0, None),            # each query sees only its own key
    (31, -1, None),          # left bound only
    (-1, -1, [700, 0]),      # padding; the second sequence is all padding
    (-1, 0, [333, 690]),     # causal with padding
    (50, -1, [512, 17]),     # left window and padding: rows past the keys see nothing
    (7, 3, [1, 650]),        # narrow window and a one-key sequence
]
DIMS = (32, 64, 96, 128, 256, 512, 1024)


def _ids(m):
    return f"w{m[0]}_{m[1]}_" + ("nolens" if m[2] is None else "lens" + "-".join(map(str, m[2])))


@pytest.mark.parametrize("mask", MASKS, ids=[_ids(m) for m in MASKS])
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
def test_masked_every_element(gpu_device, mask, d, dtype):
    wleft, wright, lens = mask
    w = wl.Workload("m", 2, 2, 700, d, dtype, False)
    q, k, v = wl.make_inputs(w, seed=9)
    o, lse = run_gpu(q, k, v, dtype, w.softmax_scale(), False, gpu_device, window=(wleft, wright), key_lens=lens)
    o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, dtype) for x in (q, k, v)), w.softmax_scale(),
                                          wleft, wright, lens)
    assert_close_masked(o, lse, o_ref, lse_ref, dtype, f"d{d} {dtype} window=({wleft},{wright}) lens={lens}")


@pytest.mark.parametrize("n", [1, 33, 255, 1027])
@pytest.mark.parametrize("d,dtype", [(64, wl.FP16), (128, wl.BF16), (256, wl.FP16)])
def test_masked_ragged_lengths(gpu_device, n, d, dtype):
    w = wl.Workload("r", 2, 1, n, d, dtype, False)
    q, k, v = wl.make_inputs(w, seed=n + 1)
    lens = [max(1, n // 3), n]
    for wleft, wright in ((64, 0), (5, 5)):
        o, lse = run_gpu(q, k, v, dtype, w.softmax_scale(), False, gpu_device, window=(wleft, wright),
                         key_lens=lens)
        o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, dtype) for x in (q, k, v)), w.softmax_scale(),
                                              wleft, wright, lens)
        assert_close_masked(o, lse, o_ref, lse_ref, dtype, f"N={n} d{d} window=({wleft},{wright})")


@pytest.mark.parametrize("d", DIMS)
def test_masked_without_mask_is_fwd_bit_for_bit(gpu_device, d):
    """No window and no lengths runs fa2_fwd's kernel; window (<0, 0) its causal one."""
    w = wl.Workload("b", 1, 3, 600, d, wl.FP16, False)
    q, k, v = wl.make_inputs(w, seed=2)
    for causal, window in ((False, (-1, -1)), (False, (600, 5000)), (True, (-1, 0)), (True, (900, 0))):
        o1, l1 = run_gpu(q, k, v, wl.FP16, w.softmax_scale(), causal, gpu_device)
        o2, l2 = run_gpu(q, k, v, wl.FP16, w.softmax_scale(), False, gpu_device, window=window)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_key_lens_are_clamped(gpu_device):
    w = wl.Workload("c", 2, 2, 300, 64, wl.BF16, False)
    q, k, v = wl.make_inputs(w, seed=4)
    o1, l1 = run_gpu(q, k, v, wl.BF16, w.softmax_scale(), False, gpu_device, window=(40, 2), key_lens=[-5, 1000])
    o2, l2 = run_gpu(q, k, v, wl.BF16, w.softmax_scale(), False, gpu_device, window=(40, 2), key_lens=[0, 300])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    assert np.all(np.isposinf(l1[0])) and np.all(o1[0] == 0)


def test_padding_contents_do_not_leak(gpu_device):
    """Keys and values past the key length may hold anything, NaN included."""
    import torch
    from exact_attention_21_amd import forward
    from tests.gpu_helpers import to_device
    w = wl.Workload("p", 2, 2, 500, 128, wl.FP16, False)
    q, k, v = wl.make_inputs(w, seed=6)
    lens = [123, 400]
    tq, tk, tv = (to_device(x, wl.FP16, gpu_device) for x in (q, k, v))
    kl = torch.tensor(lens, dtype=torch.int32, device=gpu_device)
    o1, l1 = forward(tq, tk, tv, window=(64, 8), key_lens=kl)
    tk2, tv2 = tk.clone(), tv.clone()
    for b, n_b in enumerate(lens):
        tk2[b, :, n_b:] = float("nan")
        tv2[b, :, n_b:] = float("inf")
    o2, l2 = forward(tq, tk2, tv2, window=(64, 8), key_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_masked_stress_late_window_start(gpu_device):
    """A narrow window far from the first key: each wave's rows see none of
    the workgroup's first tiles, so the checked pipeline meets fully hidden
    tiles before its first visible key (the -inf guards of the pages)."""
    w = wl.Workload("g", 1, 2, 2048, 64, wl.FP16, False)
    q, k, v = wl.make_inputs(w, seed=12)
    scale = 1 / math.sqrt(64)
    o, lse = run_gpu(q, k, v, wl.FP16, scale, False, gpu_device, window=(3, 0))
    o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, wl.FP16) for x in (q, k, v)), scale, 3, 0, None)
    assert_close_masked(o, lse, o_ref, lse_ref, wl.FP16, "window (3, 0)")


@pytest.mark.parametrize("w", wl.MASKED_WORKLOADS, ids=[w.name for w in wl.MASKED_WORKLOADS])
def test_masked_workload_full_size_sampled_rows(gpu_device, w):
    """The masked benchmark workloads at full size, in the launch the benchmark
    times; the oracle evaluates both ends of the sequence and random rows."""
    q, k, v = wl.make_inputs(w, seed=0)
    left, right = w.window if w.window is not None else (-1, -1)
    if w.causal:
        right = 0 if right < 0 else min(right, 0)
    o, lse = run_gpu(q, k, v, w.dtype, w.softmax_scale(), w.causal, gpu_device, window=w.window,
                     key_lens=list(w.key_lens) if w.key_lens is not None else None)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.N - 64, w.N), rng.choice(w.N, 128, replace=False)]))
    o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, w.dtype) for x in (q, k, v)), w.softmax_scale(),
                                          left, right, w.key_lens, rows=rows)
    assert_close_masked(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, w.dtype, w.name)


@pytest.mark.parametrize("d", (32, 64, 96, 256, 512, 1024))
@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
@pytest.mark.parametrize("mask", [(300, 0, None), (-1, 40, [1500, 900])], ids=["window", "padded"])
def test_masked_late_score_jumps(gpu_device, d, dtype, mask):
    """Score jumps half-way through the keys under a mask: the fixed base of
    the first (unchecked) run overflows and the workgroup reruns its keys
    through the checked pipeline.  O allows the P-rounding bound, as in the
    unmasked stress tests."""
    wleft, wright, lens = mask
    q, k, v = spiky_inputs(2, 2, 1500, d, dtype, seed=41, factor=12.0, where=(0.5, 0.83))
    scale = 1 / math.sqrt(d)
    o, lse = run_gpu(q, k, v, dtype, scale, False, gpu_device, window=(wleft, wright), key_lens=lens)
    o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, dtype) for x in (q, k, v)), scale, wleft, wright, lens)
    hidden = np.isposinf(lse_ref)
    assert np.array_equal(np.isposinf(lse), hidden) and np.all(o[hidden] == 0)
    bound = p_rounding_bound(q, k, v, o_ref, dtype, scale, False, mask=(wleft, wright, lens))
    seen = ~hidden
    assert_close_stress(o[seen], lse[seen], o_ref[seen], lse_ref[seen], bound[seen], dtype,
                        f"masked late jumps d{d} {dtype} window=({wleft},{wright}) lens={lens}")
