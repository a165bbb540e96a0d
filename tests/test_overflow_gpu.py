"""Scores far above the exponent base of the unchecked first run.

For d <= 256 the kernel first runs every key tile with each row's exponent
base fixed at the row max of its first key tile, and reruns the workgroup's
keys through the checked pipeline (which moves the base whenever a tile's
probabilities could overflow) if that first run overflowed: a row sum that is
not finite, or, for bf16, an output accumulator that is not finite.  The
pages rescale on every tile instead ("第 15 章 FA2 前向：Tiling 与 Online
Softmax", §15.4.1); the lazily moved base has to reach the same result.

Inputs (jump_inputs): N(0,1) queries and keys with q[0] = 4; a few keys score
a fixed number of base-2 units for every query, far above the others.
  * jumps of 140 and 175 units: every probability of those keys overflows
    16-bit storage against the first tile's base, so the rerun must run;
  * a jump of 127 units on a key whose value row is +-300: the bf16
    probability (about 2^121..2^126) and the row sum stay finite, while
    p * v overflows the fp32 accumulator; the first run must be rejected on
    its accumulators;
  * scale 0: every visible key weighs the same; hidden keys meet a 0 * -inf
    exponent that the guards must turn into probability 0.
Rows that see a jump put all their weight on one key, so O is that key's
value row; the stated tolerances apply to every element, with no extra
allowance.
"""
import math

import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from oracle import attention_ref_masked
from tests.gpu_helpers import assert_close_masked, jump_above_rest, jump_inputs, run_gpu, visible_matrix

pytestmark = pytest.mark.gpu

B, H, N = 2, 1, 1100
DIMS = (32, 64, 96, 128, 256, 512, 1024)
# (window_left, window_right, key_lens); a negative bound is none.  (-1, -1)
# runs the unmasked kernel and (-1, 0) the causal one (with key lengths when
# given); the others run the general-mask kernel.
MASKS = {
    "none": (-1, -1, None),
    "causal": (-1, 0, None),
    "causal_window": (450, 0, None),
    "two_sided": (300, 50, None),
    "lens": (-1, -1, [1000, 640]),
}


def run_case(dev, q, k, v, dtype, scale, mask, label):
    left, right, lens = mask
    o, lse = run_gpu(q, k, v, dtype, scale, False, dev, window=(left, right), key_lens=lens)
    o_ref, lse_ref = attention_ref_masked(*(wl.to_float64(x, dtype) for x in (q, k, v)), scale, left, right, lens)
    assert_close_masked(o, lse, o_ref, lse_ref, dtype, label)


def seen_jumps(q, k, dtype, scale, spikes, mask):
    left, right, lens = mask
    vis = visible_matrix(N, window=(left, right), key_lens=lens, B=B)
    j = jump_above_rest(q, k, dtype, scale, spikes, vis)
    return j[np.isfinite(j)]


@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
def test_jump_forces_checked_rerun(gpu_device, d, dtype, mask):
    scale = 1 / math.sqrt(d)
    q, k, v, spikes = jump_inputs(B, H, N, d, dtype, seed=d + 7, scale=scale, jumps=[(0.5, 140.0), (0.83, 175.0)])
    j = seen_jumps(q, k, dtype, scale, spikes, MASKS[mask])
    assert j.size > 0 and j.min() >= 130.0, f"jump above the other keys {j.min():.1f} < 130"
    print(f"  jump above every other visible key: {j.min():.1f} .. {j.max():.1f} base-2 units", flush=True)
    run_case(gpu_device, q, k, v, dtype, scale, MASKS[mask], f"jump d{d} {dtype} {mask}")


@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
def test_jump_overflows_accumulator_not_row_sum(gpu_device, d, dtype, mask):
    scale = 1 / math.sqrt(d)
    q, k, v, spikes = jump_inputs(B, H, N, d, dtype, seed=d + 9, scale=scale, jumps=[(0.6, 127.0)], v_spike=300.0)
    j = seen_jumps(q, k, dtype, scale, spikes, MASKS[mask])
    assert j.size > 0 and 115.0 <= j.min() and j.max() <= 127.5, (j.min(), j.max())
    print(f"  jump above every other visible key: {j.min():.1f} .. {j.max():.1f} base-2 units; |v| = 300",
          flush=True)
    run_case(gpu_device, q, k, v, dtype, scale, MASKS[mask], f"accumulator overflow d{d} {dtype} {mask}")


@pytest.mark.parametrize("mask", sorted(MASKS))
@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
def test_scale_zero(gpu_device, d, dtype, mask):
    w = wl.Workload("z", B, H, N, d, dtype, False)
    q, k, v = wl.make_inputs(w, seed=d + 11)
    run_case(gpu_device, q, k, v, dtype, 0.0, MASKS[mask], f"scale 0 d{d} {dtype} {mask}")
