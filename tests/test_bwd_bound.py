"""CPU check of the backward parity tests' error bound (tests/bwd_helpers.py):
the kernels' rounding steps, replayed in fp64, stay within it, and the bound
is not so loose that a wrong gradient would pass (a gradient off by one
rounding step of dS per key, or with Delta dropped, exceeds it)."""
import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from tests import bwd_helpers as bh


CASES = [
    (1, 2, 67, 64, wl.FP16, False, None, (1, 1, 1, 1)),
    (1, 2, 67, 64, wl.FP16, True, None, (1, 1, 1, 1)),
    (2, 1, 130, 128, wl.BF16, True, None, (1, 1, 1, 1)),
    (1, 1, 96, 128, wl.BF16, False, -0.3, (1, 1, 1, 1)),
    (1, 1, 80, 64, wl.FP16, True, None, (3, 3, 1, 2)),  # peaked rows
    (1, 1, 64, 64, wl.FP16, False, 0.0, (1, 1, 1, 1)),
]


def _case(B, H, N, d, dtype, causal, scale, sigma, seed=5, mask=None):
    w, q, k, v, do = bh.make_case(B, H, N, d, dtype, seed, causal=causal, scale=scale, sigma=sigma)
    q64, k64, v64, do64 = (wl.to_float64(x, dtype) for x in (q, k, v, do))
    o_in, lse_in = bh.forward_inputs(q64, k64, v64, w.softmax_scale(), causal, dtype, mask=mask)
    return w, q64, k64, v64, do64, wl.to_float64(o_in, dtype), lse_in.astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[2]}d{c[3]}{c[4]}{'c' if c[5] else ''}s{c[6]}")
def test_replayed_rounding_within_bound(case):
    w, q64, k64, v64, do64, o_in, lse_in = _case(*case)
    refs, bounds = bh.grad_bounds(q64, k64, v64, do64, o_in, lse_in, w.softmax_scale(), w.causal, w.dtype)
    sim = bh.simulate_kernel_rounding(q64, k64, v64, do64, o_in, lse_in, w.softmax_scale(), w.causal, w.dtype)
    got = {n: sim[n].reshape(refs[n].shape) for n in sim}
    bh.assert_grads_within(got, refs, bounds, "replayed rounding")


def test_bound_rejects_wrong_gradients():
    w, q64, k64, v64, do64, o_in, lse_in = _case(1, 2, 67, 64, wl.FP16, True, None, (1, 1, 1, 1))
    refs, bounds = bh.grad_bounds(q64, k64, v64, do64, o_in, lse_in, w.softmax_scale(), w.causal, w.dtype)
    # dV from unnormalised rows (P scaled by 1.01), and dQ with Delta dropped.
    for name, bad in (("dv", refs["dv"] * 1.01), ("dq", None)):
        got = {n: refs[n].copy() for n in refs}
        if name == "dq":
            from oracle import attention_bwd_ref
            import oracle.attention as om
            saved = om._row_delta
            om._row_delta = lambda do, o: np.zeros((do.shape[0], 1))
            try:
                got["dq"] = attention_bwd_ref(q64, k64, v64, do64, w.softmax_scale(), True)[0].reshape(
                    refs["dq"].shape)
            finally:
                om._row_delta = saved
        else:
            got[name] = bad
        with pytest.raises(AssertionError):
            bh.assert_grads_within(got, refs, bounds, f"wrong {name}")


MASKS = [(8, 0, None), (-1, -1, [40, 0]), (5, 3, [70, 33]), (-1, 0, [50, 17]), (0, 0, None)]


@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_replayed_rounding_within_bound_masked(mask):
    w, q64, k64, v64, do64, o_in, lse_in = _case(2, 1, 75, 64, wl.FP16, False, None, (1, 1, 1, 1), mask=mask)
    refs, bounds = bh.grad_bounds(q64, k64, v64, do64, o_in, lse_in, w.softmax_scale(), False, w.dtype, mask=mask)
    sim = bh.simulate_kernel_rounding(q64, k64, v64, do64, o_in, lse_in, w.softmax_scale(), False, w.dtype,
                                      mask=mask)
    got = {n: sim[n].reshape(refs[n].shape) for n in sim}
    bh.assert_grads_within(got, refs, bounds, f"replayed rounding {mask}")
