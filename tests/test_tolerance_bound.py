"""CPU checks of the P-rounding bound used by the stress parity tests.

The pages round the probabilities to the input dtype once before P.V and
accumulate O in fp32 (yangyitao.com ch.15 §15.4.2).  Here that rounding is
emulated in fp64 against several exponent bases (the row max, and bases below
it as a kernel with a lagging base uses), and the emulated O must stay within
p_rounding_bound of the exact O, while the bound is far from vacuous.
"""
import math

import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from oracle import attention_ref
from tests.gpu_helpers import p_rounding_bound, spiky_inputs


def emulate_rounded_p(q, k, v, dtype, scale, causal, shift):
    """O with every probability exp2(s - m + shift) rounded to `dtype`
    (m: row max of the base-2 scores) and normalised by the rounded sum."""
    qf, kf, vf = (wl.to_float64(x, dtype) for x in (q, k, v))
    s = np.einsum("bhid,bhjd->bhij", qf, kf) * float(np.float32(scale)) * math.log2(math.e)
    n = s.shape[-1]
    if causal:
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    p = np.exp2(s - s.max(axis=-1, keepdims=True) + shift)
    pr = wl.to_float64(wl.round_to_storage(p, dtype), dtype)
    return (pr @ vf) / pr.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("dtype", [wl.FP16, wl.BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shift", [0.0, 0.37, 3.81])
def test_rounded_p_within_bound(dtype, causal, shift):
    d = 32
    q, k, v = spiky_inputs(1, 2, 300, d, dtype, seed=7, factor=12.0, where=(0.5, 0.83))
    scale = 1 / math.sqrt(d)
    o_ref, _ = attention_ref(*(wl.to_float64(x, dtype) for x in (q, k, v)), scale, causal)
    bound = p_rounding_bound(q, k, v, o_ref, dtype, scale, causal)
    err = np.abs(emulate_rounded_p(q, k, v, dtype, scale, causal, shift) - o_ref)
    assert np.all(err <= bound + 1e-12)
    # The rounding reaches a sizeable share of the bound somewhere.
    assert np.max(err / np.maximum(bound, 1e-300)) > 0.1


def test_bound_zero_for_single_key():
    """One visible key (causal row 0) has no spread of V: the bound is 0 for
    bf16 and only the fp16 subnormal term for fp16."""
    q, k, v = spiky_inputs(1, 1, 64, 32, wl.BF16, seed=3, factor=1.0, where=())
    o_ref, _ = attention_ref(*(wl.to_float64(x, wl.BF16) for x in (q, k, v)), 0.2, True)
    bound = p_rounding_bound(q, k, v, o_ref, wl.BF16, 0.2, True)
    assert np.all(bound[:, :, 0] <= 1e-7)
    assert np.all(bound[:, :, 1:].max(axis=-1) > 0)
