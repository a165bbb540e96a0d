"""Seeded random shapes through both entry points, every element against the
fp64 oracle: batch, heads, length (1..900, so ragged tails of every kind),
head dim (every supported one), dtype, scale (either sign), and the mask
(none, causal, a random window, random key lengths, window and lengths,
causal and lengths).  Every element is held to the stated tolerances, except
that under a window or key lengths a row with fewer than 64 visible keys
adds the P-rounding bound (gpu_helpers.p_rounding_bound): with a scale up to
1.5/sqrt(d) a narrow window leaves a row a handful of keys, where the
rounding of P does not average out.  Each case prints the largest share of
that bound it needed."""
import math

import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl
from oracle import attention_ref, attention_ref_masked
from tests.gpu_helpers import assert_close, assert_close_stress, p_rounding_bound, run_gpu, visible_matrix

pytestmark = pytest.mark.gpu

DIMS = (32, 64, 96, 128, 256, 512, 1024)
# Rows with fewer visible keys than this carry the P-rounding bound.
FEW_KEYS = 64


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice(DIMS))
    # Keep the oracle's work (B H N^2 d) to a few GFLOP.
    n_max = 900 if d <= 256 else 400
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    N = int(rng.integers(1, n_max + 1))
    dtype = wl.FP16 if rng.random() < 0.5 else wl.BF16
    scale = float(rng.choice([1.0, -1.0]) * rng.uniform(0.3, 1.5) / math.sqrt(d))
    kind = ["none", "causal", "window", "lens", "window+lens", "causal+lens"][int(rng.integers(0, 6))]
    window = (-1, 0) if kind == "causal+lens" else None
    lens = None
    if "window" in kind:
        left = int(rng.integers(-1, N + 2))
        right = int(rng.integers(-1, 40)) if rng.random() < 0.5 else 0
        window = (left, right)
    if "lens" in kind:
        lens = [int(x) for x in rng.integers(0, N + 1, size=B)]
    return dict(B=B, H=H, N=N, d=d, dtype=dtype, scale=scale, causal=kind == "causal", window=window, lens=lens)


CASES = [draw_case(i) for i in range(40)]


@pytest.mark.parametrize("c", CASES, ids=[f"{i}-d{c['d']}-N{c['N']}-{c['dtype']}" for i, c in enumerate(CASES)])
def test_random_shape(gpu_device, c):
    w = wl.Workload("rand", c["B"], c["H"], c["N"], c["d"], c["dtype"], c["causal"])
    q, k, v = wl.make_inputs(w, seed=c["N"] + c["d"])
    f64 = [wl.to_float64(x, c["dtype"]) for x in (q, k, v)]
    label = str(c)
    if c["window"] is None and c["lens"] is None:
        o, lse = run_gpu(q, k, v, c["dtype"], c["scale"], c["causal"], gpu_device)
        o_ref, lse_ref = attention_ref(*f64, c["scale"], c["causal"])
        assert_close(o, lse, o_ref, lse_ref, c["dtype"], label)
        return
    left, right = c["window"] if c["window"] is not None else (-1, -1)
    o, lse = run_gpu(q, k, v, c["dtype"], c["scale"], False, gpu_device, window=(left, right), key_lens=c["lens"])
    o_ref, lse_ref = attention_ref_masked(*f64, c["scale"], left, right, c["lens"])
    hidden = np.isposinf(lse_ref)
    assert np.array_equal(np.isposinf(lse), hidden), f"{label}: fully hidden rows differ"
    assert np.all(o[hidden] == 0), f"{label}: O of a fully hidden row is not 0"
    if (~hidden).any():
        bound = p_rounding_bound(q, k, v, o_ref, c["dtype"], c["scale"], False, mask=(left, right, c["lens"]))
        n_vis = visible_matrix(c["N"], window=(left, right), key_lens=c["lens"], B=c["B"]).sum(axis=-1)
        bound = np.where((n_vis < FEW_KEYS)[:, None, :, None], bound, 0.0)
        seen = ~hidden
        assert_close_stress(o[seen], lse[seen], o_ref[seen], lse_ref[seen], bound[seen], c["dtype"], label)
