"""The seeded input generator: shapes, determinism, and round-to-nearest-even."""
import numpy as np
import pytest

from exact_attention_21_amd import workloads as wl


def test_five_workloads():
    assert [w.name for w in wl.WORKLOADS] == [wl.TINY.name, wl.HEADLINE.name, wl.CAUSAL_TRAIN.name,
                                               wl.LONG_CAUSAL.name, wl.WIDE_RAGGED.name]
    assert wl.HEADLINE.flops() == 4 * 8 * 8192 ** 2 * 64
    assert wl.LONG_CAUSAL.flops() == 4 * 4 * 32768 ** 2 * 64 / 2


def test_deterministic_and_shaped():
    a = wl.make_inputs(wl.TINY, seed=0)
    b = wl.make_inputs(wl.TINY, seed=0)
    c = wl.make_inputs(wl.TINY, seed=1)
    for x, y in zip(a, b):
        assert x.shape == (1, 1, 128, 64) and x.dtype == np.float16
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_fp16_is_round_to_nearest_even():
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, -0.1], dtype=np.float64)
    r = wl.round_to_storage(x, wl.FP16)
    assert r.dtype == np.float16
    np.testing.assert_array_equal(wl.to_float64(r, wl.FP16), [1.0, 1.0 + 2.0 ** -9, 65504.0, float(np.float16(-0.1))])


def test_bf16_matches_torch_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(3).standard_normal(10000) * 10.0
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0]   # exact ties go to even
    bits = wl.round_to_storage(x, wl.BF16)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    up = wl.to_float64(bits, wl.BF16)
    assert up[0] == 1.0 and up[1] == 1.0 + 2.0 ** -6


def test_wide_ragged_distributions():
    q, k, v = wl.make_inputs(wl.WIDE_RAGGED, seed=0, B=1, H=1)
    qf, vf = wl.to_float64(q, wl.BF16), wl.to_float64(v, wl.BF16)
    assert q.shape == (1, 1, 2047, 256)
    assert 2.8 < qf.std() < 3.2
    assert vf.min() >= -1.0 and vf.max() <= 1.0


def test_masked_workload_flops_count_visible_pairs():
    w = wl.WINDOW
    n, left = w.N, w.window[0]
    pairs = sum(min(i, left) + 1 for i in range(n))
    assert w.flops() == 4.0 * w.H * w.d * pairs
    p = wl.PADDED_CAUSAL
    pairs = sum(sum(min(i + 1, n_b) for i in range(p.N)) for n_b in p.key_lens)
    assert p.flops() == 4.0 * p.H * p.d * pairs
    # The unmasked count is unchanged: causal halves the square.
    assert wl.CAUSAL_TRAIN.flops() == 4 * 2 * 16 * 4096 ** 2 * 128 / 2
