"""Pins for the fp64 oracle, checked against things other than itself.

* brute force: the literal textbook softmax (exp(s_ij) / sum_k exp(s_ik), no
  max shift) in pure Python with math.fsum, on tiny shapes;
* closed forms derived by hand (tests/golden/closed_forms.json);
* special cases: one key, identical keys, causal row 0, scale 0;
* invariants: shifting every key by u shifts LSE_i by scale * q_i . u and
  leaves O unchanged; permuting keys and values together changes nothing;
* library routines: torch scaled_dot_product_attention in fp64 on the CPU for
  O, scipy.special.logsumexp for LSE;
* the method's own algebra: the online (m, l) merge over key blocks of any
  size, in either order, reaches the same result;
* planted mistakes in the oracle are caught by the brute-force and
  closed-form pins: LSE in the wrong log base, a perturbed exponential, the
  causal diagonal excluded, the scale dropped, keys weighted unevenly, the
  scores transposed, the causal mask missing, the merge's rescale factor
  inverted, and (masked oracle) window bounds off by
  one, an exclusive right bound and the padding ignored;
* the row-subset evaluation (rows=) equals the matching rows of the full one.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_online_merge, attention_ref
import oracle.attention as oracle_mod

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def brute_force(q, k, v, scale, causal):
    """Pure-Python definition: P_ij = exp(s_ij) / sum_k exp(s_ik) (inputs kept small)."""
    c = float(np.float32(scale))
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                e = {j: math.exp(c * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t])
                                              for t in range(d))) for j in js}
                z = math.fsum(e.values())
                for t in range(d):
                    O[b, h, i, t] = math.fsum(e[j] * float(v[b, h, j, t]) for j in js) / z
                L[b, h, i] = math.log(z)
    return O, L


def _rand(shape, seed, width=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * width


TINY_SHAPES = [(1, 1, 1, 1), (1, 1, 2, 4), (2, 1, 3, 8), (1, 2, 17, 4), (2, 2, 5, 1), (1, 1, 17, 8)]


def check_brute_force(fn, tol=1e-12):
    for n_case, shape in enumerate(TINY_SHAPES):
        for causal in (False, True):
            q, k, v = (_rand(shape, 10 * n_case + t) for t in range(3))
            scale = 1.0 / math.sqrt(shape[-1])
            O, L = fn(q, k, v, scale, causal)
            Ob, Lb = brute_force(q, k, v, scale, causal)
            assert np.max(np.abs(O - Ob)) <= tol, (shape, causal)
            assert np.max(np.abs(L - Lb)) <= tol, (shape, causal)


def check_closed_forms(fn, tol=1e-12):
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        q = np.array(case["q"], dtype=np.float64)[None, None]
        k = np.array(case["k"], dtype=np.float64)[None, None]
        v = np.array(case["v"], dtype=np.float64)[None, None]
        for causal, key in ((False, "noncausal"), (True, "causal")):
            O, L = fn(q, k, v, case["scale"], causal)
            assert np.max(np.abs(O[0, 0] - np.array(case[key]["O"]))) <= tol, (case["name"], key)
            assert np.max(np.abs(L[0, 0] - np.array(case[key]["LSE"]))) <= tol, (case["name"], key)


def test_brute_force():
    check_brute_force(attention_ref)


def test_closed_forms():
    check_closed_forms(attention_ref)


def test_single_key():
    q, k, v = (_rand((2, 3, 1, 8), s) for s in range(3))
    for causal in (False, True):
        O, L = attention_ref(q, k, v, 0.3, causal)
        np.testing.assert_array_equal(O, v)
        c = float(np.float32(0.3))
        np.testing.assert_allclose(L, c * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_values():
    B, H, N, d = 1, 2, 33, 8
    q = _rand((B, H, N, d), 1)
    k = np.broadcast_to(_rand((B, H, 1, d), 2), (B, H, N, d)).copy()
    v = _rand((B, H, N, d), 3)
    c = float(np.float32(0.25))
    s = c * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0])
    O, L = attention_ref(q, k, v, 0.25, False)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-12)
    np.testing.assert_allclose(L, s + math.log(N), atol=1e-12)
    Oc, Lc = attention_ref(q, k, v, 0.25, True)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(Oc, prefix_mean, atol=1e-12)
    np.testing.assert_allclose(Lc, s + np.log(np.arange(1, N + 1))[None, None], atol=1e-12)


def test_causal_row_zero_is_first_value():
    q, k, v = (_rand((2, 2, 9, 4), s) for s in range(3))
    O, _ = attention_ref(q, k, v, 1.7, True)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])


def test_scale_zero_is_uniform():
    B, H, N, d = 1, 2, 20, 4
    q, k, v = (_rand((B, H, N, d), s, 5.0) for s in range(3))
    O, L = attention_ref(q, k, v, 0.0, False)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-12)
    np.testing.assert_allclose(L, np.full((B, H, N), math.log(N)), atol=1e-13)
    Oc, Lc = attention_ref(q, k, v, 0.0, True)
    np.testing.assert_allclose(Oc, np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None],
                               atol=1e-12)
    np.testing.assert_allclose(Lc, np.broadcast_to(np.log(np.arange(1, N + 1)), Lc.shape), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    # Shift every key by u: scores of row i move by c * q_i.u, softmax unchanged.
    # A large negative shift (c * q.u << 0) is the case where a running max
    # started at 0 instead of -inf underflows every exponential.
    B, H, N, d = 1, 2, 40, 16
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    q = np.abs(q) + 0.5
    c = float(np.float32(0.125))
    O, L = attention_ref(q, k, v, 0.125, causal)
    for shift in (3.0, -200.0):
        u = np.full(d, shift)
        O2, L2 = attention_ref(q, k + u, v, 0.125, causal)
        np.testing.assert_allclose(O2, O, atol=1e-10)
        np.testing.assert_allclose(L2, L + c * (q @ u), rtol=1e-13, atol=1e-9)
        assert np.all(np.isfinite(O2)) and np.all(np.isfinite(L2))


def test_key_value_permutation_invariance():
    B, H, N, d = 2, 1, 31, 8
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    perm = np.random.default_rng(7).permutation(N)
    O, L = attention_ref(q, k, v, 0.4, False)
    O2, L2 = attention_ref(q, k[:, :, perm], v[:, :, perm], 0.4, False)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)


def test_probabilities_sum_to_one():
    # P_ij = exp(s_ij - LSE_i) must sum to one over the visible keys.
    B, H, N, d = 1, 2, 50, 8
    q, k, v = (_rand((B, H, N, d), s, 2.0) for s in range(3))
    c = float(np.float32(0.35))
    for causal in (False, True):
        _, L = attention_ref(q, k, v, 0.35, causal)
        s = c * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        psum = np.exp(s - L[..., None]).sum(axis=-1)
        np.testing.assert_allclose(psum, 1.0, atol=1e-12)


def test_lse_against_scipy_logsumexp():
    from scipy.special import logsumexp
    B, H, N, d = 2, 2, 37, 8
    q, k, v = (_rand((B, H, N, d), s, 3.0) for s in range(3))
    c = float(np.float32(0.2))
    for causal in (False, True):
        _, L = attention_ref(q, k, v, 0.2, causal)
        s = c * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        np.testing.assert_allclose(L, logsumexp(s, axis=-1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(causal):
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 45, 16
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    scale = 0.3
    O, _ = attention_ref(q, k, v, scale, causal)
    t = [torch.from_numpy(x) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *t, is_causal=causal, scale=float(np.float32(scale))).numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12)


@pytest.mark.parametrize("block", [1, 7, 64])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_online_merge_reaches_definition(block, reverse, causal):
    B, H, N, d = 1, 2, 70, 8
    q, k, v = (_rand((B, H, N, d), s, 2.0) for s in range(3))
    O, L = attention_ref(q, k, v, 0.5, causal)
    O2, L2 = attention_online_merge(q, k, v, 0.5, causal, block, reverse)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)


def test_online_merge_brute_force_and_closed_forms():
    check_brute_force(lambda q, k, v, s, c: attention_online_merge(q, k, v, s, c, 3))
    check_closed_forms(lambda q, k, v, s, c: attention_online_merge(q, k, v, s, c, 1, True))


def test_rows_subset_matches_full():
    B, H, N, d = 2, 2, 600, 8
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    rows = np.array([0, 1, 255, 256, 257, 599, 300])
    for causal in (False, True):
        O, L = attention_ref(q, k, v, 0.3, causal)
        Os, Ls = attention_ref(q, k, v, 0.3, causal, rows=rows)
        # Equal up to BLAS summation order.
        np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Ls, L[:, :, rows], rtol=0, atol=1e-13)


class _NumpyWith:
    """numpy with one attribute replaced: plants a mistake in the oracle."""

    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        return self._over[name] if name in self._over else getattr(np, name)


MUTANTS = {
    "lse_in_log2": {"np": _NumpyWith(log=np.log2)},
    "exp_off_by_ulp_scale": {"np": _NumpyWith(exp=lambda x: np.exp(x * 1.001))},
    "causal_excludes_diagonal": {"_visible_count": lambda i, n, causal: i if causal else n},
    "scale_dropped": {"np": _NumpyWith(float32=lambda x: 1.0)},
    "exp_weights_alternate_keys": {"np": _NumpyWith(exp=lambda x: np.exp(x) * (np.arange(x.shape[-1]) % 2 + 1))},
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    for name, val in MUTANTS[mutant].items():
        monkeypatch.setattr(oracle_mod, name, val)
    caught = 0
    for check in (check_brute_force, check_closed_forms):
        try:
            check(attention_ref)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"planted mistake {mutant} went unnoticed"


# Mistakes in how the definition is assembled: the scores transposed (K Q^T
# where Q K^T belongs, so each softmax runs over queries), and the causal mask
# left out.
CALL_MUTANTS = {
    "scores_transposed": lambda q, k, v, s, c: attention_ref(k, q, v, s, c),
    "causal_mask_missing": lambda q, k, v, s, c: attention_ref(q, k, v, s, False),
}


@pytest.mark.parametrize("mutant", sorted(CALL_MUTANTS))
def test_pins_catch_planted_call_mistakes(mutant):
    caught = 0
    for check in (check_brute_force, check_closed_forms):
        try:
            check(CALL_MUTANTS[mutant])
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"planted mistake {mutant} went unnoticed"


# A mistake in the online merge: the rescale factor inverted (the slip in the
# paper's printed formula that the MMA notes point out).  (A base that is not
# moved is no mistake: any base gives the same softmax while nothing
# overflows, which is what the kernel's lazily moved base relies on.)
MERGE_MUTANTS = {
    "rescale_inverted": {"_rescale_factor": lambda m_old, m_new: np.exp(m_new - m_old)},
}


@pytest.mark.parametrize("mutant", sorted(MERGE_MUTANTS))
def test_merge_pins_catch_planted_mistakes(monkeypatch, mutant):
    for name, val in MERGE_MUTANTS[mutant].items():
        monkeypatch.setattr(oracle_mod, name, val)
    caught = 0
    checks = (lambda: check_brute_force(lambda q, k, v, s, c: attention_online_merge(q, k, v, s, c, 3)),
              lambda: check_closed_forms(lambda q, k, v, s, c: attention_online_merge(q, k, v, s, c, 1, True)),
              lambda: test_online_merge_reaches_definition(7, False, False))
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"planted mistake {mutant} went unnoticed"


# ---- sliding-window and padding masks -------------------------------------

from oracle import attention_ref_masked  # noqa: E402

MASKS = [(-1, -1, None), (0, 0, None), (1, 0, None), (2, 1, None), (0, -1, None), (-1, 0, None),
         (-1, -1, [0, 1]), (-1, -1, [1, 3]), (3, 2, [2, 17]), (-1, 0, [5, 0])]


def brute_force_masked(q, k, v, scale, window_left, window_right, key_lens):
    """Pure-Python definition with the mask written out: key j counts for
    query i when j < len, (left bound absent or j >= i - left) and (right
    bound absent or j <= i + right); no visible key gives O = 0, LSE = inf."""
    c = float(np.float32(scale))
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.full((B, H, N), math.inf)
    for b in range(B):
        n_keys = N if key_lens is None else min(max(key_lens[b], 0), N)
        for h in range(H):
            for i in range(N):
                js = [j for j in range(N) if j < n_keys
                      and (window_left < 0 or j >= i - window_left)
                      and (window_right < 0 or j <= i + window_right)]
                if not js:
                    continue
                e = {j: math.exp(c * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t])
                                              for t in range(d))) for j in js}
                z = math.fsum(e.values())
                for t in range(d):
                    O[b, h, i, t] = math.fsum(e[j] * float(v[b, h, j, t]) for j in js) / z
                L[b, h, i] = math.log(z)
    return O, L


def _assert_close_inf(a, b, tol, what):
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    assert np.array_equal(np.isinf(a), np.isinf(b)), what
    assert np.max(np.where(both_inf, 0.0, np.abs(np.where(both_inf, 0.0, a) - np.where(both_inf, 0.0, b)))) <= tol, what


def check_brute_force_masked(fn, tol=1e-12):
    for n_case, shape in enumerate(TINY_SHAPES):
        for wl, wr, lens in MASKS:
            lens_b = None if lens is None else (lens * shape[0])[:shape[0]]
            q, k, v = (_rand(shape, 10 * n_case + t) for t in range(3))
            scale = 1.0 / math.sqrt(shape[-1])
            O, L = fn(q, k, v, scale, wl, wr, lens_b)
            Ob, Lb = brute_force_masked(q, k, v, scale, wl, wr, lens_b)
            assert np.max(np.abs(O - Ob)) <= tol, (shape, wl, wr, lens_b)
            _assert_close_inf(L, Lb, tol, (shape, wl, wr, lens_b))


def check_closed_forms_masked(fn, tol=1e-12):
    for case in json.load(open(GOLDEN))["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, None]
        k = np.array(case["k"], dtype=np.float64)[None, None]
        v = np.array(case["v"], dtype=np.float64)[None, None]
        for m in case["masked"]:
            O, L = fn(q, k, v, case["scale"], m["window_left"], m["window_right"], [m["key_len"]])
            what = (case["name"], m["window_left"], m["window_right"], m["key_len"])
            assert np.max(np.abs(O[0, 0] - np.array(m["O"]))) <= tol, what
            _assert_close_inf(L[0, 0], np.array(m["LSE"], dtype=np.float64), tol, what)


def test_masked_brute_force():
    check_brute_force_masked(attention_ref_masked)


def test_masked_closed_forms():
    check_closed_forms_masked(attention_ref_masked)


def test_masked_reduces_to_full_and_causal():
    q, k, v = (_rand((2, 2, 300, 8), s) for s in range(3))
    for causal, (wl, wr) in ((False, (-1, -1)), (True, (-1, 0))):
        O, L = attention_ref(q, k, v, 0.4, causal)
        Om, Lm = attention_ref_masked(q, k, v, 0.4, wl, wr, None)
        np.testing.assert_allclose(Om, O, rtol=0, atol=1e-13)
        np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-13)
    # A key length of N is no padding; a window wider than N is no window.
    Om, Lm = attention_ref_masked(q, k, v, 0.4, 300, 299, [300, 300])
    O, L = attention_ref(q, k, v, 0.4, False)
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-13)


def test_masked_padding_does_not_leak():
    """Keys and values past the key length may hold anything."""
    B, H, N, d = 2, 2, 40, 8
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    lens = [23, 7]
    k2, v2 = k.copy(), v.copy()
    for b, n_b in enumerate(lens):
        k2[b, :, n_b:] = 1e3
        v2[b, :, n_b:] = -1e6
    for wl, wr in ((-1, -1), (5, 0), (3, 3)):
        O, L = attention_ref_masked(q, k, v, 0.3, wl, wr, lens)
        O2, L2 = attention_ref_masked(q, k2, v2, 0.3, wl, wr, lens)
        np.testing.assert_array_equal(O, O2)
        np.testing.assert_array_equal(L, L2)


def test_masked_fully_hidden_rows():
    """Rows that see no key: all keys padding, or a window that lies past the
    key length."""
    q, k, v = (_rand((2, 1, 12, 4), s) for s in range(3))
    O, L = attention_ref_masked(q, k, v, 1.0, 0, 2, [0, 4])
    assert np.all(O[0] == 0) and np.all(np.isposinf(L[0]))
    # batch 1: rows 0..3 see their own key; rows >= 4 see none (keys 4.. are padding).
    np.testing.assert_array_equal(np.isposinf(L[1, 0]), np.arange(12) >= 4)
    assert np.all(O[1, 0, 4:] == 0)


@pytest.mark.parametrize("block", [1, 7, 64])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mask", [(5, 0, None), (2, 9, [40, 13]), (-1, -1, [0, 70]), (0, 0, None)])
def test_online_merge_masked_reaches_definition(block, reverse, mask):
    """Under these masks some rows see only hidden keys in their first blocks
    (or in every block): the merge's -inf guards decide the result."""
    wl, wr, lens = mask
    q, k, v = (_rand((2, 2, 70, 8), s, 2.0) for s in range(3))
    O, L = attention_ref_masked(q, k, v, 0.5, wl, wr, lens)
    O2, L2 = attention_online_merge(q, k, v, 0.5, False, block, reverse, window=(wl, wr), key_lens=lens)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    _assert_close_inf(L2, L, 1e-12, (block, reverse, mask))


MASK_MUTANTS = {
    "left_bound_off_by_one": lambda i, wl, wr, n: (0 if wl < 0 else max(0, i - wl + 1),
                                                   n if wr < 0 else min(n, i + wr + 1)),
    "right_bound_exclusive": lambda i, wl, wr, n: (0 if wl < 0 else max(0, i - wl),
                                                   n if wr < 0 else min(n, i + wr)),
    "padding_ignored": lambda i, wl, wr, n: (0 if wl < 0 else max(0, i - wl),
                                             10 ** 9 if wr < 0 else i + wr + 1),
}


@pytest.mark.parametrize("mutant", sorted(MASK_MUTANTS))
def test_masked_pins_catch_planted_mistakes(monkeypatch, mutant):
    bad = MASK_MUTANTS[mutant]
    monkeypatch.setattr(oracle_mod, "_visible_range", lambda i, wl, wr, n: (lambda lo, hi: (lo, max(lo, hi)))(*bad(i, wl, wr, n)))
    caught = 0
    for check in (check_brute_force_masked, check_closed_forms_masked):
        try:
            check(attention_ref_masked)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"planted mistake {mutant} went unnoticed"


@pytest.mark.parametrize("mask", [(-1, -1, None), (40, 0, None), (100, 37, None), (0, 0, None), (31, -1, None),
                                  (-1, -1, [600, 0]), (-1, 0, [333, 590]), (50, -1, [300, 17]), (7, 3, [1, 560])])
def test_masked_rows_subset_matches_full(mask):
    """attention_ref_masked(rows=...) returns exactly the matching rows of the
    full evaluation: unsorted rows, rows on both sides of the 256-row block
    boundaries, repeated rows and fully hidden rows (all padding, or a window
    past the key length)."""
    left, right, lens = mask
    B, H, N, d = 2, 2, 600, 8
    q, k, v = (_rand((B, H, N, d), s) for s in range(3))
    O, L = attention_ref_masked(q, k, v, 0.3, left, right, lens)
    rng = np.random.default_rng(17)
    for rows in (np.array([599, 0, 255, 256, 257, 511, 512, 513, 300, 300, 1]),
                 np.arange(250, 520), rng.choice(N, size=300, replace=False), np.array([42])):
        Os, Ls = attention_ref_masked(q, k, v, 0.3, left, right, lens, rows=rows)
        assert Os.shape == (B, H, rows.size, d) and Ls.shape == (B, H, rows.size)
        np.testing.assert_allclose(Os, O[:, :, rows], rtol=0, atol=1e-13)
        _assert_close_inf(Ls, L[:, :, rows], 1e-13, (mask, rows[:3]))
    if lens is not None and 0 in lens:
        assert np.all(np.isposinf(L[lens.index(0)]))
