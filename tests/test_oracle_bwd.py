"""Pins for the fp64 backward oracle (attention_bwd_ref), checked against
things other than its own formulas.

* central finite differences of the (separately pinned) forward oracle:
  the gradient of f(Q, K, V) = sum(dO * O) element by element, on tiny shapes;
* a closed form derived by hand: one query dimension and two keys, where the
  softmax is a logistic function of the score difference;
* special cases: one key (O = V, so dV = dO and dQ = dK = 0), the causal
  row 0 (one visible key, so dQ_0 = 0), scale 0 (uniform P: dV_j is the mean
  of dO over the rows that see key j);
* invariants: the rows of dS sum to zero, so sum_j dK_j = 0; the rows of P
  sum to one, so sum_j dV_j = sum_i dO_i; scaling Q by t and K by 1/t leaves
  S unchanged, so sum q . dQ = sum k . dK; O is linear in V, so
  sum v . dV = sum dO . O;
* a library routine: torch autograd through scaled_dot_product_attention in
  fp64 on the CPU;
* planted mistakes in the oracle (the row term Delta dropped, dS transposed,
  the causal mask missing, the scores transposed, a perturbed exponential,
  the scale dropped) are each caught by at least one of the pins above.

The masked backward (attention_bwd_ref_masked: sliding window and key
lengths) is pinned by finite differences through the (separately pinned)
masked forward oracle, including rows that see no key; torch autograd with a
boolean mask built here from the definition (and dQ = 0 on hidden rows);
reduction to attention_bwd_ref for no window, the causal window and a window
wider than N; and padding that changes nothing (K, V rows past a length
replaced, dK = dV = 0 there).  Planted mistakes: the left bound off by one,
the key lengths ignored.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as oracle_mod
from oracle import attention_bwd_ref, attention_ref

TINY = [(1, 1, 1, 1), (1, 1, 3, 2), (1, 2, 5, 3), (2, 1, 4, 4), (1, 1, 6, 2)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(shape, seed):
    return tuple(_rand(shape, 100 * seed + t) for t in range(4))


def finite_difference_grads(q, k, v, do, scale, causal, h=1e-5):
    """Central differences of sum(dO * O) through the forward oracle."""
    def f(qq, kk, vv):
        return float(np.sum(do * attention_ref(qq, kk, vv, scale, causal)[0]))

    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            base = args[which][idx]
            args[which][idx] = base + h
            fp = f(*args)
            args[which][idx] = base - h
            fm = f(*args)
            args[which][idx] = base
            g[idx] = (fp - fm) / (2 * h)
        grads.append(g)
    return grads


def check_finite_differences(fn, tol=1e-7):
    for n_case, shape in enumerate(TINY):
        for causal in (False, True):
            q, k, v, do = _inputs(shape, n_case)
            scale = 0.7 / math.sqrt(shape[-1])
            got = fn(q, k, v, do, scale, causal)
            want = finite_difference_grads(q, k, v, do, scale, causal)
            for name, a, b in zip(("dQ", "dK", "dV"), got, want):
                assert np.max(np.abs(a - b)) <= tol, (shape, causal, name, np.max(np.abs(a - b)))


def check_two_key_closed_form(fn, tol=1e-12):
    """d = 1, two keys a and b, values v1 and v2, non-causal.

    With x_i = c q_i (a - b) the softmax gives p_i = sigma(x_i) to key a, so
    O_i = v2 + p_i (v1 - v2) and, by hand:
      dO_i/dq_i = p_i (1 - p_i) c (a - b) (v1 - v2)
      dO_i/da   = p_i (1 - p_i) c q_i (v1 - v2),   dO_i/db = -dO_i/da
      dO_i/dv1  = p_i,                             dO_i/dv2 = 1 - p_i
    """
    c = float(np.float32(0.9))
    q = np.array([0.3, -1.2])
    a, bb, v1, v2 = 0.8, -0.5, 2.0, -1.5
    do = np.array([0.7, -0.4])
    x = c * q * (a - bb)
    p = 1.0 / (1.0 + np.exp(-x))
    w = p * (1 - p)
    dq_want = do * w * c * (a - bb) * (v1 - v2)
    da = float(np.sum(do * w * c * q * (v1 - v2)))
    dk_want = np.array([da, -da])
    dv_want = np.array([float(np.sum(do * p)), float(np.sum(do * (1 - p)))])
    dq, dk, dv = fn(q.reshape(1, 1, 2, 1), np.array([a, bb]).reshape(1, 1, 2, 1),
                    np.array([v1, v2]).reshape(1, 1, 2, 1), do.reshape(1, 1, 2, 1), 0.9, False)
    assert np.max(np.abs(dq.ravel() - dq_want)) <= tol
    assert np.max(np.abs(dk.ravel() - dk_want)) <= tol
    assert np.max(np.abs(dv.ravel() - dv_want)) <= tol


def check_invariants(fn, tol=1e-11):
    for n_case, shape in enumerate([(1, 2, 9, 4), (2, 1, 16, 8), (1, 1, 1, 3)]):
        for causal in (False, True):
            q, k, v, do = _inputs(shape, 50 + n_case)
            scale = 0.5
            dq, dk, dv = fn(q, k, v, do, scale, causal)
            o = attention_ref(q, k, v, scale, causal)[0]
            assert np.max(np.abs(dk.sum(axis=2))) <= tol, (shape, causal, "sum dK")
            assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= tol, (shape, causal, "sum dV")
            lhs = np.einsum("bhnd,bhnd->bh", q, dq)
            rhs = np.einsum("bhnd,bhnd->bh", k, dk)
            assert np.max(np.abs(lhs - rhs)) <= tol, (shape, causal, "q.dQ = k.dK")
            lhs = np.einsum("bhnd,bhnd->bh", v, dv)
            rhs = np.einsum("bhnd,bhnd->bh", do, o)
            assert np.max(np.abs(lhs - rhs)) <= tol, (shape, causal, "v.dV = dO.O")


def check_against_torch(fn, tol=1e-12):
    for n_case, shape in enumerate([(2, 2, 7, 5), (1, 1, 33, 16)]):
        for causal in (False, True):
            q, k, v, do = _inputs(shape, 70 + n_case)
            scale = 0.4
            got = fn(q, k, v, do, scale, causal)
            t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
            o = torch.nn.functional.scaled_dot_product_attention(
                *t, is_causal=causal, scale=float(np.float32(scale)))
            o.backward(torch.tensor(do))
            for name, a, b in zip(("dQ", "dK", "dV"), got, t):
                assert np.max(np.abs(a - b.grad.numpy())) <= tol, (shape, causal, name)


CHECKS = (check_finite_differences, check_two_key_closed_form, check_invariants, check_against_torch)


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_backward_oracle(check):
    check(attention_bwd_ref)


def test_single_key_and_causal_row_zero():
    q, k, v, do = _inputs((2, 3, 1, 6), 3)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.8, False)
    assert np.max(np.abs(dv - do)) <= 1e-15
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    q, k, v, do = _inputs((1, 2, 11, 4), 4)
    dq = attention_bwd_ref(q, k, v, do, 0.8, True)[0]
    assert np.max(np.abs(dq[:, :, 0])) <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_uniform_weights(causal):
    n = 9
    q, k, v, do = _inputs((1, 2, n, 4), 5)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, 0.0, causal)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0
    for j in range(n):
        rows = range(j, n) if causal else range(n)
        want = sum(do[:, :, i] / ((i + 1) if causal else n) for i in rows)
        assert np.max(np.abs(dv[:, :, j] - want)) <= 1e-14


class _NumpyWith:
    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        return self._over[name] if name in self._over else getattr(np, name)


MODULE_MUTANTS = {
    "delta_dropped": {"_row_delta": lambda do, o: np.zeros((do.shape[0], 1))},
    "score_grad_transposed": {"_score_grad": lambda p, dp, delta: (p * (dp - delta)).T},
    "exp_perturbed": {"np": _NumpyWith(exp=lambda x: np.exp(x * 1.001))},
    "scale_dropped": {"np": _NumpyWith(float32=lambda x: 1.0)},
}

CALL_MUTANTS = {
    "causal_mask_missing": lambda q, k, v, do, s, c: attention_bwd_ref(q, k, v, do, s, False),
    "scores_transposed": lambda q, k, v, do, s, c: (lambda g: (g[1], g[0], g[2]))(
        attention_bwd_ref(k, q, v, do, s, c)),
}


def _caught(fn):
    caught = 0
    for check in CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(fn)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    return caught


@pytest.mark.parametrize("mutant", sorted(MODULE_MUTANTS))
def test_backward_pins_catch_planted_mistakes(monkeypatch, mutant):
    for name, val in MODULE_MUTANTS[mutant].items():
        monkeypatch.setattr(oracle_mod, name, val)
    assert _caught(oracle_mod.attention_bwd_ref) >= 1, f"planted mistake {mutant} went unnoticed"


@pytest.mark.parametrize("mutant", sorted(CALL_MUTANTS))
def test_backward_pins_catch_planted_call_mistakes(mutant):
    assert _caught(CALL_MUTANTS[mutant]) >= 1, f"planted mistake {mutant} went unnoticed"


# ---- sliding window and key lengths ------------------------------------------
from oracle import attention_bwd_ref_masked, attention_ref_masked  # noqa: E402

# (shape, window_left, window_right, key_lens): windows on both sides, one
# side, none; key lengths with a padded tail, a fully padded sequence, and
# windows that leave rows with no visible key.
MASK_CASES = [
    ((1, 2, 6, 3), 2, 1, None),
    ((2, 1, 7, 2), -1, 0, [5, 7]),
    ((2, 1, 6, 4), 1, -1, [3, 0]),
    ((1, 1, 8, 2), 0, 0, None),
    ((2, 2, 5, 3), 1, 0, [2, 4]),  # rows 3, 4 of batch 0 see no key
]


def _mask_matrix(n, left, right, key_len):
    """Test-side visibility, written from the definition: key j is visible to
    query i iff j < key_len, j >= i - left (left >= 0) and j <= i + right
    (right >= 0)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = j < key_len
    if left >= 0:
        vis = vis & (j >= i - left)
    if right >= 0:
        vis = vis & (j <= i + right)
    return vis


def check_masked_finite_differences(fn, tol=1e-7):
    for n_case, (shape, left, right, lens) in enumerate(MASK_CASES):
        q, k, v, do = _inputs(shape, 200 + n_case)
        scale = 0.6

        def f(qq, kk, vv):
            return float(np.sum(do * attention_ref_masked(qq, kk, vv, scale, left, right, lens)[0]))

        got = fn(q, k, v, do, scale, left, right, lens)
        for which in range(3):
            args = [q.copy(), k.copy(), v.copy()]
            g = np.zeros_like(args[which])
            for idx in np.ndindex(g.shape):
                base = args[which][idx]
                args[which][idx] = base + 1e-5
                fp = f(*args)
                args[which][idx] = base - 1e-5
                fm = f(*args)
                args[which][idx] = base
                g[idx] = (fp - fm) / 2e-5
            assert np.max(np.abs(got[which] - g)) <= tol, (shape, left, right, lens, which)


def check_masked_against_torch(fn, tol=1e-12):
    """torch autograd through scaled_dot_product_attention with a boolean
    mask, on rows that see at least one key (torch gives NaN on the others);
    the oracle's hidden rows must have dQ = 0."""
    for n_case, (shape, left, right, lens) in enumerate(MASK_CASES):
        q, k, v, do = _inputs(shape, 300 + n_case)
        B, H, N, d = shape
        scale = 0.6
        got = fn(q, k, v, do, scale, left, right, lens)
        for b in range(B):
            vis = _mask_matrix(N, left, right, N if lens is None else lens[b])
            seen = vis.any(axis=1)
            assert np.all(got[0][b][:, ~seen] == 0.0), "hidden rows must have dQ = 0"
            if not seen.any():
                assert np.all(got[1][b] == 0.0) and np.all(got[2][b] == 0.0)
                continue
            rows = np.nonzero(seen)[0]
            t = [torch.tensor(x[b:b + 1], requires_grad=True) for x in (q, k, v)]
            qs = t[0][:, :, rows]
            o = torch.nn.functional.scaled_dot_product_attention(
                qs, t[1], t[2], attn_mask=torch.tensor(vis[rows]), scale=float(np.float32(scale)))
            o.backward(torch.tensor(do[b:b + 1, :, rows]))
            assert np.max(np.abs(got[0][b][:, rows] - t[0].grad.numpy()[0][:, rows])) <= tol
            assert np.max(np.abs(got[1][b] - t[1].grad.numpy()[0])) <= tol
            assert np.max(np.abs(got[2][b] - t[2].grad.numpy()[0])) <= tol


def check_masked_reduces_to_unmasked(fn, tol=1e-13):
    q, k, v, do = _inputs((2, 2, 9, 4), 400)
    for (left, right), causal in (((-1, -1), False), ((-1, 0), True), ((20, 30), False)):
        got = fn(q, k, v, do, 0.5, left, right, None)
        want = attention_bwd_ref(q, k, v, do, 0.5, causal)
        for a, b in zip(got, want):
            assert np.max(np.abs(a - b)) <= tol, (left, right)


def check_padding_is_inert(fn, tol=1e-13):
    """K and V rows at or past a sequence's length change nothing; their dK
    and dV are 0."""
    q, k, v, do = _inputs((2, 2, 8, 3), 500)
    lens = [5, 8]
    got = fn(q, k, v, do, 0.7, 2, -1, lens)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 5:] = 1e3 * _rand(k2[0, :, 5:].shape, 1)
    v2[0, :, 5:] = -7.0
    got2 = fn(q, k2, v2, do, 0.7, 2, -1, lens)
    for a, b in zip(got, got2):
        assert np.max(np.abs(a - b)) <= tol
    assert np.all(got[1][0, :, 5:] == 0.0) and np.all(got[2][0, :, 5:] == 0.0)


MASKED_CHECKS = (check_masked_finite_differences, check_masked_against_torch, check_masked_reduces_to_unmasked,
                 check_padding_is_inert)


@pytest.mark.parametrize("check", MASKED_CHECKS, ids=lambda c: c.__name__)
def test_masked_backward_oracle(check):
    check(attention_bwd_ref_masked)


MASKED_MUTANTS = {
    # The left bound exclusive (one key fewer), and the key lengths ignored.
    "left_bound_off_by_one": lambda q, k, v, do, s, l, r, lens: attention_bwd_ref_masked(
        q, k, v, do, s, l - 1 if l > 0 else l, r, lens),
    "padding_ignored": lambda q, k, v, do, s, l, r, lens: attention_bwd_ref_masked(q, k, v, do, s, l, r, None),
}


@pytest.mark.parametrize("mutant", sorted(MASKED_MUTANTS))
def test_masked_backward_pins_catch_planted_mistakes(mutant):
    caught = 0
    for check in MASKED_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(MASKED_MUTANTS[mutant])
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, f"planted mistake {mutant} went unnoticed"
