"""Shared helpers for the GPU parity tests: move seeded storage arrays to the
GPU, run the HIP library, and compare against the fp64 oracle."""
import math

import numpy as np

from exact_attention_21_amd import workloads as wl

# Max-abs tolerances on O and LSE per storage dtype.
TOL = {wl.FP16: (2e-3, 1e-3), wl.BF16: (4e-3, 2e-3)}


def to_device(x, dtype, device):
    import torch
    if dtype == wl.FP16:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)


def run_gpu(q, k, v, dtype, scale, causal, device, stream=None, window=None, key_lens=None):
    """Run fa2_fwd (fa2_fwd_masked when a window or key lengths are given) on
    storage arrays; return (O, LSE) as float64 numpy arrays."""
    import torch
    from exact_attention_21_amd import forward
    tq, tk, tv = (to_device(x, dtype, device) for x in (q, k, v))
    kw = dict(scale=scale, causal=causal)
    if window is not None:
        kw["window"] = window
    if key_lens is not None:
        kw["key_lens"] = torch.tensor(key_lens, dtype=torch.int32, device=device)
    if stream is None:
        o, lse = forward(tq, tk, tv, **kw)
    else:
        with torch.cuda.stream(stream):
            o, lse = forward(tq, tk, tv, **kw)
    torch.cuda.synchronize(device)
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


# Significand bits (with the implicit one) and smallest normal exponent.
_FORMAT = {wl.FP16: (11, -14), wl.BF16: (8, -126)}


def half_ulp(x, dtype):
    """Half a unit in the last place of the storage dtype at |x|: the largest
    error of rounding the exact value to that dtype."""
    bits, emin = _FORMAT[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.where(ax > 0, np.floor(np.log2(np.where(ax > 0, ax, 1.0))), emin)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - bits).astype(np.int64))


def max_errors(o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    """(raw max |dO|, max |dO| beyond half an output ulp, max |dLSE|)."""
    assert np.all(np.isfinite(o_gpu)), "non-finite value in O"
    assert np.all(np.isfinite(lse_gpu)), "non-finite value in LSE"
    d = np.abs(o_gpu - o_ref)
    return (float(np.max(d)), float(np.max(d - half_ulp(o_ref, dtype))),
            float(np.max(np.abs(lse_gpu - lse_ref))))


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """O: the error beyond the unavoidable rounding of the exact result to the
    output dtype must be within the tolerance; for fp16 the raw max-abs error
    must be too (bf16 cannot meet it once |O| >= 1, where half an ulp is
    already >= 2^-8).  LSE is fp32: raw max-abs error."""
    raw, net, el = max_errors(o_gpu, lse_gpu, o_ref, lse_ref, dtype)
    to, tl = TOL[dtype]
    print(f"  {label}: max|dO| = {raw:.3e}, beyond half-ulp = {net:.3e} (tol {to:.0e}), "
          f"max|dLSE| = {el:.3e} (tol {tl:.0e})", flush=True)
    assert net <= to, f"{label}: O error beyond output rounding {net:.3e} > {to}"
    if dtype == wl.FP16:
        assert raw <= to, f"{label}: O error {raw:.3e} > {to}"
    assert el <= tl, f"{label}: LSE error {el:.3e} > {tl}"


def spiky_inputs(B, H, N, d, dtype, seed, factor, where):
    """N(0,1) inputs whose keys at the given relative positions are scaled by
    ``factor``: the running row max jumps in the middle of the key sequence,
    so the online softmax must move its exponent base (and rescale O and l)
    after many tiles have already been accumulated."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    for frac in where:
        j = int(frac * N)
        k[:, :, j:j + 3] *= factor
    return tuple(wl.round_to_storage(x, dtype) for x in (q, k, v))


# Unit roundoff of rounding a probability to the storage dtype (relative,
# normal range) and half the fp16 subnormal spacing (absolute).
_U_P = {wl.FP16: 2.0 ** -11, wl.BF16: 2.0 ** -8}
_FP16_SUB_HALF = 2.0 ** -25


def p_rounding_bound(q, k, v, o_ref, dtype, scale, causal, mask=None):
    """First-order bound, per element of O, of rounding P once to the input
    dtype before P.V (the pages round P to the input type and accumulate O in
    fp32; O is normalised by the sum of the rounded P).

    With p~_j = p_j (1 + e_j), |e_j| <= u and weights w_j = p_j / sum p:
      O~ - O = sum_j w_j e_j (v_j - O) / (1 + sum_j w_j e_j),
    so |O~ - O| <= u / (1 - u) * sum_j w_j |v_j - O| <= u / (1 - u) * sigma,
    where sigma^2 = E_w[v^2] - O^2 is the spread of V under the attention
    weights (one more oracle evaluation, with V squared).  For fp16, P values
    below 2^-14 are subnormal: each is off by at most 2^-25 absolutely, and the
    row sum is at least about 1 (the largest P is at least 1 against a base at
    or below the row max), which adds n_visible * 2^-25 * max_j |v_j - O|.

    On N(0,1) inputs the error terms of many keys average out and the stated
    tolerance holds on its own; inputs built to put the weight on a few keys
    with different V rows reach this bound.
    """
    from oracle import attention_ref, attention_ref_masked
    n = q.shape[2]
    v64 = wl.to_float64(v, dtype)
    q64, k64 = wl.to_float64(q, dtype), wl.to_float64(k, dtype)
    if mask is None:
        ev2, _ = attention_ref(q64, k64, v64 * v64, scale, causal)
    else:  # (window_left, window_right, key_lens) of attention_ref_masked
        ev2, _ = attention_ref_masked(q64, k64, v64 * v64, scale, *mask)
    sigma = np.sqrt(np.maximum(ev2 - o_ref * o_ref, 0.0))
    u = _U_P[dtype]
    bound = u / (1.0 - u) * sigma
    if dtype == wl.FP16:
        # (n visible keys at most: the whole row length bounds every mask)
        n_vis = (np.arange(n) + 1.0) if causal else np.full(n, float(n))
        vmax = np.abs(v64).max(axis=2, keepdims=True)  # [B, H, 1, d]
        bound = bound + n_vis[None, None, :, None] * _FP16_SUB_HALF * (vmax + np.abs(o_ref))
    return bound


def assert_close_stress(o_gpu, lse_gpu, o_ref, lse_ref, p_bound, dtype, label=""):
    """assert_close for inputs that concentrate the attention on a few keys:
    the O tolerance is widened element by element by the P-rounding bound
    (p_rounding_bound); the LSE check is unchanged (the kernel sums the
    unrounded probabilities for it)."""
    assert np.all(np.isfinite(o_gpu)), "non-finite value in O"
    assert np.all(np.isfinite(lse_gpu)), "non-finite value in LSE"
    to, tl = TOL[dtype]
    d = np.abs(o_gpu - o_ref)
    net = float(np.max(d - half_ulp(o_ref, dtype) - p_bound))
    raw = float(np.max(d - p_bound))
    el = float(np.max(np.abs(lse_gpu - lse_ref)))
    share = bound_share(o_gpu, o_ref, p_bound, dtype)
    print(f"  {label}: max|dO| = {float(d.max()):.3e}, beyond half-ulp and P-rounding bound = {net:.3e} "
          f"(tol {to:.0e}; bound max {float(p_bound.max()):.2e}, largest share of it needed {share:.2f}), "
          f"max|dLSE| = {el:.3e} (tol {tl:.0e})", flush=True)
    assert net <= to, f"{label}: O error beyond output rounding and P rounding {net:.3e} > {to}"
    if dtype == wl.FP16:
        assert raw <= to, f"{label}: O error beyond P rounding {raw:.3e} > {to}"
    assert el <= tl, f"{label}: LSE error {el:.3e} > {tl}"


def assert_close_masked(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """assert_close for masked attention: a row the oracle marks fully hidden
    (LSE = +inf) must come back as O = 0 and LSE = +inf exactly; the other
    rows are held to the usual tolerances."""
    hidden = np.isposinf(lse_ref)
    assert np.array_equal(np.isposinf(lse_gpu), hidden), f"{label}: fully hidden rows differ"
    assert np.all(o_gpu[hidden] == 0.0), f"{label}: O of a fully hidden row is not 0"
    seen = ~hidden
    if seen.any():
        assert_close(o_gpu[seen], lse_gpu[seen], o_ref[seen], lse_ref[seen], dtype, label)
    print(f"  {label}: {int(hidden.sum())} fully hidden rows", flush=True)


def jump_inputs(B, H, N, d, dtype, seed, scale, jumps, v_spike=None):
    """N(0,1) inputs with a few keys whose scores stand a fixed number of
    base-2 units above zero for every query.

    Every query gets q[0] = 4; key j = int(frac * N) of ``jumps`` = [(frac,
    units), ...] becomes units / (4 * scale * log2(e)) in dimension 0 and 0
    elsewhere, so its score is ``units`` (base 2) for every row, far above the
    N(0,1) scores (a few units).  ``v_spike`` (if given) replaces those keys'
    value rows by +-v_spike with random signs.  Returns the storage arrays and
    the key indices."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    q[..., 0] = 4.0
    c2 = float(np.float32(scale)) * math.log2(math.e)
    idx = []
    for frac, units in jumps:
        j = min(N - 1, int(frac * N))
        k[:, :, j, :] = 0.0
        k[:, :, j, 0] = units / (4.0 * c2)
        if v_spike is not None:
            v[:, :, j, :] = v_spike * rng.choice([-1.0, 1.0], size=(B, H, d))
        idx.append(j)
    return tuple(wl.round_to_storage(x, dtype) for x in (q, k, v)) + (idx,)


def jump_above_rest(q, k, dtype, scale, spikes, visible):
    """Per row: the largest base-2 score among the spike keys it sees minus the
    largest score among the other keys it sees (NaN for rows that see no spike
    or nothing else).  ``visible`` is a [B, N, N] (or [N, N]) boolean mask."""
    qf, kf = wl.to_float64(q, dtype), wl.to_float64(k, dtype)
    s = (qf @ np.swapaxes(kf, -1, -2)) * float(np.float32(scale)) * math.log2(math.e)
    vis = np.broadcast_to(visible if visible.ndim == 3 else visible[None], (s.shape[0],) + s.shape[2:])[:, None]
    is_spike = np.zeros(s.shape[-1], dtype=bool)
    is_spike[spikes] = True
    top = np.where(vis & is_spike, s, -np.inf).max(axis=-1)
    rest = np.where(vis & ~is_spike, s, -np.inf).max(axis=-1)
    with np.errstate(invalid="ignore"):
        out = top - rest
    return np.where(np.isfinite(out), out, np.nan)


def visible_matrix(N, causal=False, window=None, key_lens=None, B=1):
    """[B, N, N] mask of the keys each query sees (the masks' definition, for
    building test inputs; the oracle applies its own)."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if causal:
        vis &= j <= i
    if window is not None:
        if window[0] >= 0:
            vis &= j >= i - window[0]
        if window[1] >= 0:
            vis &= j <= i + window[1]
    out = np.broadcast_to(vis, (B, N, N)).copy()
    if key_lens is not None:
        for b, n_b in enumerate(key_lens):
            out[b] &= j < min(max(int(n_b), 0), N)
    return out


def bound_share(o_gpu, o_ref, p_bound, dtype):
    """Largest share of the P-rounding bound an element needed: the error
    beyond half an output ulp and the plain tolerance, over the bound (0 when
    the plain tolerance covers every element)."""
    to = TOL[dtype][0]
    extra = np.abs(o_gpu - o_ref) - half_ulp(o_ref, dtype) - to
    with np.errstate(divide="ignore", invalid="ignore"):
        share = np.where(extra > 0, extra / p_bound, 0.0)
    return float(np.max(share)) if share.size else 0.0


def oracle_all_rows(q64, k64, v64, scale, causal, chunk=2048):
    """attention_ref over every row, evaluated as independent (batch, head,
    row range) calls on a thread pool (BLAS held to one thread per call), so
    that the full-size workloads finish in seconds; the pieces are the
    oracle's own rows= evaluations, put back in place."""
    import os
    import time
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention_ref
    B, H, N, d = q64.shape
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    tasks = [(b, h, r0) for b in range(B) for h in range(H) for r0 in range(0, N, chunk)]

    def one(t):
        b, h, r0 = t
        rows = np.arange(r0, min(N, r0 + chunk))
        ob, lb = attention_ref(q64[b:b + 1, h:h + 1], k64[b:b + 1, h:h + 1], v64[b:b + 1, h:h + 1],
                               scale, causal, rows=rows)
        o[b, h, rows] = ob[0, 0]
        lse[b, h, rows] = lb[0, 0]

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for _ in ex.map(one, tasks):
            pass
    print(f"  oracle: {len(tasks)} pieces on {workers} threads, {time.perf_counter() - t0:.1f} s", flush=True)
    return o, lse
