"""Helpers of the backward parity tests: seeded inputs, the oracle's
gradients, and an element-wise bound on the error that the kernels' rounding
can make.

Error model (first order, every term taken with the worst sign).  The
kernels compute S, dP, Delta and the accumulators in fp32, round P (for dV)
and dS (for dQ, dK) once to the input dtype, and round each gradient once at
the end.  With u the unit roundoff of that dtype, ``sub`` half its subnormal
spacing, and the exact values of the definition written P, dP, Delta, dS:

* P as computed (fp32, before rounding) has a relative error rel_P of at most
  2^-22 (exp2 and the argument's rounding) + |c| (d/16 + 1) 2^-24 (|Q||K|^T)
  (the fp32 score) + 2^-23 |LSE| + |LSE_in - LSE| (the statistic as given);
* dP has an absolute error of at most (d/16 + 1) 2^-24 (|dO||V|^T), and the
  kernels' Delta differs from the exact one by |sum_d dO (O_in - O)| (O as
  given, rounded) plus d 2^-24 sum_d |dO O_in|;
* so  E_P  = (u + rel_P) P + sub   bounds the error of the rounded P, and
       E_dS = (u + rel_P) |dS| + P (err dP + err Delta) + sub  that of dS;
* the products add the fp32 rounding of their running sums, at most
  (N/16 + 2) 2^-24 times the sum of the magnitudes of their terms.

    |dV - dV_ref| <= E_P^T |dO| + acc + half an ulp
    |dQ - dQ_ref| <= |c| (E_dS |K|) + acc + half an ulp
    |dK - dK_ref| <= |c| (E_dS^T |Q|) + acc + half an ulp

(half an ulp of the output dtype at |ref| plus the rest of the bound, the
largest value the unrounded result can take).

Hidden (causal) pairs have P = dS = 0 in both the kernels and the oracle.
"""
import numpy as np

from exact_attention_21_amd import workloads as wl

_U = {wl.FP16: 2.0 ** -11, wl.BF16: 2.0 ** -8}
_SUB = {wl.FP16: 2.0 ** -25, wl.BF16: 0.0}
_BITS = {wl.FP16: (11, -14), wl.BF16: (8, -126)}


def half_ulp(x, dtype):
    bits, emin = _BITS[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.where(ax > 0, np.floor(np.log2(np.where(ax > 0, ax, 1.0))), emin)
    return np.ldexp(1.0, (np.maximum(e, emin) - bits).astype(np.int64))


def make_case(B, H, N, d, dtype, seed, causal=False, scale=None, sigma=(1.0, 1.0, 1.0, 1.0)):
    """Seeded storage arrays (q, k, v, do) of one backward case and its
    Workload (the draw recipe of the workloads module)."""
    w = wl.Workload(f"bwd_b{B}h{H}n{N}d{d}_{dtype}", B, H, N, d, dtype, causal,
                    q_dist=("normal", sigma[0]), k_dist=("normal", sigma[1]), v_dist=("normal", sigma[2]),
                    scale=scale)
    q, k, v = wl.make_inputs(w, seed=seed)
    do = wl.make_grad_output(w, seed=seed, sigma=sigma[3])
    return w, q, k, v, do


def forward_inputs(q64, k64, v64, scale, causal, dtype, mask=None):
    """O and LSE for the backward as a caller would pass them, from the oracle:
    O rounded to the storage dtype, LSE to float32.  ``mask`` = (window_left,
    window_right, key_lens) selects the masked forward."""
    from oracle import attention_ref, attention_ref_masked
    if mask is None:
        o, lse = attention_ref(q64, k64, v64, scale, causal)
    else:
        o, lse = attention_ref_masked(q64, k64, v64, scale, *mask)
    return wl.round_to_storage(o, dtype), lse.astype(np.float32)


def visibility(n, causal=False, mask=None, b=0):
    """[N, N] boolean: key j visible to query i (the definitions of the two
    forward entry points, written out here)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    if mask is None:
        return (j <= i) if causal else np.ones((n, n), dtype=bool)
    left, right, lens = mask
    vis = j < (n if lens is None else min(max(int(lens[b]), 0), n))
    if 0 <= left < n:
        vis = vis & (j >= i - left)
    if 0 <= right < n:
        vis = vis & (j <= i + right)
    return vis


def grad_bounds(q64, k64, v64, do64, o_in64, lse_in64, scale, causal, dtype, heads=None, mask=None):
    """The oracle's gradients and the error bound above, for the (b, h) pairs
    in ``heads`` (all by default); ``mask`` as for forward_inputs.  Returns
    dicts name -> [n_pairs, N, d]."""
    from oracle import attention_bwd_ref, attention_bwd_ref_masked, attention_ref, attention_ref_masked
    B, H, N, d = q64.shape
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    c = float(np.float32(scale))
    u, sub = _U[dtype], _SUB[dtype]
    acc = (N / 16 + 2) * 2.0 ** -24
    refs = {"dq": [], "dk": [], "dv": []}
    bounds = {"dq": [], "dk": [], "dv": []}
    for b, h in pairs:
        sl = (slice(b, b + 1), slice(h, h + 1))
        q, k, v, do = (x[sl] for x in (q64, k64, v64, do64))
        if mask is None:
            dq_r, dk_r, dv_r = attention_bwd_ref(q, k, v, do, scale, causal)
            o_r, lse_r = attention_ref(q, k, v, scale, causal)
        else:
            m = (mask[0], mask[1], None if mask[2] is None else [mask[2][b]])
            dq_r, dk_r, dv_r = attention_bwd_ref_masked(q, k, v, do, scale, *m)
            o_r, lse_r = attention_ref_masked(q, k, v, scale, *m)
        q, k, v, do, o_r, lse_r = q[0, 0], k[0, 0], v[0, 0], do[0, 0], o_r[0, 0], lse_r[0, 0]
        o_in, lse_in = o_in64[b, h], lse_in64[b, h]
        vis = visibility(N, causal, mask, b).astype(np.float64)
        seen = np.isfinite(lse_r)
        # Rows that see no key have P = 0 (their LSE is +inf on both sides).
        lse_r = np.where(seen, lse_r, 0.0)
        lse_in = np.where(seen, lse_in, 0.0)
        vis = vis * seen[:, None]
        p = np.exp(np.where(vis > 0, c * (q @ k.T) - lse_r[:, None], -np.inf))
        dp = do @ v.T
        delta = np.sum(do * o_r, axis=1)
        ds = p * (dp - delta[:, None])
        rel_p = (2.0 ** -22 + abs(c) * (d / 16 + 1) * 2.0 ** -24 * (np.abs(q) @ np.abs(k).T)
                 + 2.0 ** -23 * np.abs(lse_r)[:, None] + np.abs(lse_in - lse_r)[:, None])
        err_dp = (d / 16 + 1) * 2.0 ** -24 * (np.abs(do) @ np.abs(v).T)
        err_delta = np.abs(np.sum(do * (o_in - o_r), axis=1)) + d * 2.0 ** -24 * np.sum(np.abs(do * o_in), axis=1)
        e_p = vis * ((u + rel_p) * p + sub)
        e_ds = vis * ((u + rel_p) * np.abs(ds) + p * (err_dp + err_delta[:, None]) + sub)
        pre = {"dv": e_p.T @ np.abs(do) + acc * (p.T @ np.abs(do)),
               "dq": abs(c) * (e_ds @ np.abs(k) + acc * (np.abs(ds) @ np.abs(k))),
               "dk": abs(c) * (e_ds.T @ np.abs(q) + acc * (np.abs(ds).T @ np.abs(q)))}
        for name, r in (("dq", dq_r[0, 0]), ("dk", dk_r[0, 0]), ("dv", dv_r[0, 0])):
            # The final rounding: half an ulp at the largest value the
            # unrounded result can take.
            refs[name].append(r)
            bounds[name].append(pre[name] + half_ulp(np.abs(r) + pre[name], dtype))
    return ({n: np.stack(x) for n, x in refs.items()}, {n: np.stack(x) for n, x in bounds.items()})


def assert_grads_within(got, refs, bounds, label=""):
    """Every element of dQ, dK, dV within its bound; prints the largest error,
    its size against the largest reference value, and the largest share of
    the bound an element needed."""
    for name in ("dq", "dk", "dv"):
        g, r, bd = got[name], refs[name], bounds[name]
        assert np.all(np.isfinite(g)), f"{label} {name}: non-finite value"
        err = np.abs(g - r)
        share = float(np.max(err / bd))
        print(f"  {label} {name}: max err {float(err.max()):.3e} (max|ref| {float(np.abs(r).max()):.3e}), "
              f"largest share of the bound needed {share:.3f}", flush=True)
        worst = np.unravel_index(int(np.argmax(err - bd)), err.shape)
        assert share <= 1.0, (f"{label} {name}: error {float(err[worst]):.3e} above its bound "
                              f"{float(bd[worst]):.3e} at {worst}")


def simulate_kernel_rounding(q64, k64, v64, do64, o_in64, lse_in64, scale, causal, dtype, mask=None):
    """The kernels' rounding steps replayed in fp64 on the CPU (P and dS
    rounded to the storage dtype, Delta from the O given, outputs rounded):
    a check that the bound above covers what it claims to (it is not the
    kernels' code and takes no part in the parity tests' expected values)."""
    B, H, N, d = q64.shape
    c = float(np.float32(scale))
    out = {"dq": np.zeros_like(q64), "dk": np.zeros_like(q64), "dv": np.zeros_like(q64)}
    rnd = (lambda x: wl.to_float64(wl.round_to_storage(x, dtype), dtype))
    for b in range(B):
        for h in range(H):
            q, k, v, do = q64[b, h], k64[b, h], v64[b, h], do64[b, h]
            vis = visibility(N, causal, mask, b) & np.isfinite(lse_in64[b, h])[:, None]
            lse = np.where(np.isfinite(lse_in64[b, h]), lse_in64[b, h], 0.0)
            p = np.exp(np.where(vis, c * (q @ k.T) - lse[:, None], -np.inf))
            delta = np.sum(do * o_in64[b, h], axis=1)
            ds = p * (do @ v.T - delta[:, None])
            out["dv"][b, h] = rnd(rnd(p).T @ do)
            out["dq"][b, h] = rnd(c * (rnd(ds) @ k))
            out["dk"][b, h] = rnd(c * (rnd(ds).T @ q))
    return out


def to_np(t):
    """A GPU fp16/bf16 tensor as float64 numpy."""
    return t.float().cpu().numpy().astype(np.float64)
