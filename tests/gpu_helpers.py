"""Shared helpers for the GPU parity tests: move seeded storage arrays to the
GPU, run the HIP library, and compare against the fp64 oracle."""
import numpy as np

from exact_attention_21_amd import workloads as wl

# Max-abs tolerances on O and LSE per storage dtype.
TOL = {wl.FP16: (2e-3, 1e-3), wl.BF16: (4e-3, 2e-3)}


def to_device(x, dtype, device):
    import torch
    if dtype == wl.FP16:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)


def run_gpu(q, k, v, dtype, scale, causal, device, stream=None):
    """Run fa2_fwd on storage arrays; return (O, LSE) as float64 numpy arrays."""
    import torch
    from exact_attention_21_amd import forward
    tq, tk, tv = (to_device(x, dtype, device) for x in (q, k, v))
    if stream is None:
        o, lse = forward(tq, tk, tv, scale=scale, causal=causal)
    else:
        with torch.cuda.stream(stream):
            o, lse = forward(tq, tk, tv, scale=scale, causal=causal)
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
