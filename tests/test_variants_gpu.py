"""The design-ablation builds against the fp64 oracle.

Each ablation build (exact_attention_21_amd/ablation.py: the library with one
design switch flipped, compiled for d = 64 and 128) must compute the same
attention as the shipped build does: every element of a multi-tile shape with
a ragged tail is compared with the oracle, with the stated tolerances, through
each build's own C ABI.  The builds are made by `ablation.py --build`; a build
that is not there is skipped with that reason.
"""
import numpy as np
import pytest

from exact_attention_21_amd import ablation
from exact_attention_21_amd import workloads as wl
from oracle import attention_ref, attention_ref_masked
from tests.gpu_helpers import assert_close, assert_close_masked, to_device

pytestmark = pytest.mark.gpu

BUILDS = [name for name, defines, _ in ablation.VARIANTS if defines is not None]
# (d, dtype, causal, window, key_lens); B = 2, H = 2, N = 700.
CASES = [
    (64, wl.FP16, False, None, None),
    (64, wl.BF16, True, None, None),
    (64, wl.FP16, False, (300, 0), None),
    (128, wl.BF16, True, None, None),
    (128, wl.FP16, False, None, [700, 333]),
    (128, wl.BF16, False, (100, 37), None),
]


def _case_id(c):
    d, dt, causal, window, lens = c
    return f"d{d}-{dt}-" + ("causal" if causal else "window" if window else "lens" if lens else "full")


_LIBS = {}


def _library(name):
    import os
    from exact_attention_21_amd import _binding as bd
    path = ablation.lib_path(name)
    if not os.path.exists(path):
        pytest.skip(f"{path} is not built (python exact_attention_21_amd/ablation.py --build)")
    if name not in _LIBS:
        _LIBS[name] = bd.open_library(path)
    return _LIBS[name]


@pytest.mark.parametrize("case", CASES, ids=[_case_id(c) for c in CASES])
@pytest.mark.parametrize("build", BUILDS)
def test_ablation_build_matches_oracle(gpu_device, build, case):
    import torch
    from exact_attention_21_amd import _binding as bd
    lib = _library(build)
    d, dtype, causal, window, lens = case
    B, H, N = 2, 2, 700
    w = wl.Workload("v", B, H, N, d, dtype, causal)
    q, k, v = wl.make_inputs(w, seed=d + 3)
    tq, tk, tv = (to_device(x, dtype, gpu_device) for x in (q, k, v))
    o = torch.empty_like(tq)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=gpu_device)
    dt = bd.FA2_DTYPE_FP16 if dtype == wl.FP16 else bd.FA2_DTYPE_BF16
    stream = torch.cuda.current_stream(gpu_device).cuda_stream
    scale = w.softmax_scale()
    if window is None and lens is None:
        st = lib.fa2_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, scale, int(causal), dt, stream)
    else:
        left, right = window if window is not None else (-1, -1)
        tl = torch.tensor(lens, dtype=torch.int32, device=gpu_device) if lens is not None else None
        st = lib.fa2_fwd_masked(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, N, d, scale, left, right, tl.data_ptr() if tl is not None else None, dt,
                                stream)
    assert st == bd.FA2_OK, f"{build}: status {st}"
    torch.cuda.synchronize(gpu_device)
    o64 = o.float().cpu().numpy().astype(np.float64)
    l64 = lse.cpu().numpy().astype(np.float64)
    f64 = [wl.to_float64(x, dtype) for x in (q, k, v)]
    label = f"{build} {_case_id(case)}"
    if window is None and lens is None:
        o_ref, lse_ref = attention_ref(*f64, scale, causal)
        assert_close(o64, l64, o_ref, lse_ref, dtype, label)
    else:
        o_ref, lse_ref = attention_ref_masked(*f64, scale, left, right, lens)
        assert_close_masked(o64, l64, o_ref, lse_ref, dtype, label)
