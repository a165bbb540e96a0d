"""FlashAttention-2 forward and backward for AMD MI355X (gfx950): HIP kernels behind a C ABI.

* ``fa2_fwd`` / ``fa2_fwd_masked`` / ``fa2_bwd`` / ``fa2_bwd_masked`` / ``fa2_bwd_noalloc`` /
  ``fa2_status_string`` / ``fa2_launch_info``: the C functions of include/fa2.h, called through ctypes
  with integer pointers.
* ``forward(q, k, v, scale=None, causal=False, window=None, key_lens=None)``:
  torch tensors in, (O, LSE) out.
* ``backward(q, k, v, o, lse, do, scale=None, causal=False, window=None, key_lens=None)``:
  (dQ, dK, dV).
* ``workloads``: seeded synthetic inputs (no attention arithmetic).

The shared library is loaded on first use; importing the package needs no GPU.
"""
from ._binding import (EXPORTED, FA2_DTYPE_BF16, FA2_DTYPE_FP16, FA2_OK, Fa2Error,  # noqa: F401
                       fa2_bwd, fa2_bwd_masked, fa2_bwd_noalloc, fa2_fwd, fa2_fwd_masked, fa2_launch_info,
                       fa2_status_string, library)


def forward(*args, **kwargs):
    from .torch_api import forward as _forward
    return _forward(*args, **kwargs)


def backward(*args, **kwargs):
    from .torch_api import backward as _backward
    return _backward(*args, **kwargs)
