"""PyTorch entry points: allocate outputs with torch and call the C ABI.

torch supplies device memory and the current stream; the computation runs in
the HIP kernels behind ``fa2_fwd``, ``fa2_fwd_masked`` and ``fa2_bwd``.
"""
from __future__ import annotations

import math

import torch

from ._binding import (FA2_DTYPE_BF16, FA2_DTYPE_FP16, FA2_OK, Fa2Error, fa2_bwd, fa2_bwd_masked, fa2_fwd,
                       fa2_fwd_masked)

_DTYPES = {torch.float16: FA2_DTYPE_FP16, torch.bfloat16: FA2_DTYPE_BF16}


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
            causal: bool = False, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, window: tuple[int, int] | None = None,
            key_lens: torch.Tensor | None = None):
    """Attention forward on [B, H, N, d] fp16/bf16 CUDA(HIP) tensors.

    Returns (O, LSE): O has q's shape and dtype, LSE is float32 [B, H, N].
    ``scale`` defaults to 1/sqrt(d).  ``out``/``lse`` may be given to reuse
    buffers.  The kernel is enqueued on torch's current stream.

    ``window`` = (left, right) keeps key j for query i only when
    i - left <= j <= i + right (a negative bound is none; ``causal`` sets
    right = 0), and ``key_lens`` (int32 [B] on the same GPU) hides the keys at
    or past each sequence's length; either one calls ``fa2_fwd_masked``.
    """
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must all be float16 or all bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one GPU")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    masked = window is not None or key_lens is not None
    if masked:
        left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        if causal:
            right = 0 if right < 0 else min(right, 0)
        lens_ptr = None
        if key_lens is not None:
            if key_lens.shape != (B,) or key_lens.dtype != torch.int32 or not key_lens.is_contiguous() \
                    or key_lens.device != q.device:
                raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
            lens_ptr = key_lens.data_ptr()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if masked:
            st = fa2_fwd_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                B, H, N, d, float(scale), left, right, lens_ptr, _DTYPES[q.dtype], stream)
        else:
            st = fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                         B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype], stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fwd_masked" if masked else "fa2_fwd")
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             do: torch.Tensor, scale: float | None = None, causal: bool = False,
             workspace: torch.Tensor | None = None, out: tuple | None = None,
             window: tuple[int, int] | None = None, key_lens: torch.Tensor | None = None):
    """Gradients (dQ, dK, dV) of the attention of ``forward`` given dO.

    q, k, v, o, do: [B, H, N, d] fp16/bf16 tensors of one dtype on one GPU
    (d = 32, 64, 96, 128 or 256); o and lse are forward's outputs for the same q, k, v,
    scale and causal.  ``workspace`` (float32, 2*B*H*N elements) and ``out``
    (a (dq, dk, dv) tuple of tensors like q) may be given to reuse buffers.
    ``window`` and ``key_lens`` are those of ``forward`` (through
    ``fa2_bwd_masked``; o and lse must then come from the masked forward).
    The two kernels are enqueued on torch's current stream.
    """
    ts = (q, k, v, o, do)
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o, do must share one [B, H, N, d] shape")
    if q.dtype not in _DTYPES or any(t.dtype != q.dtype for t in ts):
        raise TypeError("q, k, v, o, do must all be float16 or all bfloat16")
    if not all(t.is_cuda and t.device == q.device for t in ts + (lse,)):
        raise ValueError("all tensors must be on one GPU")
    if not all(t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("all tensors must be contiguous")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device)
    if workspace.numel() < 2 * B * H * N or workspace.dtype != torch.float32 or not workspace.is_contiguous() \
            or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous float32 tensor of 2*B*H*N elements on q's device")
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = out
    if any(t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device
           for t in out):
        raise ValueError("out must be three contiguous tensors like q")
    masked = window is not None or key_lens is not None
    if masked:
        left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
        if causal:
            right = 0 if right < 0 else min(right, 0)
        lens_ptr = None
        if key_lens is not None:
            if key_lens.shape != (B,) or key_lens.dtype != torch.int32 or not key_lens.is_contiguous() \
                    or key_lens.device != q.device:
                raise ValueError("key_lens must be a contiguous int32 [B] tensor on q's device")
            lens_ptr = key_lens.data_ptr()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr())
        if masked:
            st = fa2_bwd_masked(*ptrs, B, H, N, d, float(scale), left, right, lens_ptr, _DTYPES[q.dtype], stream)
        else:
            st = fa2_bwd(*ptrs, B, H, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype], stream)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_bwd_masked" if masked else "fa2_bwd")
    return dq, dk, dv
