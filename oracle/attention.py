"""fp64 CPU oracle for the FlashAttention-2 forward pass and its gradients
(test infrastructure).

This module is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code,
constants or helpers with the HIP library.

Sources (page title, then the part of the page followed):

* "FlashAttention-2 MMA 代码学习" (chuoer47.github.io, leetCUDA study notes),
  step 0: attention is O = softmax(Q K^T * scale) V; step 1: the online (m, l)
  merge over key blocks.
* "第 15 章 FA2 前向：Tiling 与 Online Softmax" (yangyitao.com), §15.1 change 4:
  the statistic kept per row is the log-sum-exp L = m + log l; §15.3 kernel
  skeleton: Q, K, V, O are [B, H, N, d], LSE is [B, H, N] fp32, the scale is
  applied to the scores before the row max, the causal mask hides key j from
  query i when j > i, a row with no visible key gives O = 0 and LSE = +inf;
  §15.4.3: masking happens before the softmax; the note after the §15.3
  skeleton: with sliding-window or padding masks a row can meet only hidden keys
  in its first tiles, which is what the -inf guards (exponent base 0 while the
  row max is -inf, O = 0 and LSE = +inf when l = 0) are there for; the
  chapter's closing summary: the backward recomputes S and P from Q, K and
  the stored statistic instead of reading them (attention_bwd_ref gives the
  gradients that computation reaches).

Precision: every step is fp64.  Inputs are the already-rounded fp16/bf16 values,
upcast exactly by the caller.  ``scale`` is rounded to fp32 first, because that
is the value a caller passing a C ``float`` hands to the GPU library.

Every function here is pinned by tests that do not re-use its own formulas
(tests/test_oracle.py): a pure-Python brute force on tiny shapes, closed forms
derived by hand (tests/golden/closed_forms.json), invariants (key shift,
key/value permutation), special cases (one key, identical keys, scale 0) and a
library routine (torch scaled_dot_product_attention in fp64 on the CPU).  The
backward is pinned in tests/test_oracle_bwd.py by finite differences of the
forward oracle, a hand-derived two-key closed form, special cases,
invariants and torch autograd in fp64.
"""
from __future__ import annotations

import numpy as np

# Rows of one (batch, head) handled per matmul.  This only bounds memory: every
# block computes complete softmax rows, so the result is the plain definition.
_ROW_BLOCK = 256


def _visible_count(i: int, n: int, causal: bool) -> int:
    """Number of keys visible to query row ``i``.

    Causal reading (yangyitao.com ch.15 §15.3 skeleton, mask step): key j is
    visible to query i iff j <= i, with queries and keys indexed from 0 in the
    same sequence (square, top-left aligned).
    """
    return i + 1 if causal else n


def _visible_range(i: int, window_left: int, window_right: int, key_len: int):
    """Keys visible to query row ``i`` under a sliding window and a key length.

    Reading (yangyitao.com ch.15, the note after the §15.3 skeleton, names
    sliding-window and padding masks without fixing their form): key j is
    visible to query i iff j < key_len (keys at or past it are padding),
    j >= i - window_left (no left bound when window_left < 0) and
    j <= i + window_right (no right bound when window_right < 0).  The visible
    keys are the range [lo, hi), empty when hi == lo.  window_left < 0 with
    window_right = 0 is the causal mask.
    """
    lo = 0 if window_left < 0 else max(0, i - window_left)
    hi = key_len if window_right < 0 else min(key_len, i + window_right + 1)
    return lo, max(lo, hi)


def attention_ref(q, k, v, scale: float, causal: bool, rows=None):
    """O = softmax(scale * Q K^T [+ causal mask]) V and LSE, straight from the definition.

    Args:
      q, k, v: float arrays of shape [B, H, N, d]; converted to fp64.
      scale: softmax scale (a C float on the GPU side, so rounded to fp32 here).
      causal: hide key j from query i when j > i.
      rows: optional 1-D integer array of query rows to evaluate (the same rows
        for every batch and head).  ``None`` means all rows.

    Returns:
      (O, LSE): O is fp64 [B, H, R, d] and LSE is fp64 [B, H, R], where R is N or
      len(rows).  LSE is the natural log of the sum over visible keys of
      exp(scale * q.k) (yangyitao.com ch.15 §15.1 change 4 and §15.3 LSE store).
      A row with no visible key gets O = 0 and LSE = +inf (§15.3, final
      normalisation and LSE store); with N >= 1 every row sees at least key 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    b_, h_, n, d = q.shape
    c = float(np.float32(scale))
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim != 1 or (rows.size and (rows.min() < 0 or rows.max() >= n)):
        raise ValueError("rows must be a 1-D array of indices in [0, N)")
    r_ = rows.size
    out = np.zeros((b_, h_, r_, d), dtype=np.float64)
    lse = np.full((b_, h_, r_), np.inf, dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            for r0 in range(0, r_, _ROW_BLOCK):
                idx = rows[r0:r0 + _ROW_BLOCK]
                # Keys any row in this block can see.
                kmax = max(_visible_count(int(i), n, causal) for i in idx)
                # Scores, with the scale applied before the row max.
                s = (q[b, h, idx, :] @ k[b, h, :kmax, :].T) * c
                if causal:
                    j = np.arange(kmax)[None, :]
                    s = np.where(j <= idx[:, None], s, -np.inf)
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])
                l = p.sum(axis=1)
                out[b, h, r0:r0 + idx.size, :] = (p @ v[b, h, :kmax, :]) / l[:, None]
                lse[b, h, r0:r0 + idx.size] = m + np.log(l)
    return out, lse


def _rescale_factor(m_old, m_new):
    """Factor that moves sums taken against the exponent base m_old onto the
    base m_new: exp(m_old - m_new), which multiplies the old O and l.

    "FlashAttention-2 MMA 代码学习" (chuoer47.github.io) step 1 points out that
    the paper's printed update has this factor inverted, and both pages' code
    multiply the old O by exp(m_old - m_new).
    """
    return np.exp(m_old - m_new)


def attention_online_merge(q, k, v, scale: float, causal: bool, block: int, reverse: bool = False,
                           window=None, key_lens=None):
    """The same result through the pages' online (m, l) merge over key blocks, in fp64.

    Follows "FlashAttention-2 MMA 代码学习" (chuoer47.github.io) step 1: for
    every key block, take the block's row max, m = max(m_old, m_block),
    P = exp(S*scale - m), l = exp(m_old - m) * l_old + rowsum(P),
    O = exp(m_old - m) * O_old + P V; and yangyitao.com ch.15 §15.1 change 4 /
    §15.3: divide O by l once after the last block, LSE = m + log l, and while a
    row has seen only masked keys use 0 as the exponent base so that
    exp(-inf - (-inf)) is never formed.

    ``block`` is the number of keys per block; ``reverse`` walks the blocks from
    the last to the first.  The result must not depend on either: the tests use
    that to pin the algebra against ``attention_ref``.  ``window`` = (left,
    right) and ``key_lens`` add the masks of ``attention_ref_masked`` (a
    negative bound is no bound; lengths are clamped to [0, N]); under them a row
    can see only hidden keys in its first blocks, where the -inf guards act.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, h_, n, d = q.shape
    c = float(np.float32(scale))
    out = np.zeros_like(q)
    lse = np.zeros(q.shape[:3], dtype=np.float64)
    starts = list(range(0, n, block))
    if reverse:
        starts = starts[::-1]
    qi = np.arange(n)[:, None]
    for b in range(b_):
        for h in range(h_):
            m_run = np.full(n, -np.inf)
            l_run = np.zeros(n)
            o_run = np.zeros((n, d))
            for k0 in starts:
                k1 = min(n, k0 + block)
                s = (q[b, h] @ k[b, h, k0:k1].T) * c
                kj = np.arange(k0, k1)[None, :]
                hidden = np.zeros((n, k1 - k0), dtype=bool)
                if causal:
                    hidden |= kj > qi
                if window is not None:
                    if window[0] >= 0:
                        hidden |= kj < qi - window[0]
                    if window[1] >= 0:
                        hidden |= kj > qi + window[1]
                if key_lens is not None:
                    hidden |= kj >= min(max(int(key_lens[b]), 0), n)
                s = np.where(hidden, -np.inf, s)
                m_blk = s.max(axis=1)
                m_new = np.maximum(m_run, m_blk)
                base = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = _rescale_factor(m_run, base)
                p = np.exp(s - base[:, None])
                l_run = alpha * l_run + p.sum(axis=1)
                o_run = alpha[:, None] * o_run + p @ v[b, h, k0:k1]
                m_run = m_new
            safe_l = np.where(l_run == 0.0, 1.0, l_run)
            out[b, h] = o_run / safe_l[:, None]
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(l_run == 0.0, np.inf, m_run + np.log(safe_l))
    return out, lse


def attention_ref_masked(q, k, v, scale: float, window_left: int, window_right: int,
                         key_lens=None, rows=None):
    """attention_ref with a sliding window and per-sequence key lengths.

    Key j is visible to query i as ``_visible_range`` states; ``key_lens`` is
    None (no padding) or B integers, each clamped to [0, N].  The softmax runs
    over the visible keys only (masking before the softmax, ch.15 §15.4.3); a
    row with no visible key gets O = 0 and LSE = +inf (§15.3, final
    normalisation and LSE store).  Returns (O, LSE) shaped as attention_ref's.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    b_, h_, n, d = q.shape
    c = float(np.float32(scale))
    lens = [n] * b_ if key_lens is None else [min(max(int(x), 0), n) for x in key_lens]
    if len(lens) != b_:
        raise ValueError("key_lens must hold one length per batch")
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    r_ = rows.size
    out = np.zeros((b_, h_, r_, d), dtype=np.float64)
    lse = np.full((b_, h_, r_), np.inf, dtype=np.float64)
    j = np.arange(n)[None, :]
    for b in range(b_):
        bounds = np.array([_visible_range(int(i), window_left, window_right, lens[b]) for i in rows],
                          dtype=np.int64).reshape(r_, 2)
        for h in range(h_):
            for r0 in range(0, r_, _ROW_BLOCK):
                idx = rows[r0:r0 + _ROW_BLOCK]
                lo = bounds[r0:r0 + idx.size, :1]
                hi = bounds[r0:r0 + idx.size, 1:]
                visible = (j >= lo) & (j < hi)
                s = np.where(visible, (q[b, h, idx, :] @ k[b, h].T) * c, -np.inf)
                seen = visible.any(axis=1)
                m = np.where(seen, s.max(axis=1), 0.0)
                p = np.where(visible, np.exp(s - m[:, None]), 0.0)
                l = p.sum(axis=1)
                safe_l = np.where(seen, l, 1.0)
                out[b, h, r0:r0 + idx.size, :] = np.where(seen[:, None], (p @ v[b, h]) / safe_l[:, None], 0.0)
                lse[b, h, r0:r0 + idx.size] = np.where(seen, m + np.log(safe_l), np.inf)
    return out, lse


def _row_delta(do, o):
    """Delta_i = sum_d dO_id O_id: the row term the softmax backward subtracts."""
    return (do * o).sum(axis=1, keepdims=True)


def _score_grad(p, dp, delta):
    """dS = P * (dP - Delta): the softmax backward, row by row."""
    return p * (dp - delta)


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool):
    """Gradients of sum(dO * O) with O = attention_ref(q, k, v), in fp64.

    The backward of the definition, written out (chain rule through the
    softmax; "第 15 章 FA2 前向：Tiling 与 Online Softmax", closing summary:
    the backward recomputes S and P from the stored statistic and loops over
    key tiles outside, query tiles inside; the arithmetic here is the
    definition those steps reach):

      S = scale * Q K^T (hidden keys -inf),  P = softmax_rows(S) = exp(S - LSE)
      dV = P^T dO
      dP = dO V^T
      Delta_i = sum_j P_ij dP_ij = sum_d dO_id O_id
      dS = P * (dP - Delta)          (elementwise; Delta broadcast over keys)
      dQ = scale * dS K,   dK = scale * dS^T Q

    Returns (dQ, dK, dV), fp64 [B, H, N, d].  ``scale`` is rounded to fp32
    first, as in the forward.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if q.ndim != 4 or any(x.shape != q.shape for x in (k, v, do)):
        raise ValueError("q, k, v, do must share one [B, H, N, d] shape")
    b_, h_, n, d = q.shape
    c = float(np.float32(scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    for b in range(b_):
        for h in range(h_):
            s = (q[b, h] @ k[b, h].T) * c
            if causal:
                s = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ v[b, h]
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = _score_grad(p, dp, _row_delta(do[b, h], o))
            dq[b, h] = c * (ds @ k[b, h])
            dk[b, h] = c * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_bwd_ref_masked(q, k, v, do, scale: float, window_left: int, window_right: int, key_lens=None):
    """attention_bwd_ref for attention_ref_masked's visibility: the same chain
    rule with P the softmax over each row's visible keys (``_visible_range``;
    key lengths clamped to [0, N]).  A row with no visible key has P = 0 and
    O = 0, so its dQ is 0 and it adds nothing to dK or dV; keys at or past a
    sequence's length get dK = dV = 0.  Returns (dQ, dK, dV), fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if q.ndim != 4 or any(x.shape != q.shape for x in (k, v, do)):
        raise ValueError("q, k, v, do must share one [B, H, N, d] shape")
    b_, h_, n, d = q.shape
    c = float(np.float32(scale))
    lens = [n] * b_ if key_lens is None else [min(max(int(x), 0), n) for x in key_lens]
    if len(lens) != b_:
        raise ValueError("key_lens must hold one length per batch")
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    j = np.arange(n)[None, :]
    for b in range(b_):
        bounds = np.array([_visible_range(i, window_left, window_right, lens[b]) for i in range(n)],
                          dtype=np.int64).reshape(n, 2)
        visible = (j >= bounds[:, :1]) & (j < bounds[:, 1:])
        seen = visible.any(axis=1)
        for h in range(h_):
            s = np.where(visible, (q[b, h] @ k[b, h].T) * c, -np.inf)
            m = np.where(seen, s.max(axis=1), 0.0)
            e = np.where(visible, np.exp(s - m[:, None]), 0.0)
            p = e / np.where(seen, e.sum(axis=1), 1.0)[:, None]
            o = p @ v[b, h]
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = _score_grad(p, dp, _row_delta(do[b, h], o))
            dq[b, h] = c * (ds @ k[b, h])
            dk[b, h] = c * (ds.T @ q[b, h])
    return dq, dk, dv
