"""GPU parity of fa2_bwd against the fp64 oracle's gradients
(attention_bwd_ref), element by element, within the rounding bound of
tests/bwd_helpers.py.

O and LSE passed to the kernels come from the oracle's forward (rounded as a
caller's would be), except in the chained test, which feeds the GPU
forward's own O and LSE.  The full-size shapes are checked on sampled heads
(every element of those heads); heads are independent."""
import numpy as np
import pytest
import torch

from exact_attention_21_amd import backward, forward
from exact_attention_21_amd import workloads as wl
from tests import bwd_helpers as bh
from tests.gpu_helpers import to_device

pytestmark = pytest.mark.gpu


def _run(case_args, device, heads=None, seed=3, chained=False, stream=None, mask=None):
    """One backward case; ``mask`` = (window_left, window_right, key_lens)
    runs fa2_bwd_masked (the forward inputs from the masked oracle), with the
    GPU's K and V rows at or past each key length set to NaN (the kernels
    must never read them)."""
    B, H, N, d, dtype, causal, scale, sigma = case_args
    w, q, k, v, do = bh.make_case(B, H, N, d, dtype, seed, causal=causal, scale=scale, sigma=sigma)
    sc = w.softmax_scale()
    print(f"case {w.name} causal={causal} scale={sc} sigma={sigma} chained={chained} mask={mask}", flush=True)
    q64, k64, v64, do64 = (wl.to_float64(x, dtype) for x in (q, k, v, do))
    tq, tk, tv, tdo = (to_device(x, dtype, device) for x in (q, k, v, do))
    kw = {}
    if mask is not None:
        kw["window"] = (mask[0], mask[1])
        if mask[2] is not None:
            kw["key_lens"] = torch.tensor(mask[2], dtype=torch.int32, device=device)
            if not chained:
                for b, n_b in enumerate(mask[2]):
                    tk[b, :, max(n_b, 0):] = float("nan")
                    tv[b, :, max(n_b, 0):] = float("nan")
    if chained:
        o_t, lse_t = forward(tq, tk, tv, scale=sc, causal=causal, **kw)
    else:
        o_in, lse_in = bh.forward_inputs(q64, k64, v64, sc, causal, dtype, mask=mask)
        o_t = to_device(o_in, dtype, device)
        lse_t = torch.from_numpy(lse_in).to(device)
    if stream is None:
        dq, dk, dv = backward(tq, tk, tv, o_t, lse_t, tdo, scale=sc, causal=causal, **kw)
    else:
        with torch.cuda.stream(stream):
            dq, dk, dv = backward(tq, tk, tv, o_t, lse_t, tdo, scale=sc, causal=causal, **kw)
    torch.cuda.synchronize(device)
    o_in64 = bh.to_np(o_t)
    lse_in64 = lse_t.cpu().numpy().astype(np.float64)
    refs, bounds = bh.grad_bounds(q64, k64, v64, do64, o_in64, lse_in64, sc, causal, dtype, heads=heads, mask=mask)
    got = {}
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        g = bh.to_np(t)
        got[name] = np.stack([g[b, h] for b, h in heads]) if heads is not None else g.reshape(refs[name].shape)
    bh.assert_grads_within(got, refs, bounds, w.name)
    return (tq, tk, tv, o_t, lse_t, tdo, dq, dk, dv)


ONE = (1.0, 1.0, 1.0, 1.0)
SMALL = [
    (1, 2, 300, 64, wl.FP16, False, None, ONE),
    (1, 2, 300, 64, wl.FP16, True, None, ONE),
    (2, 1, 257, 128, wl.BF16, False, None, ONE),
    (2, 1, 257, 128, wl.BF16, True, None, ONE),
    (1, 1, 1, 64, wl.FP16, True, None, ONE),
    (1, 1, 1, 128, wl.BF16, False, None, ONE),
    (1, 1, 33, 128, wl.FP16, False, None, ONE),
    (1, 3, 129, 64, wl.BF16, True, None, ONE),
    (1, 2, 64, 64, wl.FP16, False, None, ONE),
    (1, 1, 128, 128, wl.BF16, True, None, ONE),
    (1, 2, 256, 128, wl.FP16, True, -0.2, ONE),
    (1, 1, 200, 64, wl.BF16, False, 0.0, ONE),
    (1, 1, 500, 64, wl.FP16, True, None, (3.0, 3.0, 1.0, 2.0)),
    (1, 1, 380, 128, wl.BF16, False, None, (3.0, 3.0, 1.0, 0.5)),
    (2, 2, 191, 64, wl.BF16, False, 0.5, ONE),
    (1, 2, 700, 128, wl.FP16, True, None, ONE),
    (2, 2, 333, 32, wl.FP16, False, None, ONE),
    (1, 3, 515, 32, wl.BF16, True, None, ONE),
    (1, 1, 1, 32, wl.BF16, False, None, ONE),
    (1, 2, 300, 256, wl.BF16, False, None, ONE),
    (2, 1, 257, 256, wl.FP16, True, None, ONE),
    (1, 1, 70, 256, wl.BF16, True, 0.2, (3.0, 3.0, 1.0, 1.0)),
    (2, 2, 301, 96, wl.FP16, False, None, ONE),
    (1, 2, 257, 96, wl.BF16, True, -0.15, ONE),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"b{c[0]}h{c[1]}n{c[2]}d{c[3]}{c[4]}"
                         f"{'_causal' if c[5] else ''}_s{c[6]}_sig{c[7][0]:g}")
def test_bwd_small(gpu_device, case):
    _run(case, gpu_device)


@pytest.mark.parametrize("case", [(1, 2, 2048, 64, wl.FP16, True, None, ONE),
                                  (1, 2, 1024, 128, wl.BF16, False, None, ONE),
                                  (1, 1, 1500, 128, wl.FP16, False, None, ONE)],
                         ids=["n2048d64_fp16_causal", "n1024d128_bf16", "n1500d128_fp16"])
def test_bwd_medium(gpu_device, case):
    _run(case, gpu_device)


# The bench's backward workloads at full size, every element of sampled heads.
@pytest.mark.parametrize("w,heads", [(wl.HEADLINE, [(0, 0), (0, 5)]),
                                     (wl.CAUSAL_TRAIN, [(0, 3), (1, 14)])],
                         ids=["headline_b1h8n8192d64_fp16", "causal_b2h16n4096d128_bf16"])
def test_bwd_full_size_sampled_heads(gpu_device, w, heads):
    _run((w.B, w.H, w.N, w.d, w.dtype, w.causal, None, ONE), gpu_device, heads=heads, seed=0)


@pytest.mark.parametrize("case", [(1, 2, 520, 64, wl.FP16, True, None, ONE),
                                  (2, 1, 300, 128, wl.BF16, False, None, ONE)],
                         ids=["d64_fp16_causal", "d128_bf16"])
def test_bwd_chained_after_gpu_forward(gpu_device, case):
    _run(case, gpu_device, chained=True)


def test_bwd_workspace_holds_row_statistics_and_results_repeat_bit_for_bit(gpu_device):
    from exact_attention_21_amd import fa2_bwd, FA2_OK
    B, H, N, d, dtype = 1, 2, 333, 128, wl.FP16
    tq, tk, tv, o_t, lse_t, tdo, dq, dk, dv = _run((B, H, N, d, dtype, True, None, ONE), gpu_device)
    ws = torch.full((2, B, H, N), float("nan"), dtype=torch.float32, device=gpu_device)
    outs = [torch.empty_like(tq) for _ in range(3)]
    st = fa2_bwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o_t.data_ptr(), tdo.data_ptr(), lse_t.data_ptr(),
                 outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), ws.data_ptr(), B, H, N, d,
                 1.0 / np.sqrt(d), 1, 0, torch.cuda.current_stream(gpu_device).cuda_stream)
    assert st == FA2_OK
    torch.cuda.synchronize(gpu_device)
    # No atomics: a second call gives the same bits.
    for a, b in zip(outs, (dq, dk, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # The workspace: -Delta, then -LSE * log2(e), of every row.
    do64, o64 = bh.to_np(tdo), bh.to_np(o_t)
    delta = np.sum(do64 * o64, axis=3)
    tol = d * 2.0 ** -24 * np.sum(np.abs(do64 * o64), axis=3)
    got = ws.cpu().numpy().astype(np.float64)
    print(f"  Delta: max err {float(np.max(np.abs(-got[0] - delta))):.3e}", flush=True)
    assert np.all(np.abs(-got[0] - delta) <= tol)
    l2 = lse_t.cpu().numpy().astype(np.float64) * np.log2(np.e)
    assert np.all(np.abs(-got[1] - l2) <= 2.0 ** -22 * np.abs(l2))


def test_bwd_on_a_side_stream(gpu_device):
    s = torch.cuda.Stream(device=gpu_device)
    _run((1, 2, 400, 64, wl.BF16, True, None, ONE), gpu_device, stream=s)


def _draw_bwd_case(i):
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice((32, 64, 96, 128, 256)))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    N = int(rng.integers(1, 700))
    dtype = wl.FP16 if rng.random() < 0.5 else wl.BF16
    scale = float(rng.choice([1.0, -1.0]) * rng.uniform(0.3, 1.5) / np.sqrt(d))
    causal = bool(rng.random() < 0.5)
    return (B, H, N, d, dtype, causal, scale, ONE)


RANDOM_CASES = [_draw_bwd_case(i) for i in range(24)]


@pytest.mark.parametrize("case", RANDOM_CASES,
                         ids=[f"{i}-b{c[0]}h{c[1]}n{c[2]}d{c[3]}{c[4]}{'c' if c[5] else ''}"
                              for i, c in enumerate(RANDOM_CASES)])
def test_bwd_random_shapes(gpu_device, case):
    """Seeded random batch, heads, length (ragged tails of every kind), head
    dim, dtype, scale of either sign and mask: every element of dQ, dK, dV
    within the rounding bound."""
    _run(case, gpu_device, seed=case[2] + case[3])



# (B, H, N, d, dtype) with (window_left, window_right, key_lens): two-sided,
# left-only and right-only windows, key lengths with a fully padded sequence
# (and rows that see no key), the causal window with lengths, a window wider
# than N.
MASKED = [
    ((1, 2, 300, 64, wl.FP16), (40, 7, None)),
    ((2, 1, 257, 128, wl.BF16), (-1, -1, [200, 0])),
    ((2, 2, 333, 64, wl.BF16), (64, 0, [333, 90])),
    ((1, 1, 500, 128, wl.FP16), (-1, 0, [311])),
    ((2, 1, 190, 128, wl.FP16), (5, 3, [100, 40])),
    ((1, 2, 700, 64, wl.FP16), (129, -1, None)),
    ((1, 1, 260, 64, wl.BF16), (1000, 1000, None)),
    ((3, 1, 150, 64, wl.FP16), (0, 0, [150, 1, 77])),
    ((2, 2, 280, 32, wl.BF16), (50, 10, [280, 99])),
    ((2, 1, 300, 256, wl.BF16), (70, 0, [300, 130])),
    ((1, 3, 222, 96, wl.FP16), (-1, 20, [150])),
]


@pytest.mark.parametrize("shape,mask", MASKED, ids=[f"{s[2]}d{s[3]}{s[4]}-{m}" for s, m in MASKED])
def test_bwd_masked(gpu_device, shape, mask):
    """fa2_bwd_masked against the masked oracle's gradients, every element;
    keys past a length get dK = dV = 0 and rows that see no key dQ = 0,
    exactly."""
    B, H, N, d, dtype = shape
    tq, tk, tv, o_t, lse_t, tdo, dq, dk, dv = _run((B, H, N, d, dtype, False, None, ONE), gpu_device, mask=mask)
    lens = mask[2]
    if lens is not None:
        for b, n_b in enumerate(lens):
            assert torch.count_nonzero(dk[b, :, n_b:]).item() == 0 and torch.count_nonzero(dv[b, :, n_b:]).item() == 0
    hidden = torch.isinf(lse_t)
    assert torch.count_nonzero(dq[hidden]).item() == 0


@pytest.mark.parametrize("case", [(2, 2, 400, 64, wl.FP16, False, None, ONE),
                                  (1, 2, 300, 128, wl.BF16, False, None, ONE)],
                         ids=["d64_fp16", "d128_bf16"])
def test_bwd_masked_chained_after_gpu_forward(gpu_device, case):
    _run(case, gpu_device, chained=True, mask=(100, 0, [400, 250][:case[0]]))


# (B, H, N, d, key lengths or None, sampled (b, h) pairs)
GROUPED = [
    (8, 16, 1100, 64, None, [(0, 0), (2, 9), (5, 3), (7, 15)]),
    (8, 16, 1100, 64, [1100, 700, 1, 1099, 0, 256, 900, 129], [(0, 0), (2, 9), (5, 3), (7, 15)]),
    (10, 13, 700, 32, [700, 5, 699, 0, 333, 128, 129, 650, 1, 512], [(0, 0), (4, 7), (9, 11), (9, 12)]),
]


@pytest.mark.parametrize("case", GROUPED, ids=["causal", "causal_key_lens", "key_lens_last_group_of_2"])
def test_bwd_grouped_work_order(gpu_device, case):
    """Masked grids of 128 slices or more take the work in XCD-sized slice
    groups (8 slices; 130 slices leave a last group of 2), and with key
    lengths in two phases of steps (9 tiles per slice at N = 1100: phases of
    5 and 4; 6 at N = 700: 3 and 3): every element of dQ, dK, dV is written
    (the outputs start as NaN) and sampled heads, from the first and the
    last groups among others, match the oracle."""
    B, H, N, d, lens, heads = case
    dtype = wl.FP16
    w, q, k, v, do = bh.make_case(B, H, N, d, dtype, 9, causal=True)
    sc = w.softmax_scale()
    q64, k64, v64, do64 = (wl.to_float64(x, dtype) for x in (q, k, v, do))
    tq, tk, tv, tdo = (to_device(x, dtype, gpu_device) for x in (q, k, v, do))
    mask = (-1, 0, lens) if lens is not None else None
    kw = dict(window=(-1, 0), key_lens=torch.tensor(lens, dtype=torch.int32, device=gpu_device)) \
        if lens is not None else dict(causal=True)
    o_t, lse_t = forward(tq, tk, tv, scale=sc, **kw)
    out = tuple(torch.full_like(tq, float("nan")) for _ in range(3))
    dq, dk, dv = backward(tq, tk, tv, o_t, lse_t, tdo, scale=sc, out=out, **kw)
    torch.cuda.synchronize(gpu_device)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all().item()), "an output tile was not written"
    refs, bounds = bh.grad_bounds(q64, k64, v64, do64, bh.to_np(o_t), lse_t.cpu().numpy().astype(np.float64), sc,
                                  True, dtype, heads=heads, mask=mask)
    got = {name: np.stack([bh.to_np(t)[b, h] for b, h in heads]) for name, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    bh.assert_grads_within(got, refs, bounds, "grouped work order")
