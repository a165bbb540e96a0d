"""The C ABI on the host: the library loads, exports what include/fa2.h declares,
and rejects bad arguments with status codes before any HIP call (so these
tests need no GPU and launch nothing)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_attention_21_amd as fa
from exact_attention_21_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_functions():
    assert declared_functions() == sorted(bd.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = fa.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        for name in declared_functions():
            assert re.search(rf"\bT {name}$", out.stdout, re.M), name


def test_status_strings():
    for st in range(0, 10):
        s = fa.fa2_status_string(st)
        assert isinstance(s, str) and s and s != "unknown status"
    assert fa.fa2_status_string(99) == "unknown status"


# Fake, 16-byte aligned, non-overlapping "device" addresses: the checks under
# test return before anything dereferences them.
Q, K, V, O, L = (0x10000000 * (i + 1) for i in range(5))


def call(**kw):
    args = dict(Q=Q, K=K, V=V, O=O, LSE=L, B=1, H=2, N=100, d=64, scale=0.125, is_causal=0,
                dtype=fa.FA2_DTYPE_FP16, stream=0)
    args.update(kw)
    return fa.fa2_fwd(**args)


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "LSE"])
def test_null_pointer(name):
    assert call(**{name: 0}) == bd.FA2_ERR_NULL_POINTER


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(B=-1), dict(N=-5),
                                dict(N=1 << 24, d=64), dict(N=(1 << 22), d=256),
                                dict(B=1 << 20, H=1 << 20)])
def test_bad_shape(kw):
    assert call(**kw) == bd.FA2_ERR_BAD_SHAPE


@pytest.mark.parametrize("d", [0, 1, 16, 31, 48, 63, 65, 80, 160, 192, 384, 768, 2048])
def test_unsupported_head_dim(d):
    assert call(d=d) == bd.FA2_ERR_UNSUPPORTED_HEAD_DIM


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_unsupported_dtype(dtype):
    assert call(dtype=dtype) == bd.FA2_ERR_UNSUPPORTED_DTYPE


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_bad_scale(scale):
    assert call(scale=scale) == bd.FA2_ERR_BAD_SCALE


@pytest.mark.parametrize("kw", [dict(Q=Q + 2), dict(K=K + 8), dict(V=V + 4), dict(O=O + 1),
                                dict(LSE=L + 2)])
def test_misaligned(kw):
    assert call(**kw) == bd.FA2_ERR_MISALIGNED


@pytest.mark.parametrize("kw", [dict(O=Q), dict(O=K + 16), dict(LSE=V + 64), dict(LSE=O + 32),
                                dict(O=L - 16)])
def test_overlap(kw):
    assert call(**kw) == bd.FA2_ERR_OVERLAP


def test_launch_info_headline_shape():
    info = fa.fa2_launch_info(1, 8, 8192, 64, 0, fa.FA2_DTYPE_FP16)
    assert info["rows_per_wg"] * math.ceil(8192 / info["rows_per_wg"]) * 8 \
        == info["workgroups"] * info["rows_per_wg"]
    assert info["threads"] % 64 == 0 and info["lds_bytes"] <= 160 * 1024
    for d in (32, 64, 96, 128, 256, 512, 1024):
        i = fa.fa2_launch_info(4, 8, 2047, d, 1, fa.FA2_DTYPE_BF16)
        assert i["workgroups"] == 32 * math.ceil(2047 / i["rows_per_wg"])
        assert i["lds_bytes"] <= 160 * 1024


# (B, H, N, d, causal, dtype) -> threads per workgroup the launch picks for
# d = 32, 64 and 128 (512: 8-wave form, 256: 4-wave form).  Without a GPU
# the library assumes 256 compute units, so the grid sizes below are 1, 2 and
# 3 workgroups per CU (256 query rows per workgroup at d = 64, 128 at d = 32)
# and, for d = 128, 0.5 to 4 workgroups of the 8-wave form per CU (256 rows).
# (B, H, N, d, is_causal, dtype), threads, query rows per workgroup
FORM_CHOICES = [
    ((1, 8, 8192, 64, 0, 0), 512, 256),  # no mask, one per CU: split-KV
    ((2, 8, 8192, 64, 0, 0), 256, 256),  # no mask, two per CU: 4-wave
    ((2, 8, 8192, 64, 0, 1), 256, 256),
    ((2, 8, 8192, 64, 1, 0), 512, 256),  # fp16 causal d = 64 keeps split-KV at two per CU
    ((3, 8, 8192, 64, 1, 0), 256, 256),  # and takes the 4-wave form from three
    ((1, 8, 8192, 64, 1, 1), 256, 256),  # bf16 d = 64 under a mask: 4-wave at every grid size
    ((1, 2, 300, 64, 1, 1), 256, 256),
    ((1, 8, 4096, 32, 1, 0), 512, 128),  # d = 32 causal, one per CU: split-KV
    ((2, 8, 4096, 32, 1, 0), 256, 128),  # two per CU: 4-wave
    ((4, 8, 8192, 128, 1, 1), 512, 256),  # d = 128 causal, four 8-wave workgroups per CU: 8 waves
    ((1, 8, 8192, 128, 0, 0), 256, 256),  # no mask, one per CU: 4 waves of 64 rows
    ((4, 8, 8192, 128, 0, 1), 256, 256),  # no mask, four per CU: 4 waves of 64 rows
    ((1, 16, 4096, 128, 1, 1), 256, 128),  # causal, one per CU: 4 waves of 32 rows
    ((1, 32, 1024, 128, 0, 0), 256, 128),  # no mask, half a round: 4 waves of 32 rows
    ((2, 16, 4096, 128, 1, 0), 512, 256),  # causal, two per CU: 8 waves
]


@pytest.mark.parametrize("args,threads,rows", FORM_CHOICES, ids=[str(a) for a, _, _ in FORM_CHOICES])
def test_launch_form_choice_without_gpu(args, threads, rows):
    info = fa.fa2_launch_info(*args)
    assert info["threads"] == threads
    assert info["rows_per_wg"] == rows
    B, H, N = args[:3]
    assert info["workgroups"] == B * H * math.ceil(N / info["rows_per_wg"])


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256, 512, 1024])
def test_slice_size_limit(d):
    """(N + 256) * d * 2 bytes must stay below 2^31."""
    n_max = -(-(1 << 31) // (2 * d)) - 256 - 1  # largest N with (N + 256) * 2d < 2^31
    fa.fa2_launch_info(1, 1, n_max, d, 0, fa.FA2_DTYPE_FP16)
    with pytest.raises(bd.Fa2Error):
        fa.fa2_launch_info(1, 1, n_max + 1, d, 0, fa.FA2_DTYPE_FP16)


def test_launch_info_rejects_what_fwd_rejects():
    with pytest.raises(bd.Fa2Error):
        fa.fa2_launch_info(1, 1, 1, 80, 0, 0)
    with pytest.raises(bd.Fa2Error):
        fa.fa2_launch_info(1, 1, 0, 64, 0, 0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "libfa2.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bd.library()


# ---- fa2_fwd_masked --------------------------------------------------------

LENS = 0x60000000  # fake, 4-byte aligned key-length array


def call_masked(**kw):
    args = dict(Q=Q, K=K, V=V, O=O, LSE=L, B=2, H=2, N=100, d=64, scale=0.125, window_left=16,
                window_right=0, key_lens=LENS, dtype=fa.FA2_DTYPE_FP16, stream=0)
    args.update(kw)
    return fa.fa2_fwd_masked(**args)


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "LSE"])
def test_masked_null_pointer(name):
    assert call_masked(**{name: 0}) == bd.FA2_ERR_NULL_POINTER


@pytest.mark.parametrize("kw", [dict(key_lens=LENS + 2), dict(key_lens=LENS + 1), dict(Q=Q + 8), dict(LSE=L + 2)])
def test_masked_misaligned(kw):
    assert call_masked(**kw) == bd.FA2_ERR_MISALIGNED


@pytest.mark.parametrize("kw", [dict(key_lens=O + 64), dict(key_lens=L), dict(key_lens=L + 4 * 2 * 2 * 100 - 4),
                                dict(O=Q)])
def test_masked_overlap(kw):
    assert call_masked(**kw) == bd.FA2_ERR_OVERLAP


def test_masked_shares_fwd_checks():
    assert call_masked(d=80) == bd.FA2_ERR_UNSUPPORTED_HEAD_DIM
    assert call_masked(N=0) == bd.FA2_ERR_BAD_SHAPE
    assert call_masked(dtype=5) == bd.FA2_ERR_UNSUPPORTED_DTYPE
    assert call_masked(scale=math.nan) == bd.FA2_ERR_BAD_SCALE



# ---- fa2_bwd: the same checks, before any HIP call --------------------------
BQ_, BK_, BV_, BO_, BDO_, BL_, BDQ_, BDK_, BDV_, BW_ = (0x10000000 * (i + 1) for i in range(10))


def call_bwd(**kw):
    args = dict(Q=BQ_, K=BK_, V=BV_, O=BO_, dO=BDO_, LSE=BL_, dQ=BDQ_, dK=BDK_, dV=BDV_, workspace=BW_,
                B=1, H=2, N=100, d=64, scale=0.125, is_causal=0, dtype=fa.FA2_DTYPE_FP16, stream=0)
    args.update(kw)
    return fa.fa2_bwd(**args)


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "dO", "LSE", "dQ", "dK", "dV", "workspace"])
def test_bwd_null_pointer(name):
    assert call_bwd(**{name: 0}) == bd.FA2_ERR_NULL_POINTER


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=-3), dict(N=1 << 24, d=64),
                                dict(B=1 << 20, H=1 << 20)])
def test_bwd_bad_shape(kw):
    assert call_bwd(**kw) == bd.FA2_ERR_BAD_SHAPE


@pytest.mark.parametrize("d", [0, 16, 48, 80, 512, 1024])
def test_bwd_unsupported_head_dim(d):
    assert call_bwd(d=d) == bd.FA2_ERR_UNSUPPORTED_HEAD_DIM


@pytest.mark.parametrize("dtype", [-1, 2])
def test_bwd_unsupported_dtype(dtype):
    assert call_bwd(dtype=dtype) == bd.FA2_ERR_UNSUPPORTED_DTYPE


@pytest.mark.parametrize("scale", [math.inf, math.nan])
def test_bwd_bad_scale(scale):
    assert call_bwd(scale=scale) == bd.FA2_ERR_BAD_SCALE


@pytest.mark.parametrize("kw", [dict(Q=BQ_ + 2), dict(dO=BDO_ + 8), dict(dV=BDV_ + 4), dict(LSE=BL_ + 2),
                                dict(workspace=BW_ + 1)])
def test_bwd_misaligned(kw):
    assert call_bwd(**kw) == bd.FA2_ERR_MISALIGNED


@pytest.mark.parametrize("kw", [dict(dQ=BQ_), dict(dK=BO_ + 16), dict(dV=BDK_ + 32), dict(workspace=BL_ + 4),
                                dict(workspace=BDQ_ + 64), dict(dQ=BL_ - 16)])
def test_bwd_overlap(kw):
    assert call_bwd(**kw) == bd.FA2_ERR_OVERLAP


def test_bwd_noalloc_checks_and_scratch_limit():
    # 4 GiB apart: tensors of 2^21 rows of 64 dims do not overlap.
    p = [(i + 1) << 32 for i in range(9)]
    base = dict(Q=p[0], K=p[1], V=p[2], O=p[3], dO=p[4], LSE=p[5], dQ=p[6], dK=p[7], dV=p[8],
                B=1, H=64, N=(1 << 21) // 64 + 1, d=64, scale=0.125, is_causal=0, dtype=0, stream=0)
    assert fa.fa2_bwd_noalloc(**base) == bd.FA2_ERR_TOO_LARGE
    assert fa.fa2_bwd_noalloc(**{**base, "dQ": 0}) == bd.FA2_ERR_NULL_POINTER
    assert fa.fa2_bwd_noalloc(**{**base, "d": 80}) == bd.FA2_ERR_UNSUPPORTED_HEAD_DIM
    assert fa.fa2_bwd_noalloc(**{**base, "dK": p[0]}) == bd.FA2_ERR_OVERLAP


def test_bwd_masked_checks():
    base = dict(Q=BQ_, K=BK_, V=BV_, O=BO_, dO=BDO_, LSE=BL_, dQ=BDQ_, dK=BDK_, dV=BDV_, workspace=BW_,
                B=2, H=2, N=100, d=64, scale=0.125, window_left=16, window_right=0, key_lens=LENS,
                dtype=0, stream=0)
    assert fa.fa2_bwd_masked(**{**base, "workspace": 0}) == bd.FA2_ERR_NULL_POINTER
    assert fa.fa2_bwd_masked(**{**base, "d": 80}) == bd.FA2_ERR_UNSUPPORTED_HEAD_DIM
    assert fa.fa2_bwd_masked(**{**base, "key_lens": LENS + 2}) == bd.FA2_ERR_MISALIGNED
    assert fa.fa2_bwd_masked(**{**base, "dQ": LENS}) == bd.FA2_ERR_OVERLAP
    assert fa.fa2_bwd_masked(**{**base, "N": 0}) == bd.FA2_ERR_BAD_SHAPE
