"""C-ABI boundary checks that need no GPU.

Every call here either only loads the library or passes an argument that the
library must reject before it makes any HIP call; none of them launches work.
The fake device pointers are never dereferenced.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest
import torch

import attention_fa_fwd_06_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, HEADDIM, DTYPE, ALIGN, ARG = 0, -1, -2, -3, -4, -5, -6
P = 0x10000  # 16-byte aligned, never dereferenced


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built: run python -m attention_fa_fwd_06_amd.build")
    return fa.load_library()


def test_header_declares_every_exported_call():
    assert _declared() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name


def test_status_strings(lib):
    for code in range(-7, 1):
        s = fa.status_string(code)
        assert isinstance(s, str) and s
    assert fa.status_string(0) == "ok"
    assert fa.status_string(-99) == "unknown status"


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Lq=64, Lkv=64, D=64, scale=0.125, causal=1, window=0,
         dtype=fa.FA_BF16):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lkv, D, scale, causal, window, dtype, None)


def _dkv(lib, ptrs=(P,) * 8, B=1, Hq=4, Hkv=2, Lq=64, Lkv=64, D=64, scale=0.125, causal=1, window=0,
         dtype=fa.FA_BF16):
    return lib.fa_bwd_dkv(*ptrs, B, Hq, Hkv, Lq, Lkv, D, scale, causal, window, dtype, None)


def _dq(lib, ptrs=(P,) * 7, B=1, Hq=4, Hkv=2, Lq=64, Lkv=64, D=64, scale=0.125, causal=1, window=0,
        dtype=fa.FA_BF16):
    return lib.fa_bwd_dq(*ptrs, B, Hq, Hkv, Lq, Lkv, D, scale, causal, window, dtype, None)


@pytest.mark.parametrize("which", range(5))
def test_fwd_null_pointers(lib, which):
    args = dict(q=P, k=P, v=P, o=P, lse=P)
    args[list(args)[which]] = None
    assert _fwd(lib, **args) == NULL


@pytest.mark.parametrize("which", range(8))
def test_dkv_null_pointers(lib, which):
    ptrs = [P] * 8
    ptrs[which] = None
    assert _dkv(lib, ptrs) == NULL


@pytest.mark.parametrize("which", range(7))
def test_dq_null_pointers(lib, which):
    ptrs = [P] * 7
    ptrs[which] = None
    assert _dq(lib, ptrs) == NULL


@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(B=0), SHAPE),
        (dict(Hq=0), SHAPE),
        (dict(Hkv=0), SHAPE),
        (dict(Lq=0), SHAPE),
        (dict(Lkv=0), SHAPE),
        (dict(Hq=6, Hkv=4), SHAPE),
        (dict(Lq=1 << 24), SHAPE),
        (dict(B=1 << 12, Hq=64, Hkv=64, Lq=1 << 12, Lkv=16, D=128), SHAPE),
        (dict(Lq=(1 << 21) + 8, Lkv=64, D=256), SHAPE),
        (dict(Lq=64, Lkv=(1 << 20) + 8, D=512), SHAPE),
        (dict(D=24), HEADDIM),
        (dict(D=36), HEADDIM),
        (dict(D=520), HEADDIM),
        (dict(D=520, dtype=fa.FA_F32), HEADDIM),
        (dict(dtype=3), DTYPE),
        (dict(dtype=-1), DTYPE),
        (dict(window=-1), ARG),
        (dict(scale=math.inf), ARG),
        (dict(scale=math.nan), ARG),
    ],
)
def test_bad_arguments_are_rejected_by_all_attention_calls(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert _dkv(lib, **kw) == code
    assert _dq(lib, **kw) == code


@pytest.mark.parametrize("which", range(5))
def test_fwd_misaligned_pointer(lib, which):
    args = dict(q=P, k=P, v=P, o=P, lse=P)
    args[list(args)[which]] = P + 8
    assert _fwd(lib, **args) == ALIGN


@pytest.mark.parametrize("which", range(8))
def test_dkv_misaligned_pointer(lib, which):
    ptrs = [P] * 8
    ptrs[which] = P + 4
    assert _dkv(lib, ptrs) == ALIGN


def test_preprocess_rejections(lib):
    f = lib.fa_bwd_preprocess
    assert f(None, P, P, 1, 2, 16, 64, fa.FA_F16, None) == NULL
    assert f(P, None, P, 1, 2, 16, 64, fa.FA_F16, None) == NULL
    assert f(P, P, None, 1, 2, 16, 64, fa.FA_F16, None) == NULL
    assert f(P, P, P, 0, 2, 16, 64, fa.FA_F16, None) == SHAPE
    assert f(P, P, P, 1, 2, 0, 64, fa.FA_F16, None) == SHAPE
    assert f(P, P, P, 1, 2, 16, 60, fa.FA_F16, None) == HEADDIM
    assert f(P, P, P, 1, 2, 16, 64, 7, None) == DTYPE
    assert f(P + 2, P, P, 1, 2, 16, 64, fa.FA_F16, None) == ALIGN
    assert f(P, P, P + 12, 1, 2, 16, 64, fa.FA_F16, None) == ALIGN


def test_binding_rejects_cpu_tensors_before_calling(lib):
    q = torch.zeros(1, 2, 16, 32)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous(), q.clone(), torch.zeros(1, 2, 16), 0.1)


def test_binding_checks_shapes(lib):
    q = torch.zeros(1, 2, 16, 32)
    k = torch.zeros(1, 1, 16, 32)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, torch.zeros(1, 1, 8, 32), q.clone(), torch.zeros(1, 2, 16), 0.1)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, torch.zeros(1, 1, 16, 64), torch.zeros(1, 1, 16, 64), q.clone(), torch.zeros(1, 2, 16), 0.1)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(RuntimeError):
        fa.load_library(str(tmp_path / "nope.so"))


def _fwdm(lib, mask=P, msb=0, msh=0, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Lq=64, Lkv=64, D=64, scale=0.125, causal=1, window=0,
                dtype=fa.FA_BF16)
    args.update(kw)
    a = args
    return lib.fa_fwd_masked(a["q"], a["k"], a["v"], mask, msb, msh, a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["Lq"], a["Lkv"], a["D"], a["scale"], a["causal"], a["window"], a["dtype"], None)


def _dkvm(lib, mask=P, msb=0, msh=0, D=64, dtype=fa.FA_BF16):
    return lib.fa_bwd_dkv_masked(P, P, P, P, P, P, mask, msb, msh, P, P, 1, 4, 2, 64, 64, D, 0.125, 1, 0, dtype, None)


def _dqm(lib, mask=P, msb=0, msh=0, D=64, dtype=fa.FA_BF16):
    return lib.fa_bwd_dq_masked(P, P, P, P, P, P, mask, msb, msh, P, 1, 4, 2, 64, 64, D, 0.125, 1, 0, dtype, None)


@pytest.mark.parametrize("mask,msb,msh,code", [
    (None, 0, 0, NULL),
    (P + 2, 0, 0, ALIGN),
    (P + 4, 0, 0, OK),  # 4-byte aligned is enough (4-byte loads); launch is not reached below
    (P, -1, 0, ARG),
    (P, 0, -4096, ARG),
    (P, (1 << 40) + 4, 0, ARG),
])
def test_masked_calls_check_the_mask(lib, mask, msb, msh, code):
    if code == OK:
        # a valid mask with an invalid head dim: the call must fail on the head dim, never launch
        assert _fwdm(lib, mask, msb, msh, D=36) == HEADDIM
        assert _dkvm(lib, mask, msb, msh, D=36) == HEADDIM
        assert _dqm(lib, mask, msb, msh, D=36) == HEADDIM
        return
    assert _fwdm(lib, mask, msb, msh) == code
    assert _dkvm(lib, mask, msb, msh) == code
    assert _dqm(lib, mask, msb, msh) == code


def test_masked_calls_check_everything_else(lib):
    assert _fwdm(lib, q=None) == NULL
    assert _fwdm(lib, o=P + 8) == ALIGN
    assert _fwdm(lib, dtype=5) == DTYPE
    assert _fwdm(lib, window=-1) == ARG
    assert _fwdm(lib, Hq=3, Hkv=2) == SHAPE
    assert _dkvm(lib, dtype=9) == DTYPE
    assert _dqm(lib, D=520) == HEADDIM
    assert lib.fa_bwd_dkv_masked(P, P, P, P, P, P, P, 0, 0, None, P, 1, 4, 2, 64, 64, 64, 0.1, 1, 0,
                                 fa.FA_F16, None) == NULL
    assert lib.fa_bwd_dq_masked(P, P, P, P, P, P, P, 0, 0, P + 4, 1, 4, 2, 64, 64, 64, 0.1, 1, 0,
                                fa.FA_F16, None) == ALIGN


def test_binding_mask_shape_checks(lib):
    m = torch.zeros(64, 64)
    with pytest.raises(ValueError):
        fa._mask_args(m, 1, 4, 64, 64, torch.device("cuda", 0))  # not on the GPU


def _desc(**kw):
    d = dict(B=1, Hq=4, Hkv=2, Lq=64, Lkv=64, D=64, Dv=128, scale=0.125, causal=1, window=0, mask=None,
             mask_stride_b=0, mask_stride_h=0, bool_mask=None)
    d.update(kw)
    return fa.FaAttnDesc(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(Dv=36), HEADDIM),
    (dict(Dv=520), HEADDIM),
    (dict(Dv=24), HEADDIM),
    (dict(D=36), HEADDIM),
    (dict(Hq=5), SHAPE),
    (dict(window=-2), ARG),
    (dict(mask=P + 2), ALIGN),
    (dict(mask=P, mask_stride_h=-1), ARG),
    (dict(mask=P, bool_mask=P), ARG),                  # at most one mask
    (dict(bool_mask=P + 1, mask_stride_b=-1), ARG),
    (dict(bool_mask=P + 1, mask_stride_h=(1 << 40) + 1), ARG),
    (dict(bool_mask=P + 1, Dv=36), HEADDIM),            # a byte mask needs no alignment
    (dict(Lq=(1 << 21) + 8, Lkv=64, Dv=256), SHAPE),
])
def test_extended_calls_check_the_descriptor(lib, kw, code):
    d = ctypes.byref(_desc(**kw))
    assert lib.fa_fwd_ex(d, P, P, P, P, P, fa.FA_BF16, None) == code
    assert lib.fa_bwd_dkv_ex(d, P, P, P, P, P, P, P, P, fa.FA_BF16, None) == code
    assert lib.fa_bwd_dq_ex(d, P, P, P, P, P, P, P, fa.FA_BF16, None) == code


def test_extended_calls_null_and_dtype(lib):
    assert lib.fa_fwd_ex(None, P, P, P, P, P, fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dkv_ex(None, P, P, P, P, P, P, P, P, fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dq_ex(None, P, P, P, P, P, P, P, fa.FA_BF16, None) == NULL
    d = ctypes.byref(_desc())
    assert lib.fa_fwd_ex(d, P, P, None, P, P, fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dkv_ex(d, P, P, P, P, P, P, P, None, fa.FA_BF16, None) == NULL
    assert lib.fa_bwd_dq_ex(d, P, P, P, P, P, P, P, 4, None) == DTYPE
    assert lib.fa_fwd_ex(ctypes.byref(_desc(Dv=520)), P, P, P, P, P, fa.FA_F32, None) == HEADDIM
    d264 = ctypes.byref(_desc(Dv=264))
    for dt in (fa.FA_F32, fa.FA_F16):  # Dv = 264 passes the head-dim check for every dtype
        assert lib.fa_fwd_ex(d264, P + 4, P, P, P, P, dt, None) == ALIGN


def test_descriptor_layout_matches_the_header():
    # int x7, float, int x2, pointer, long long x2, pointer (C layout: 72 bytes,
    # the additive mask at 40, the boolean mask at 64)
    assert ctypes.sizeof(fa.FaAttnDesc) == 72
    assert fa.FaAttnDesc.mask.offset == 40 and fa.FaAttnDesc.mask_stride_h.offset == 56
    assert fa.FaAttnDesc.bool_mask.offset == 64
