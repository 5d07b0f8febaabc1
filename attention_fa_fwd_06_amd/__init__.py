"""Python binding of libfa.so, the gfx950 FlashAttention-2 training attention.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/fa.h. torch tensors provide the
device memory and the stream. There is no fallback: if libfa.so is missing
or fails to load, every call raises.

Low-level calls (same names and argument order as the C ABI; outputs are
caller-allocated tensors):
    fa_fwd(q, k, v, o, lse, scale, causal, window)
    fa_bwd_preprocess(o, do, delta)
    fa_bwd_dkv(q, k, v, do, lse, delta, dk, dv, scale, causal, window)
    fa_bwd_dq(q, k, v, do, lse, delta, dq, scale, causal, window)
    fa_fwd_masked, fa_bwd_dkv_masked, fa_bwd_dq_masked, fa_fwd_ex, fa_bwd_dkv_ex,
    fa_bwd_dq_ex: reached through the calls above when a mask is given or v's
    head dim Dv differs from q's D (then o, dO and dv are [.., Dv])
Convenience wrappers that allocate their outputs:
    forward(q, k, v, scale=None, causal=False, window=0, mask=None) -> (o, lse)
    backward(q, k, v, o, lse, do, scale=None, causal=False, window=0, mask=None) -> (dq, dk, dv)
A mask is a float32 or bool GPU tensor whose last two dims are [Lq, Lkv]
(contiguous rows); up to two leading dims broadcast against [B, Hq] the way
torch aligns shapes (right-aligned, size 1 or the full size). A float32 mask
is added to the scaled scores (0 attends, -inf blocks); a bool mask is True
where the pair may attend (it runs through the extended calls, which read it
as one byte per pair).
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; FA_LIBRARY may name another build of the same sources.
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_SHAPE",
    -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_ALIGN",
    -6: "FA_ERR_ARG",
    -7: "FA_ERR_LAUNCH",
}
EXPORTS = ("fa_fwd", "fa_bwd_preprocess", "fa_bwd_dkv", "fa_bwd_dq", "fa_fwd_masked", "fa_bwd_dkv_masked",
           "fa_bwd_dq_masked", "fa_fwd_ex", "fa_bwd_dkv_ex", "fa_bwd_dq_ex", "fa_status_string")

_lib = None


class FaError(ValueError):
    """A status other than FA_OK returned by libfa.so."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {status_string(status)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (once) and declare its signatures. Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_fa_fwd_06_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
    lib.fa_bwd_preprocess.argtypes = [P, P, P, I, I, I, I, I, P]
    lib.fa_bwd_dkv.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
    lib.fa_bwd_dq.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P]
    LL = ctypes.c_longlong
    lib.fa_fwd_masked.argtypes = [P, P, P, P, LL, LL, P, P, I, I, I, I, I, I, F, I, I, I, P]
    lib.fa_bwd_dkv_masked.argtypes = [P, P, P, P, P, P, P, LL, LL, P, P, I, I, I, I, I, I, F, I, I, I, P]
    lib.fa_bwd_dq_masked.argtypes = [P, P, P, P, P, P, P, LL, LL, P, I, I, I, I, I, I, F, I, I, I, P]
    lib.fa_fwd_ex.argtypes = [P, P, P, P, P, P, I, P]
    lib.fa_bwd_dkv_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, P]
    lib.fa_bwd_dq_ex.argtypes = [P, P, P, P, P, P, P, P, I, P]
    for fn in ("fa_fwd", "fa_bwd_preprocess", "fa_bwd_dkv", "fa_bwd_dq", "fa_fwd_masked", "fa_bwd_dkv_masked",
               "fa_bwd_dq_masked", "fa_fwd_ex", "fa_bwd_dkv_ex", "fa_bwd_dq_ex"):
        getattr(lib, fn).restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_status_string(status: int) -> str:
    return status_string(status)


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}: use float32, float16 or bfloat16")
    return codes[t.dtype]


def _ptr(t, name, device=None, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise FaError(fn, status)


def _shape4(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _attn_shapes(q, k, v):
    """(B, Hq, Hkv, Lq, Lkv, D, Dv) of q [B,Hq,Lq,D], k [B,Hkv,Lkv,D], v [B,Hkv,Lkv,Dv]."""
    B, Hq, Lq, D = _shape4(q, "q")
    Bk, Hkv, Lkv, Dk = _shape4(k, "k")
    Bv, Hv, Lv, Dv = _shape4(v, "v")
    if (Bv, Hv, Lv) != (Bk, Hkv, Lkv):
        raise ValueError(f"v shape {tuple(v.shape)} must match k shape {tuple(k.shape)} except in the head dim")
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head dim")
    return B, Hq, Hkv, Lq, Lkv, D, Dv


def _mask_args(mask, B, Hq, Lq, Lkv, dev):
    """(pointer, batch stride, head stride, is_bool) of an additive float32 or a
    boolean mask tensor broadcast to [B, Hq, Lq, Lkv] (see include/fa.h, masked
    variants and bool_mask of the extended calls); strides in elements."""
    import torch

    if not mask.is_cuda or mask.device != dev:
        raise ValueError(f"mask must be on {dev}")
    if mask.dtype not in (torch.float32, torch.bool):
        raise ValueError(f"mask must be float32 or bool, got {mask.dtype}")
    if mask.dim() < 2 or mask.dim() > 4 or tuple(mask.shape[-2:]) != (Lq, Lkv):
        raise ValueError(f"mask shape {tuple(mask.shape)} must end in [Lq, Lkv] = [{Lq}, {Lkv}] with at most 4 dims")
    if mask.stride(-1) != 1 or (Lq > 1 and mask.stride(-2) != Lkv):
        raise ValueError("mask rows must be contiguous: strides [..., Lkv, 1]")
    lead = [1] * (4 - mask.dim()) + list(mask.shape[:-2])
    strides = [0] * (4 - mask.dim()) + list(mask.stride()[:-2])
    for n, (size, full, name) in enumerate(zip(lead, (B, Hq), ("batch", "head"))):
        if size not in (1, full):
            raise ValueError(f"mask {name} dim is {size}; it must be 1 or {full}")
    msb = strides[0] if lead[0] > 1 else 0
    msh = strides[1] if lead[1] > 1 else 0
    return mask.data_ptr(), int(msb), int(msh), mask.dtype == torch.bool


class FaAttnDesc(ctypes.Structure):
    """fa_attn_desc_t of include/fa.h (the extended calls)."""

    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("Lq", ctypes.c_int),
                ("Lkv", ctypes.c_int), ("D", ctypes.c_int), ("Dv", ctypes.c_int), ("scale", ctypes.c_float),
                ("causal", ctypes.c_int), ("window", ctypes.c_int), ("mask", ctypes.c_void_p),
                ("mask_stride_b", ctypes.c_longlong), ("mask_stride_h", ctypes.c_longlong),
                ("bool_mask", ctypes.c_void_p)]


def _desc(dims, scale, causal, window, margs):
    B, Hq, Hkv, Lq, Lkv, D, Dv = dims
    ptr, msb, msh, is_bool = margs if margs is not None else (None, 0, 0, False)
    return FaAttnDesc(B, Hq, Hkv, Lq, Lkv, D, Dv, float(scale), int(bool(causal)), int(window),
                      None if is_bool else ptr, msb, msh, ptr if is_bool else None)


def _extended(dims, margs):
    """The extended calls serve a value head dim other than D and bool masks."""
    return dims[6] != dims[5] or (margs is not None and margs[3])


def fa_fwd(q, k, v, o, lse, scale, causal=False, window=0, mask=None):
    """O and LSE of softmax attention (see include/fa.h: fa_fwd, or fa_fwd_masked
    with a mask, or fa_fwd_ex when v's head dim differs from q's)."""
    lib = load_library()
    import torch

    dims = _attn_shapes(q, k, v)
    B, Hq, Hkv, Lq, Lkv, D, Dv = dims
    dev, dt = q.device, q.dtype
    if tuple(o.shape) != (B, Hq, Lq, Dv) or tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("o must be [B, Hq, Lq, Dv] and lse [B, Hq, Lq]")
    ins = (_ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt))
    outs = (_ptr(o, "o", dev, dt), _ptr(lse, "lse", dev, torch.float32))
    margs = None if mask is None else _mask_args(mask, B, Hq, Lq, Lkv, dev)
    if _extended(dims, margs):
        desc = _desc(dims, scale, causal, window, margs)
        _check("fa_fwd_ex", lib.fa_fwd_ex(ctypes.byref(desc), *ins, *outs, _dtype_code(q), _stream(dev)))
        return
    rest = (B, Hq, Hkv, Lq, Lkv, D, float(scale), int(bool(causal)), int(window), _dtype_code(q), _stream(dev))
    if mask is None:
        _check("fa_fwd", lib.fa_fwd(*ins, *outs, *rest))
    else:
        _check("fa_fwd_masked", lib.fa_fwd_masked(*ins, *margs[:3], *outs, *rest))


def fa_bwd_preprocess(o, do, delta):
    """delta = rowsum(dO * O) (see include/fa.h, fa_bwd_preprocess)."""
    lib = load_library()
    import torch

    B, Hq, Lq, D = _shape4(o, "o")
    dev, dt = o.device, o.dtype
    if tuple(do.shape) != tuple(o.shape) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("dO must match o and delta must be [B, Hq, Lq]")
    st = lib.fa_bwd_preprocess(_ptr(o, "o", dev, dt), _ptr(do, "dO", dev, dt), _ptr(delta, "delta", dev, torch.float32),
                               B, Hq, Lq, D, _dtype_code(o), _stream(dev))
    _check("fa_bwd_preprocess", st)


def _bwd_common(q, k, v, do, lse, delta):
    import torch

    dims = _attn_shapes(q, k, v)
    B, Hq, Hkv, Lq, Lkv, D, Dv = dims
    if tuple(do.shape) != (B, Hq, Lq, Dv):
        raise ValueError("dO must be [B, Hq, Lq, Dv]")
    if tuple(lse.shape) != (B, Hq, Lq) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("lse and delta must be [B, Hq, Lq]")
    dev, dt = q.device, q.dtype
    ptrs = [_ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt), _ptr(do, "dO", dev, dt),
            _ptr(lse, "lse", dev, torch.float32), _ptr(delta, "delta", dev, torch.float32)]
    return dims, ptrs, dev, dt


def fa_bwd_dkv(q, k, v, do, lse, delta, dk, dv, scale, causal=False, window=0, mask=None):
    """dK and dV (see include/fa.h: fa_bwd_dkv, fa_bwd_dkv_masked, fa_bwd_dkv_ex)."""
    lib = load_library()
    dims, ptrs, dev, dt = _bwd_common(q, k, v, do, lse, delta)
    B, Hq, Hkv, Lq, Lkv, D, Dv = dims
    if tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(v.shape):
        raise ValueError("dk must match k and dv must match v")
    outs = (_ptr(dk, "dk", dev, dt), _ptr(dv, "dv", dev, dt))
    margs = None if mask is None else _mask_args(mask, B, Hq, Lq, Lkv, dev)
    if _extended(dims, margs):
        desc = _desc(dims, scale, causal, window, margs)
        _check("fa_bwd_dkv_ex", lib.fa_bwd_dkv_ex(ctypes.byref(desc), *ptrs, *outs, _dtype_code(q), _stream(dev)))
        return
    rest = (B, Hq, Hkv, Lq, Lkv, D, float(scale), int(bool(causal)), int(window), _dtype_code(q), _stream(dev))
    if mask is None:
        _check("fa_bwd_dkv", lib.fa_bwd_dkv(*ptrs, *outs, *rest))
    else:
        _check("fa_bwd_dkv_masked", lib.fa_bwd_dkv_masked(*ptrs, *margs[:3], *outs, *rest))


def fa_bwd_dq(q, k, v, do, lse, delta, dq, scale, causal=False, window=0, mask=None):
    """dQ (see include/fa.h: fa_bwd_dq, fa_bwd_dq_masked, fa_bwd_dq_ex)."""
    lib = load_library()
    dims, ptrs, dev, dt = _bwd_common(q, k, v, do, lse, delta)
    B, Hq, Hkv, Lq, Lkv, D, Dv = dims
    if tuple(dq.shape) != tuple(q.shape):
        raise ValueError("dq must match q")
    margs = None if mask is None else _mask_args(mask, B, Hq, Lq, Lkv, dev)
    if _extended(dims, margs):
        desc = _desc(dims, scale, causal, window, margs)
        _check("fa_bwd_dq_ex", lib.fa_bwd_dq_ex(ctypes.byref(desc), *ptrs, _ptr(dq, "dq", dev, dt), _dtype_code(q),
                                                _stream(dev)))
        return
    rest = (B, Hq, Hkv, Lq, Lkv, D, float(scale), int(bool(causal)), int(window), _dtype_code(q), _stream(dev))
    if mask is None:
        _check("fa_bwd_dq", lib.fa_bwd_dq(*ptrs, _ptr(dq, "dq", dev, dt), *rest))
    else:
        _check("fa_bwd_dq_masked", lib.fa_bwd_dq_masked(*ptrs, *margs[:3], _ptr(dq, "dq", dev, dt), *rest))


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def forward(q, k, v, scale=None, causal=False, window=0, mask=None):
    """Allocate O and LSE and run fa_fwd (fa_fwd_masked with a mask). Returns (o, lse)."""
    import torch

    B, Hq, Lq, D = q.shape
    o = torch.empty((B, Hq, Lq, v.shape[-1]), device=q.device, dtype=q.dtype)
    lse = torch.empty((B, Hq, Lq), device=q.device, dtype=torch.float32)
    fa_fwd(q, k, v, o, lse, default_scale(D) if scale is None else scale, causal, window, mask)
    return o, lse


def backward(q, k, v, o, lse, do, scale=None, causal=False, window=0, delta=None, mask=None):
    """Run the three backward phases (masked dK/dV and dQ with a mask). Returns (dq, dk, dv)."""
    import torch

    B, Hq, Lq, D = q.shape
    scale = default_scale(D) if scale is None else scale
    if delta is None:
        delta = torch.empty((B, Hq, Lq), device=q.device, dtype=torch.float32)
    fa_bwd_preprocess(o, do, delta)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd_dkv(q, k, v, do, lse, delta, dk, dv, scale, causal, window, mask)
    fa_bwd_dq(q, k, v, do, lse, delta, dq, scale, causal, window, mask)
    return dq, dk, dv
