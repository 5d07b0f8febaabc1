"""torch.autograd node for the attention path, plus the shape router in front of it.

One graph node: its forward is ``fa_fwd`` and saves Q, K, V, O and the
natural-log LSE; its backward runs ``fa_bwd_preprocess``, ``fa_bwd_dkv`` and
``fa_bwd_dq`` on the incoming dO. This is the contract of the VJP in
mlx-bun's flash-attention module (the forward returns O and LSE, the
backward takes the cotangents of both and uses only dO, so the LSE output is
not differentiable here), and of its routing function, which sends only the
shapes and dtypes the fused kernels support to them. Where mlx-bun falls back
to a materialised attention, this router raises instead: every call that
returns runs the HIP kernels.

Argument marshalling only; all arithmetic runs in libfa.so.
"""
from __future__ import annotations

import torch

from . import FaError, backward, default_scale, forward

_DTYPES = (torch.float32, torch.float16, torch.bfloat16)


def unsupported_reason(q, k, v, window: int = 0) -> str | None:
    """Why (q, k, v) cannot go to the fused kernels, or None if they can.

    Mirrors the checks of the C ABI (include/fa.h) so that a caller learns
    about an unsupported shape before anything is launched.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            return f"{name} is not a tensor"
        if t.dim() != 4:
            return f"{name} must be 4-D [B, H, L, D], got {tuple(t.shape)}"
        if not t.is_cuda:
            return f"{name} is on {t.device}; the kernels run on the GPU only"
        if t.dtype not in _DTYPES:
            return f"{name} has dtype {t.dtype}; supported: float32, float16, bfloat16"
    if not (q.dtype == k.dtype == v.dtype):
        return f"q, k, v dtypes differ ({q.dtype}, {k.dtype}, {v.dtype})"
    if not (q.device == k.device == v.device):
        return "q, k, v are on different devices"
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lkv, Dk = k.shape
    Dv = v.shape[3]
    if tuple(v.shape[:3]) != tuple(k.shape[:3]):
        return f"v shape {tuple(v.shape)} differs from k shape {tuple(k.shape)} outside the head dim"
    if Bk != B or Dk != D:
        return f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head dim"
    if min(B, Hq, Hkv, Lq, Lkv) <= 0:
        return "empty dimension"
    if Hq % Hkv:
        return f"Hq={Hq} is not a multiple of Hkv={Hkv}"
    for name, d in (("head dim", D), ("value head dim", Dv)):
        if d % 8 or d < 32 or d > 512:
            return f"{name} {d} outside the supported set (multiple of 8 in [32, 512])"
    if window < 0:
        return f"window must be >= 0, got {window}"
    return None


class FlashAttention(torch.autograd.Function):
    """O, LSE = attention(q, k, v); gradients flow to q, k and v through O."""

    @staticmethod
    def forward(ctx, q, k, v, scale: float, causal: bool, window: int, mask=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = forward(q, k, v, scale, causal, window, mask=mask)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.mask = mask  # the same mask for the gradient; it gets none itself
        ctx.attn = (scale, bool(causal), int(window))
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, window = ctx.attn
        if do is None:
            return None, None, None, None, None, None, None
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), scale, causal, window, mask=ctx.mask)
        return dq, dk, dv, None, None, None, None


def flash_attention(q, k, v, scale: float | None = None, causal: bool = False, window: int = 0,
                    return_lse: bool = False, mask=None):
    """Differentiable softmax(scale * q k^T + mask) v on the HIP kernels.

    q: [B, Hq, Lq, D]; k: [B, Hkv, Lkv, D]; v: [B, Hkv, Lkv, Dv] (Hq a multiple
    of Hkv; O is [B, Hq, Lq, Dv]); one of
    float32 / float16 / bfloat16 on one GPU. scale defaults to 1/sqrt(D).
    causal: key j is allowed for query i only if j <= i (top-left aligned).
    window > 0: additionally only keys with i - j < window (plus, without
    causal, every key after i). Returns O (and the natural-log LSE, which
    carries no gradient, when return_lse). mask (optional): float32 additive
    mask [.., Lq, Lkv] added to the scaled scores (0 attends, -inf blocks), or
    a bool mask of that shape, True where the pair may attend (see
    include/fa.h); the same for the gradient, itself without gradient.
    Raises ValueError for inputs the kernels do not support; nothing is
    computed any other way.
    """
    reason = unsupported_reason(q, k, v, window)
    if reason is not None:
        raise ValueError(f"flash_attention: {reason}")
    if scale is None:
        scale = default_scale(q.shape[-1])
    if mask is not None and mask.requires_grad:
        raise ValueError("flash_attention: the mask carries no gradient; pass mask.detach()")
    o, lse = FlashAttention.apply(q, k, v, float(scale), bool(causal), int(window), mask)
    return (o, lse) if return_lse else o


__all__ = ["FlashAttention", "flash_attention", "unsupported_reason", "FaError"]
