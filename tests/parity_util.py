"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
on seeded inputs and compare with the float64 oracle on the same stored values.

Metric (per output tensor): max|gpu - ref| / max|ref|, computed over finite
reference entries; entries where the reference LSE is -inf (rows with no
allowed key) must be exactly -inf on the GPU too.
"""
from __future__ import annotations

import numpy as np
import torch

import attention_fa_fwd_06_amd as fa
import oracle
from synth import TOL, decode, from_torch, make_inputs, to_torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    fin = np.isfinite(ref)
    if not fin.any():
        return 0.0
    den = np.abs(ref[fin]).max()
    num = np.abs(got[fin] - ref[fin]).max()
    if den == 0:
        return float(num)
    return float(num / den)


def gpu_inputs(x: dict, dtype: str, device="cuda"):
    return {k: to_torch(v, dtype).to(device) for k, v in x.items()}


def run_gpu(t: dict, scale: float, causal: bool, window: int):
    """fa_fwd -> fa_bwd_preprocess -> fa_bwd_dkv -> fa_bwd_dq on one stream."""
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = fa.forward(q, k, v, scale, causal, window)
    B, Hq, Lq, D = q.shape
    delta = torch.empty((B, Hq, Lq), device=q.device, dtype=torch.float32)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale, causal, window, delta=delta)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}


def to_f64(out: dict, dtype: str) -> dict:
    r = {}
    for key, val in out.items():
        if key in ("LSE", "Delta"):
            r[key] = val.detach().cpu().to(torch.float64).numpy()
        else:
            r[key] = from_torch(val, dtype)
    return r


def check_finite(out: dict, ref_lse: np.ndarray | None = None):
    """No NaN anywhere; no inf except LSE = -inf on rows with no allowed key."""
    for key, val in out.items():
        if key == "LSE":
            bad = np.isnan(val) | np.isposinf(val)
            assert not bad.any(), f"{key} has NaN/+inf"
            if ref_lse is not None:
                assert np.array_equal(np.isneginf(val), np.isneginf(ref_lse)), "LSE -inf pattern differs"
        else:
            assert np.isfinite(val).all(), f"{key} has NaN/inf"


def compare_full(B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window, seed, sigma_qkv=1.0, sigma_do=1.0, tol=None,
                 scale=None):
    """Whole-tensor parity of all six outputs. Returns the error dict."""
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, seed, sigma_qkv, sigma_do)
    ref = oracle.backward(*(decode(x[n], dtype) for n in ("q", "k", "v", "do")), scale, causal, window)
    got = to_f64(run_gpu(gpu_inputs(x, dtype), scale, causal, window), dtype)
    check_finite(got, ref["LSE"])
    tol = TOL[dtype] if tol is None else tol
    errs = {key: rel_err(got[key], ref[key]) for key in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"parity above {tol}: {bad} (all: {errs})"
    return errs


def run_gpu_masked(t: dict, scale: float, causal: bool, window: int, mask=None):
    """The four calls with an optional mask tensor (float32 additive or bool)."""
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o, lse = fa.forward(q, k, v, scale, causal, window, mask=mask)
    B, Hq, Lq, _ = q.shape
    delta = torch.empty((B, Hq, Lq), device=q.device, dtype=torch.float32)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale, causal, window, delta=delta, mask=mask)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}


def compare_given(x: dict, dtype: str, scale: float, causal: bool, window: int, mask=None, tol=None):
    """Whole-tensor parity of all six outputs on the given storage arrays.

    mask: None, a float32 array (additive: 0 attends, -inf blocks) or a bool
    array (True attends), broadcastable to [B, Hq, Lq, Lkv]. Returns the errors."""
    bias = None
    if mask is not None:
        bias = oracle.logical_mask_bias(mask) if mask.dtype == np.bool_ else mask.astype(np.float64)
    ref = oracle.backward(*(decode(x[n], dtype) for n in ("q", "k", "v", "do")), scale, causal, window, bias=bias)
    mt = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    got = to_f64(run_gpu_masked(gpu_inputs(x, dtype), scale, causal, window, mt), dtype)
    check_finite(got, ref["LSE"])
    tol = TOL[dtype] if tol is None else tol
    errs = {key: rel_err(got[key], ref[key]) for key in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"parity above {tol}: {bad} (all: {errs})"
    return errs
