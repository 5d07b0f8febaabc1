"""GPU parity of the masked entry points (fa_fwd_masked, fa_bwd_dkv_masked,
fa_bwd_dq_masked) against the float64 oracle's additive mask, on seeded
inputs: broadcast, per-batch and per-head masks, -inf blocks and fully
blocked rows, combined with the causal flag and windows, every dtype and
head-dim bucket, 16-byte and 4-byte mask loads."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_06_amd as fa
import oracle
from parity_util import check_finite, gpu_inputs, rel_err, to_f64
from synth import TOL, decode, make_inputs

pytestmark = pytest.mark.gpu


def _mask(shape, seed, blocked=0.2, dead_rows=()):
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal(shape) * 1.5).astype(np.float32)
    m[rng.random(shape) < blocked] = -np.inf
    for r in dead_rows:  # every key of these query rows blocked
        m[..., r, :] = -np.inf
    return m


def _run(t, mask, scale, causal, window):
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, causal, window, mask=mask)
    B, Hq, Lq, _ = t["q"].shape
    delta = torch.empty((B, Hq, Lq), device=o.device, dtype=torch.float32)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, causal, window, delta=delta, mask=mask)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}


CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window, mask shape, dead rows
    (1, 4, 2, 200, 200, 128, "bf16", True, 0, "LK", ()),
    (2, 4, 4, 130, 131, 64, "f16", False, 0, "BHLK", (5,)),
    (1, 2, 1, 70, 70, 32, "f32", True, 20, "B1LK", ()),
    (1, 4, 1, 150, 150, 256, "bf16", True, 64, "LK", (0, 77)),
    (1, 2, 1, 100, 100, 512, "f16", False, 0, "1HLK", ()),
    (1, 4, 2, 100, 300, 96, "bf16", True, 0, "HLK", ()),
    (1, 2, 2, 64, 96, 256, "f32", False, 0, "LK", (3,)),
    (2, 8, 2, 257, 257, 128, "f16", False, 33, "BHLK", ()),
    (1, 4, 4, 96, 96, 64, "bf16", False, 0, "LK", ()),
    (1, 2, 1, 90, 90, 512, "f32", True, 30, "LK", (4,)),
]


def _shape(kind, B, Hq, Lq, Lkv):
    return {"LK": (Lq, Lkv), "BHLK": (B, Hq, Lq, Lkv), "B1LK": (B, 1, Lq, Lkv), "1HLK": (1, Hq, Lq, Lkv),
            "HLK": (Hq, Lq, Lkv)}[kind]


@pytest.mark.parametrize("n", range(len(CASES)),
                         ids=["B{}_H{}:{}_L{}x{}_D{}_{}_c{}_w{}_{}".format(*c[:10]) for c in CASES])
def test_masked_parity(n):
    B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window, kind, dead = CASES[n]
    scale = 1.0 / np.sqrt(D)
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 8000 + n)
    m = _mask(_shape(kind, B, Hq, Lq, Lkv), 8100 + n, dead_rows=dead)
    if kind == "HLK":  # [Hq, Lq, Lkv] broadcasts against [B, Hq] like torch
        bias = m[None]
    else:
        bias = m
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, causal, window,
                          bias=bias.astype(np.float64))
    got = to_f64(_run(gpu_inputs(x, dtype), torch.from_numpy(m).cuda(), scale, causal, window), dtype)
    check_finite(got, ref["LSE"])
    errs = {k: rel_err(got[k], ref[k]) for k in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    if dead:
        assert np.isneginf(got["LSE"][..., list(dead)]).all()


def test_zero_mask_matches_the_unmasked_calls():
    dtype, scale = "bf16", 1.0 / np.sqrt(128)
    x = make_inputs(1, 4, 2, 180, 180, 128, dtype, 8200)
    t = gpu_inputs(x, dtype)
    zero = torch.zeros(180, 180, device="cuda")
    a = to_f64(_run(t, zero, scale, True, 0), dtype)
    b = to_f64(_run(t, None, scale, True, 0), dtype)
    for key in a:
        assert rel_err(a[key], b[key]) <= 1e-3, key


def test_causal_shaped_mask_matches_the_causal_flag():
    dtype, scale = "f16", 0.125
    x = make_inputs(1, 2, 1, 140, 140, 64, dtype, 8201)
    t = gpu_inputs(x, dtype)
    tri = torch.tril(torch.ones(140, 140, dtype=torch.bool, device="cuda"))
    m = torch.where(tri, 0.0, float("-inf")).float()
    a = to_f64(_run(t, m, scale, False, 0), dtype)
    b = to_f64(_run(t, None, scale, True, 0), dtype)
    for key in a:
        assert rel_err(a[key], b[key]) <= TOL[dtype], key


def test_masked_autograd_node():
    from attention_fa_fwd_06_amd.autograd import flash_attention

    dtype, scale = "bf16", 1.0 / np.sqrt(64)
    x = make_inputs(1, 4, 2, 120, 120, 64, dtype, 8202)
    m = _mask((120, 120), 8203)
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, False, 0,
                          bias=m.astype(np.float64))
    t = gpu_inputs(x, dtype)
    q, k, v = (t[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = flash_attention(q, k, v, scale, mask=torch.from_numpy(m).cuda())
    o.backward(t["do"])
    got = to_f64({"O": o.detach(), "dQ": q.grad, "dK": k.grad, "dV": v.grad}, dtype)
    errs = {key: rel_err(got[key], ref[key]) for key in got}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
