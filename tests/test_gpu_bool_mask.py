"""GPU parity of the boolean mask of the extended calls (fa_attn_desc_t
bool_mask; the binding sends torch.bool masks there) against the float64
oracle fed the numeric mask a logical one stands for (0 where allowed, -inf
elsewhere): broadcast, per-batch and per-head masks, fully blocked rows, with
the causal flag and windows, every dtype and head-dim bucket, the short-query
path, a value head dim other than D, and 4-byte and 1-byte mask loads. The
same pattern as a float32 0/-inf mask must give bit-identical results."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_06_amd as fa
import oracle
from parity_util import check_finite, gpu_inputs, rel_err, to_f64
from synth import TOL, decode, make_inputs

pytestmark = pytest.mark.gpu


def _allowed(shape, seed, blocked=0.25, dead_rows=()):
    rng = np.random.default_rng(seed)
    m = rng.random(shape) >= blocked
    for r in dead_rows:  # every key of these query rows blocked
        m[..., r, :] = False
    return m


def _run(t, mask, scale, causal, window):
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, causal, window, mask=mask)
    B, Hq, Lq, _ = t["q"].shape
    delta = torch.empty((B, Hq, Lq), device=o.device, dtype=torch.float32)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, causal, window, delta=delta, mask=mask)
    torch.cuda.synchronize()
    return {"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}


def _shape(kind, B, Hq, Lq, Lkv):
    return {"LK": (Lq, Lkv), "BHLK": (B, Hq, Lq, Lkv), "B1LK": (B, 1, Lq, Lkv), "1HLK": (1, Hq, Lq, Lkv),
            "HLK": (Hq, Lq, Lkv)}[kind]


CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mask shape, dead rows
    (1, 4, 2, 200, 200, 128, 128, "bf16", True, 0, "LK", ()),
    (2, 4, 4, 130, 131, 64, 64, "f16", False, 0, "BHLK", (5,)),
    (1, 2, 1, 70, 70, 32, 32, "f32", True, 20, "B1LK", ()),
    (1, 4, 1, 150, 152, 256, 256, "bf16", True, 64, "LK", (0, 77)),
    (1, 2, 1, 100, 100, 512, 512, "f16", False, 0, "1HLK", ()),
    (1, 8, 2, 12, 300, 128, 128, "bf16", True, 0, "HLK", ()),
    (2, 8, 4, 5, 97, 64, 64, "f16", False, 0, "BHLK", (2,)),
    (1, 4, 2, 96, 96, 64, 128, "bf16", False, 0, "LK", ()),
    (2, 8, 2, 257, 256, 128, 128, "f16", False, 33, "BHLK", ()),
]


@pytest.mark.parametrize("n", range(len(CASES)),
                         ids=["B{}_H{}:{}_L{}x{}_D{}v{}_{}_c{}_w{}_{}".format(*c[:11]) for c in CASES])
def test_bool_mask_parity(n):
    B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, kind, dead = CASES[n]
    scale = 1.0 / np.sqrt(D)
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 8400 + n, Dv=Dv)
    m = _allowed(_shape(kind, B, Hq, Lq, Lkv), 8500 + n, dead_rows=dead)
    bias = oracle.logical_mask_bias(m[None] if kind == "HLK" else m)
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, causal, window, bias=bias)
    got = to_f64(_run(gpu_inputs(x, dtype), torch.from_numpy(m).cuda(), scale, causal, window), dtype)
    check_finite(got, ref["LSE"])
    errs = {k: rel_err(got[k], ref[k]) for k in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    if dead:
        assert np.isneginf(got["LSE"][..., list(dead)]).all()


@pytest.mark.parametrize("Lkv", [160, 161])  # 4-byte loads / byte loads of the boolean mask
def test_bool_mask_equals_the_float_mask(Lkv):
    dtype, scale = "bf16", 1.0 / np.sqrt(128)
    x = make_inputs(2, 4, 2, 150, Lkv, 128, dtype, 8600 + Lkv)
    t = gpu_inputs(x, dtype)
    m = _allowed((2, 1, 150, Lkv), 8700, dead_rows=(9,))
    mb = torch.from_numpy(m).cuda()
    mf = torch.from_numpy(np.where(m, np.float32(0), np.float32(-np.inf))).cuda()
    a = _run(t, mb, scale, True, 40)
    b = _run(t, mf, scale, True, 40)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_bool_mask_autograd_node():
    from attention_fa_fwd_06_amd.autograd import flash_attention

    dtype, scale = "f16", 1.0 / np.sqrt(128)
    x = make_inputs(2, 8, 2, 100, 130, 128, dtype, 8800)
    m = _allowed((2, 8, 100, 130), 8801, dead_rows=(3,))
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, True, 0,
                          bias=oracle.logical_mask_bias(m))
    t = gpu_inputs(x, dtype)
    q, k, v = (t[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = flash_attention(q, k, v, scale, causal=True, mask=torch.from_numpy(m).cuda())
    o.backward(t["do"])
    got = to_f64({"O": o.detach(), "dQ": q.grad, "dK": k.grad, "dV": v.grad}, dtype)
    errs = {key: rel_err(got[key], ref[key]) for key in got}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
