"""GPU parity of the short-query path (query length <= 16, both head dims <=
128, 16-bit inputs: the MLX VJP pull request's vector path for short
sequences, here packed GQA rows with an in-workgroup key split) against the
float64 oracle, on seeded inputs, through the same C ABI calls as every other
shape.

The cases cover query lengths 1, 4, 7, 8 and 16 (the pull request's short
lengths plus the largest one routed here), key lengths from 1 to a few
thousand with ragged tails, MHA, GQA and MQA with packed tiles that span
several heads, every row-tile size the host picks (from one row to 32),
causal masks, windows, additive masks that differ per head (rows of one
packed tile read different mask heads), rows with no allowed key, and a value
head dim different from D."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_06_amd as fa
import oracle
from parity_util import check_finite, gpu_inputs, rel_err, to_f64
from synth import TOL, decode, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mask shape (None: no mask)
    (1, 1, 1, 1, 1, 64, 64, "bf16", False, 0, None),
    (2, 8, 2, 4, 300, 64, 64, "f16", False, 0, None),
    (1, 32, 4, 8, 1100, 128, 128, "bf16", False, 0, None),
    (3, 6, 3, 7, 37, 80, 80, "f16", True, 0, None),
    (2, 4, 1, 16, 500, 128, 64, "bf16", True, 5, None),
    (1, 16, 1, 8, 777, 32, 32, "bf16", False, 100, None),
    (2, 8, 8, 1, 2000, 128, 128, "f16", False, 0, "1HLK"),
    (1, 8, 2, 7, 7, 64, 128, "bf16", True, 0, "B1LK"),
    (64, 8, 8, 2, 129, 64, 64, "bf16", False, 0, None),
    (4, 32, 8, 16, 64, 128, 128, "bf16", True, 0, None),
    (1, 4, 2, 16, 4, 64, 64, "f16", True, 2, None),
    (2, 16, 2, 8, 4100, 128, 128, "bf16", False, 0, "LK"),
    (1, 12, 4, 3, 250, 96, 48, "f16", False, 17, "BHLK"),
]


def _shape(kind, B, Hq, Lq, Lkv):
    return {"LK": (Lq, Lkv), "BHLK": (B, Hq, Lq, Lkv), "B1LK": (B, 1, Lq, Lkv), "1HLK": (1, Hq, Lq, Lkv)}[kind]


def _mask(shape, seed):
    # scores shifted by up to about +-6 (some large positive entries), a fifth
    # of the pairs blocked and, with more than one query row, the first row
    # with every key blocked
    rng = np.random.default_rng(seed)
    m = (rng.standard_normal(shape) * 2.0).astype(np.float32)
    m[rng.random(shape) < 0.2] = -np.inf
    if shape[-2] > 1:
        m[..., 0, :] = -np.inf
    return m


@pytest.mark.parametrize("n", range(len(CASES)),
                         ids=["B{}_H{}:{}_L{}x{}_D{}_Dv{}_{}_c{}_w{}_{}".format(*c) for c in CASES])
def test_short_query_parity(n):
    B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, kind = CASES[n]
    scale = 1.0 / np.sqrt(D)
    print(f"short case {n}: {CASES[n]}", flush=True)
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 12000 + n, Dv=Dv)
    bias = None if kind is None else _mask(_shape(kind, B, Hq, Lq, Lkv), 12100 + n)
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, causal, window,
                          bias=None if bias is None else bias.astype(np.float64))
    t = gpu_inputs(x, dtype)
    mask = None if bias is None else torch.from_numpy(bias).cuda()
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, causal, window, mask=mask)
    delta = torch.empty((B, Hq, Lq), device="cuda", dtype=torch.float32)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, causal, window, delta=delta, mask=mask)
    torch.cuda.synchronize()
    got = to_f64({"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}, dtype)
    check_finite(got, ref["LSE"])
    errs = {k: rel_err(got[k], ref[k]) for k in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
    if kind is not None and Lq > 1:
        # the fully blocked row: O = 0, dQ = 0
        assert not got["O"][..., 0, :].any() and not got["dQ"][..., 0, :].any()


def test_short_path_is_deterministic():
    """Two runs of the same short-query step give identical bits (the merge of
    the waves' partial results adds them in a fixed order)."""
    x = make_inputs(2, 16, 2, 8, 1500, 128, "bf16", 12500)
    t = gpu_inputs(x, "bf16")
    outs = []
    for _ in range(2):
        o, lse = fa.forward(t["q"], t["k"], t["v"], 0.1, False, 0)
        dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], 0.1, False, 0)
        torch.cuda.synchronize()
        outs.append([z.clone() for z in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("Lq", [16, 17])
def test_short_and_tiled_sides_of_the_boundary(Lq):
    """Lq = 16 runs the short-query kernels and Lq = 17 the tiled ones; both
    meet the oracle on the same shape otherwise."""
    B, Hq, Hkv, Lkv, D, dtype = 2, 8, 2, 600, 128, "bf16"
    scale = 1.0 / np.sqrt(D)
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 12600 + Lq)
    ref = oracle.backward(*(decode(x[k], dtype) for k in ("q", "k", "v", "do")), scale, True, 0)
    t = gpu_inputs(x, dtype)
    o, lse = fa.forward(t["q"], t["k"], t["v"], scale, True, 0)
    delta = torch.empty((B, Hq, Lq), device="cuda", dtype=torch.float32)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, lse, t["do"], scale, True, 0, delta=delta)
    torch.cuda.synchronize()
    got = to_f64({"O": o, "LSE": lse, "Delta": delta, "dQ": dq, "dK": dk, "dV": dv}, dtype)
    check_finite(got, ref["LSE"])
    errs = {k: rel_err(got[k], ref[k]) for k in ("O", "LSE", "Delta", "dQ", "dK", "dV")}
    assert all(e <= TOL[dtype] for e in errs.values()), errs
