"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: max|gpu - ref| / max|ref| <= 1e-5 (fp32), 5e-3 (fp16), 2e-2 (bf16) for
O, LSE, Delta, dQ, dK and dV; no NaN; -inf LSE exactly where the reference
has a row with no allowed key.

Workload sizes: the two small workloads are compared whole; the 2048-token
workload is run whole on the GPU and compared whole on two (batch, kv-group)
slices; the 8192- and 32768-token workloads are run whole in the launch
configuration the benchmark times and compared on sampled rows and keys
(the oracle computes those one by one), plus identities that hold at any size.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from parity_util import check_finite, compare_full, gpu_inputs, rel_err, run_gpu, to_f64
from synth import TOL, WORKLOADS, decode, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu


def _w(i):
    return WORKLOADS[i]


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_workload_tiny_f32():
    w = _w(0)
    compare_full(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.D, w.dtype, w.causal, w.window, w.seed, w.sigma_qkv, w.sigma_do)


def test_workload_f16_causal_mha():
    w = _w(1)
    compare_full(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.D, w.dtype, w.causal, w.window, w.seed, w.sigma_qkv, w.sigma_do)


def _slice_check(w, x, got, groups):
    reps = w.Hq // w.Hkv
    for b, g in groups:
        hs = slice(g * reps, (g + 1) * reps)
        sub = [decode(x["q"][b:b + 1, hs], w.dtype), decode(x["k"][b:b + 1, g:g + 1], w.dtype),
               decode(x["v"][b:b + 1, g:g + 1], w.dtype), decode(x["do"][b:b + 1, hs], w.dtype)]
        ref = oracle.backward(*sub, w.scale, w.causal, w.window)
        errs = {
            "O": rel_err(got["O"][b:b + 1, hs], ref["O"]),
            "LSE": rel_err(got["LSE"][b:b + 1, hs], ref["LSE"]),
            "Delta": rel_err(got["Delta"][b:b + 1, hs], ref["Delta"]),
            "dQ": rel_err(got["dQ"][b:b + 1, hs], ref["dQ"]),
            "dK": rel_err(got["dK"][b:b + 1, g:g + 1], ref["dK"]),
            "dV": rel_err(got["dV"][b:b + 1, g:g + 1], ref["dV"]),
        }
        assert all(v <= w.tol for v in errs.values()), (b, g, errs)


def test_workload_bf16_gqa4_L2048():
    w = _w(2)
    x = workload_inputs(w)
    got = to_f64(run_gpu(gpu_inputs(x, w.dtype), w.scale, w.causal, w.window), w.dtype)
    check_finite(got)
    _slice_check(w, x, got, [(0, 0), (3, 7), (1, 4)])


def _sampled_check(w, x, got, heads, rows, kv_groups, keys):
    q, k, v, do = (decode(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    for b, h in heads:
        ref = oracle.sample_rows(q, k, v, do, w.scale, w.causal, w.window, b, h, rows)
        for key in ("O", "LSE", "Delta", "dQ"):
            e = rel_err(got[key][b, h, rows], ref[key])
            assert e <= w.tol, (key, b, h, e)
    for b, g in kv_groups:
        ref = oracle.sample_keys(q, k, v, do, w.scale, w.causal, w.window, b, g, keys)
        for key in ("dK", "dV"):
            e = rel_err(got[key][b, g, keys], ref[key])
            assert e <= w.tol, (key, b, g, e)


def _identities(w, x, got):
    """Identities of the exact gradient, checked on whole tensors:
    sum_j dK[b,g,j,:] = 0 (softmax shift invariance) and
    sum_j dV[b,g,j,:] = sum_{h in g} sum_i dO[b,h,i,:] (rows of P sum to 1)."""
    reps = w.Hq // w.Hkv
    do = decode(x["do"], w.dtype)
    for b in range(w.B):
        for g in range(w.Hkv):
            dk, dv = got["dK"][b, g], got["dV"][b, g]
            assert np.abs(dk.sum(axis=0)).max() <= 1e-2 * np.abs(dk).sum(axis=0).max()
            want = do[b, g * reps:(g + 1) * reps].sum(axis=(0, 1))
            assert np.abs(dv.sum(axis=0) - want).max() <= 1e-2 * np.abs(want).max()


def test_workload_bf16_gqa8_window1024_L8192_D256():
    w = _w(3)
    x = workload_inputs(w)
    got = to_f64(run_gpu(gpu_inputs(x, w.dtype), w.scale, w.causal, w.window), w.dtype)
    check_finite(got)
    rows = [0, 1, 31, 32, 63, 64, 127, 1000, 1023, 1024, 1025, 1056, 2047, 4097, 8000, 8190, 8191]
    _sampled_check(w, x, got, [(0, 0), (0, 7), (0, 8), (0, 15)], rows, [], [])
    # dK/dV element-wise on whole 64-key blocks (one dK/dV workgroup each) at the
    # start, around the first window length, in the middle and at the end of the
    # sequence, plus scattered keys, for both kv groups; each key from every query
    # row of the group's eight heads that may attend it (the oracle's row-blocked
    # key gradients)
    keys = np.concatenate([np.arange(0, 64), np.arange(960, 1088), np.arange(4096, 4160), np.arange(8128, 8192),
                           [3000, 5555, 7167, 7168]])
    q, k, v, do = (decode(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    workers = min(16, len(os.sched_getaffinity(0)))
    for g in (0, 1):
        ref = oracle.key_grads(q, k, v, do, w.scale, w.causal, w.window, 0, g, keys, workers=workers)
        for key in ("dK", "dV"):
            e = rel_err(got[key][0, g, keys], ref[key])
            assert e <= w.tol, (key, g, e)
    _identities(w, x, got)


def test_workload_bf16_gqa8_L32768():
    w = _w(4)
    x = workload_inputs(w)
    got = to_f64(run_gpu(gpu_inputs(x, w.dtype), w.scale, w.causal, w.window), w.dtype)
    check_finite(got)
    rows = [0, 1, 127, 128, 4095, 16383, 16384, 30001, 32767]
    _sampled_check(w, x, got, [(0, 0), (0, 13), (0, 31)], rows, [], [])
    # dK/dV element-wise over the whole key range of two kv groups: the first,
    # middle and last 128-key blocks whole (under the causal key-block pairing
    # the middle two are one workgroup's pair, the first and last another's),
    # plus keys scattered in between; each from every query row of the group's
    # eight heads (the oracle's row-blocked key gradients)
    keys = np.concatenate([np.arange(0, 128), np.arange(16256, 16512), np.arange(32640, 32768),
                           [1000, 4095, 4096, 8191, 8192, 12345, 20000, 24575, 24576, 30000]])
    q, k, v, do = (decode(x[n], w.dtype) for n in ("q", "k", "v", "do"))
    workers = min(16, len(os.sched_getaffinity(0)))
    for g in (0, 3):
        ref = oracle.key_grads(q, k, v, do, w.scale, w.causal, w.window, 0, g, keys, workers=workers)
        for key in ("dK", "dV"):
            e = rel_err(got[key][0, g, keys], ref[key])
            assert e <= w.tol, (key, g, e)
    _identities(w, x, got)


# ---------------------------------------------------------------------------
# shape / dtype / mask sweep (the pages' VJP test matrix: short and long L,
# head dims 32..512, GQA 1:1 .. 16:1 and MQA, three dtypes, causal or not,
# windows, batch > 1, Lq != Lkv)
# ---------------------------------------------------------------------------

SWEEP = [
    # B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window
    (1, 2, 2, 1, 1, 64, "bf16", False, 0),
    (1, 4, 1, 1, 1, 128, "f16", True, 0),
    (2, 4, 2, 7, 7, 32, "f32", True, 0),
    (1, 4, 2, 8, 8, 64, "f16", False, 0),
    (3, 2, 2, 16, 16, 96, "bf16", True, 0),
    (1, 8, 2, 33, 33, 128, "bf16", True, 0),
    (1, 16, 1, 128, 128, 64, "f16", True, 0),
    (2, 8, 8, 256, 256, 128, "bf16", False, 0),
    (1, 4, 1, 300, 300, 128, "bf16", True, 37),
    (1, 2, 2, 1000, 1000, 64, "f16", True, 128),
    (1, 4, 2, 300, 300, 256, "bf16", True, 0),
    (1, 2, 1, 200, 200, 256, "f16", False, 0),
    (1, 2, 1, 100, 100, 512, "bf16", True, 0),
    (1, 2, 2, 77, 77, 512, "f16", False, 0),
    (1, 2, 1, 130, 130, 256, "f32", True, 0),
    (1, 2, 2, 70, 70, 96, "f32", False, 0),
    (1, 4, 4, 64, 64, 128, "f32", True, 16),
    (2, 4, 2, 129, 129, 40, "bf16", True, 0),
    (1, 2, 1, 65, 65, 72, "f16", True, 0),
    (1, 2, 2, 100, 100, 200, "bf16", True, 0),
    (1, 4, 2, 50, 50, 264, "bf16", False, 0),
    (1, 4, 2, 300, 300, 64, "bf16", True, 1),
    (1, 4, 2, 300, 300, 64, "f16", True, 1024),
    (1, 4, 2, 300, 300, 64, "bf16", False, 37),
    (1, 4, 2, 100, 300, 64, "bf16", True, 0),
    (1, 4, 2, 300, 100, 64, "f16", True, 0),
    (1, 4, 2, 300, 100, 64, "bf16", True, 30),
    (1, 4, 2, 64, 200, 128, "bf16", False, 0),
    (2, 4, 1, 50, 90, 32, "f32", False, 0),
    (1, 16, 16, 17, 17, 64, "bf16", False, 0),
    # d split over two waves in dK/dV (head dims 136..256): window, ragged, Lq != Lkv
    (1, 4, 1, 333, 333, 256, "bf16", True, 100),
    (1, 2, 2, 150, 260, 248, "f16", True, 40),
    (1, 8, 2, 96, 96, 256, "f16", True, 0),
    (2, 2, 1, 70, 45, 136, "bf16", False, 0),
    # float in the 512 bucket (d in four slices, no transposed copies in the backward)
    (1, 2, 1, 100, 100, 512, "f32", True, 0),
    (1, 4, 2, 70, 90, 264, "f32", False, 0),
    (1, 2, 2, 130, 130, 512, "f32", True, 50),
    (2, 2, 1, 33, 20, 392, "f32", True, 0),
    # the 256 bucket's role-split dK/dV and dQ kernels at degenerate sizes: one
    # token, a few rows over many keys (under the causal mask most key blocks
    # see no row), window 1, Lq > Lkv, one and two tiles
    (1, 4, 2, 1, 1, 256, "bf16", True, 0),
    (1, 4, 2, 5, 300, 256, "bf16", False, 0),
    (1, 4, 2, 5, 300, 256, "f16", True, 0),
    (2, 8, 1, 40, 40, 256, "bf16", True, 1),
    (1, 2, 1, 300, 90, 256, "bf16", True, 0),
    (1, 2, 2, 64, 64, 256, "bf16", False, 0),
    (1, 2, 2, 33, 33, 256, "f16", True, 0),
]


@pytest.mark.parametrize("n", range(len(SWEEP)), ids=["B{}_H{}:{}_L{}x{}_D{}_{}_c{}_w{}".format(*c) for c in SWEEP])
def test_sweep(n):
    B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window = SWEEP[n]
    compare_full(B, Hq, Hkv, Lq, Lkv, D, dtype, causal, window, seed=100 + n)


def test_fully_masked_first_tile_rows():
    # window 1 over 300 rows with 64-key tiles: every row's first visited tile
    # is fully masked for most rows of a 128-row query tile
    compare_full(1, 2, 1, 300, 300, 128, "bf16", True, 1, seed=21)


def test_rows_without_any_key():
    # Lq > Lkv, causal + window: rows 40.. have no allowed key -> O = 0, LSE = -inf
    B, Hq, Hkv, Lq, Lkv, D = 1, 4, 2, 100, 40, 64
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, "bf16", 22)
    got = to_f64(run_gpu(gpu_inputs(x, "bf16"), 0.125, True, 3), "bf16")
    assert np.all(got["O"][:, :, 42:] == 0)
    assert np.all(np.isneginf(got["LSE"][:, :, 42:]))
    assert np.all(got["dQ"][:, :, 42:] == 0)
    compare_full(B, Hq, Hkv, Lq, Lkv, D, "bf16", True, 3, seed=22)


def test_scale_other_than_default():
    compare_full(1, 4, 2, 100, 100, 64, "f16", True, 0, seed=23, scale=0.05)
    compare_full(1, 4, 2, 100, 100, 64, "bf16", False, 0, seed=24, scale=0.3)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_zero_and_negative_scale(scale):
    # scale 0: every allowed key gets the same weight (O is the mean of the
    # allowed V rows); a negative scale is folded into Q. Tiled and
    # short-query paths, causal with a window, ragged lengths.
    compare_full(1, 4, 2, 150, 150, 128, "bf16", True, 40, seed=26, scale=scale)
    compare_full(2, 2, 1, 90, 70, 64, "f16", False, 0, seed=27, scale=scale)
    compare_full(1, 8, 2, 5, 300, 128, "bf16", True, 0, seed=28, scale=scale)
    compare_full(1, 2, 2, 40, 40, 32, "f32", True, 7, seed=29, scale=scale)


@pytest.mark.parametrize("B,Hq,Hkv,L,D,dtype", [(8, 16, 8, 850, 128, "bf16"), (8, 8, 8, 1100, 64, "f16"),
                                                 (8, 8, 8, 420, 256, "bf16")])
def test_causal_key_block_pairing_with_odd_block_count(B, Hq, Hkv, L, D, dtype):
    # Under a causal mask without window the dK/dV workgroups take key blocks p
    # and nkt-1-p when that still leaves 256 workgroups. Here the number of key
    # blocks (128 keys, 64 at D = 256) is odd (7, 9, 7), so the middle block runs
    # alone, and the last block is ragged.
    compare_full(B, Hq, Hkv, L, L, D, dtype, True, 0, seed=30 + D)


def test_deterministic():
    x = make_inputs(1, 8, 2, 300, 300, 128, "bf16", 25)
    t = gpu_inputs(x, "bf16")
    a = run_gpu(t, 0.088, True, 0)
    b = run_gpu(t, 0.088, True, 0)
    for key in a:
        bits = torch.int32 if a[key].element_size() == 4 else torch.int16
        assert torch.equal(a[key].view(bits), b[key].view(bits)), key
