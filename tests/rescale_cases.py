"""Inputs that make the forward's running maximum grow after the first key
tile a row visits, and the checks that say they do.

The forward keeps, per query row, a reference maximum m of the scores seen so
far and moves it (rescaling the partial output and row sum by 2^(m_old -
m_new)) only when a later tile's maximum exceeds m by more than 8 in log2
units (mlx-bun flash-attention.ts, forward shader, online-softmax update:
rescale = exp(m_i - m_new), l = rescale*l + sum p, o = rescale*o + sum p v;
here in base 2 and moved lazily). Inputs drawn as N(0, 1) almost never reach
that branch. These cases use synth.make_spiked_inputs: a flat score floor with
isolated keys about 9.4 log2 units higher, from key 100 on every 150 keys
(every W - 64 keys under a window of W). A row whose first
live tile holds no such key then sees its maximum jump by more than 8 at a
later tile, and the keys before the jump still carry a sizeable share of the
row's weight (about 0.0015 each against 1 for a high key), so a missing or
wrong rescale factor moves O and LSE far beyond the tolerance.

The checks run on the oracle's own scores (natural log, masked -inf),
converted to log2 units:
  * tiled kernels (key tiles of at most 64 keys, visited in key order): the
    first tile with an allowed key for row r holds no allowed key beyond
    a_r + 63 (a_r = the row's first allowed key), and every allowed key from
    a_r + 64 on lies in a later tile. So if some allowed key there scores
    more than 8 above the best allowed key in [a_r, a_r + 64), the branch is
    taken in that row, whatever the tile size and alignment.
  * short-query kernels (8 waves, wave w takes the 32-key blocks w, w + 8, ...
    from key 0 when there is no window, each with its own running maximum):
    the rule itself is replayed per wave on the oracle's scores.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from synth import decode, make_spiked_inputs

LOG2E = 1.0 / math.log(2.0)
THRESH = 8.0  # log2 units

# name, B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mask ("float", "bool" or None), path
CASES = [
    # 16-bit tiled kernels: every head-dim bucket (64, 128, 256, 512), both dtypes, masked and not
    ("bf16_d64_causal", 1, 4, 2, 400, 400, 64, 64, "bf16", True, 0, None, "tiled"),
    ("bf16_d64_window_fmask", 1, 4, 2, 700, 700, 64, 64, "bf16", True, 256, "float", "tiled"),
    ("bf16_d128_window", 2, 4, 2, 700, 700, 128, 128, "bf16", True, 256, None, "tiled"),
    ("bf16_d128_cross_bmask", 1, 4, 1, 200, 520, 128, 128, "bf16", False, 0, "bool", "tiled"),
    ("bf16_d256_causal", 1, 4, 2, 330, 330, 256, 256, "bf16", True, 0, None, "tiled"),
    ("bf16_d256_lq_gt_lkv_fmask", 1, 2, 1, 400, 300, 256, 256, "bf16", True, 0, "float", "tiled"),
    ("bf16_d512_cross", 1, 2, 1, 130, 400, 512, 512, "bf16", False, 0, None, "tiled"),
    ("bf16_d512_causal_bmask", 1, 2, 2, 350, 350, 512, 512, "bf16", True, 0, "bool", "tiled"),
    ("f16_d56_cross", 1, 4, 2, 100, 700, 56, 56, "f16", False, 0, None, "tiled"),
    ("f16_d64_causal_bmask", 1, 4, 4, 380, 380, 64, 64, "f16", True, 0, "bool", "tiled"),
    ("f16_d96_causal", 1, 8, 2, 420, 420, 96, 96, "f16", True, 0, None, "tiled"),
    ("f16_d128_window_dv64_fmask", 1, 4, 2, 800, 800, 128, 64, "f16", True, 300, "float", "tiled"),
    ("f16_d200_window", 1, 4, 2, 600, 600, 200, 200, "f16", True, 200, None, "tiled"),
    ("f16_d256_cross_bmask", 1, 2, 1, 300, 350, 256, 256, "f16", False, 0, "bool", "tiled"),
    ("f16_d392_causal", 1, 2, 1, 300, 300, 392, 392, "f16", True, 0, None, "tiled"),
    ("f16_d512_cross_fmask", 1, 2, 2, 150, 330, 512, 512, "f16", False, 0, "float", "tiled"),
    # float32 kernels: every bucket (32, 64, 96, 128, 256, 512), masked and not
    ("f32_d32_causal", 1, 2, 1, 350, 350, 32, 32, "f32", True, 0, None, "tiled"),
    ("f32_d32_cross_fmask", 1, 2, 2, 100, 400, 32, 32, "f32", False, 0, "float", "tiled"),
    ("f32_d64_window", 1, 2, 1, 600, 600, 64, 64, "f32", True, 200, None, "tiled"),
    ("f32_d64_causal_bmask", 1, 2, 2, 300, 300, 64, 64, "f32", True, 0, "bool", "tiled"),
    ("f32_d96_cross", 1, 2, 1, 120, 500, 96, 96, "f32", False, 0, None, "tiled"),
    ("f32_d80_causal_fmask", 1, 2, 1, 320, 320, 80, 80, "f32", True, 0, "float", "tiled"),
    ("f32_d128_causal", 1, 2, 2, 330, 330, 128, 128, "f32", True, 0, None, "tiled"),
    ("f32_d128_window_bmask", 1, 2, 1, 700, 700, 128, 128, "f32", True, 250, "bool", "tiled"),
    ("f32_d256_causal", 1, 2, 1, 300, 300, 256, 256, "f32", True, 0, None, "tiled"),
    ("f32_d256_cross_fmask", 1, 2, 2, 150, 380, 256, 256, "f32", False, 0, "float", "tiled"),
    ("f32_d512_causal", 1, 2, 1, 310, 310, 512, 512, "f32", True, 0, None, "tiled"),
    ("f32_d512_cross_bmask", 1, 2, 1, 100, 350, 512, 512, "f32", False, 0, "bool", "tiled"),
    # short-query kernels (query length <= 16): both buckets (64, 128), both dtypes, masked and not
    ("short_bf16_d64", 1, 8, 2, 8, 1500, 64, 64, "bf16", False, 0, None, "short"),
    ("short_bf16_d64_fmask", 2, 4, 2, 4, 900, 64, 64, "bf16", False, 0, "float", "short"),
    ("short_bf16_d128", 1, 32, 4, 1, 2000, 128, 128, "bf16", False, 0, None, "short"),
    ("short_bf16_d128_bmask", 1, 8, 4, 16, 1200, 128, 128, "bf16", False, 0, "bool", "short"),
    ("short_f16_d64", 1, 4, 1, 16, 700, 64, 64, "f16", False, 0, None, "short"),
    ("short_f16_d48_bmask", 1, 6, 2, 7, 1100, 48, 48, "f16", False, 0, "bool", "short"),
    ("short_f16_d128_dv96", 1, 8, 2, 8, 1300, 128, 96, "f16", False, 0, None, "short"),
    ("short_f16_d128_fmask", 1, 4, 4, 3, 800, 128, 128, "f16", False, 0, "float", "short"),
]

# fraction of query rows (over every batch and head) in which the branch must be taken
MIN_FRACTION = 0.5


def case_inputs(n: int):
    """Storage arrays and mask (None, float32 or bool array of shape [Lq, Lkv]) of case n."""
    name, B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mask, path = CASES[n]
    # high keys from key 100 on (past any first tile of a row that starts at key
    # 0), every 150 keys; under a window of W keys every W - 64 keys, so that
    # every window holds one past its first 64 keys and most hold none among those
    period = 150 if window == 0 else window - 64
    x = make_spiked_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 31000 + n, period=period, offset=100, Dv=Dv)
    rng = np.random.default_rng(31500 + n)
    m = None
    if mask == "float":
        m = (rng.standard_normal((Lq, Lkv)) * 0.1).astype(np.float32)
        m[rng.random((Lq, Lkv)) < 0.1] = -np.inf
    elif mask == "bool":
        m = rng.random((Lq, Lkv)) >= 0.1
    return x, m


def scores_log2(x, dtype, scale, causal, window, mask):
    """The oracle's scaled, masked scores [B, Hq, Lq, Lkv] in log2 units (-inf where not allowed)."""
    q, k, v = (decode(x[n], dtype) for n in ("q", "k", "v"))
    B, Hq, Lq, _ = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    bias = None
    if mask is not None:
        bias = oracle.logical_mask_bias(mask) if mask.dtype == np.bool_ else mask.astype(np.float64)
    out = np.empty((B, Hq, Lq, Lkv))
    rows = np.arange(Lq)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            S, _, _, _ = oracle.rows_forward(q[b, h], k[b, g], v[b, g], rows, scale, causal, window, bias_rows=bias)
            out[b, h] = S * LOG2E
    return out


def tiled_rows_taking_branch(S2, span=64):
    """Boolean [.., Lq]: rows with an allowed key at or past a_r + span scoring more
    than THRESH above every allowed key in [a_r, a_r + span)."""
    flat = S2.reshape(-1, S2.shape[-1])
    res = np.zeros(flat.shape[0], dtype=bool)
    for n, row in enumerate(flat):
        ok = np.nonzero(np.isfinite(row))[0]
        if len(ok) == 0:
            continue
        a = ok[0]
        first = row[a:a + span].max()
        later = row[a + span:].max() if a + span < len(row) else -np.inf
        res[n] = later > first + THRESH
    return res.reshape(S2.shape[:-1])


def short_rows_taking_branch(S2, waves=8, block=32):
    """Boolean [.., Lq]: rows in which at least one wave's replayed running maximum
    (blocks w, w + waves, ... from key 0) moves from a finite value."""
    flat = S2.reshape(-1, S2.shape[-1])
    nblk = (flat.shape[1] + block - 1) // block
    res = np.zeros(flat.shape[0], dtype=bool)
    for n, row in enumerate(flat):
        for w in range(waves):
            m = -np.inf
            for blk in range(w, nblk, waves):
                t = row[blk * block:(blk + 1) * block].max()
                if t > m + THRESH:
                    if np.isfinite(m):
                        res[n] = True
                    m = t
    return res.reshape(S2.shape[:-1])


def branch_fraction(n: int, x=None, mask=None) -> float:
    """Fraction of the case's query rows in which the forward's rescale branch is taken."""
    name, B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mk, path = CASES[n]
    if x is None:
        x, mask = case_inputs(n)
    S2 = scores_log2(x, dtype, 1.0 / math.sqrt(D), causal, window, mask)
    taken = tiled_rows_taking_branch(S2) if path == "tiled" else short_rows_taking_branch(S2)
    return float(taken.mean())
