"""CPU checks of the inputs that drive the forward's lazy online-softmax
rescale (tests/rescale_cases.py): every case takes the branch in most query
rows, and the inputs tell a right rescale factor from a dropped or wrong one.

The second check replays a tiled online softmax with the lazy rule in NumPy
(key tiles of 32 or 64 keys in key order, the reference maximum moved only
past 8 log2 units, the partial output and row sum rescaled by 2^(m_old -
m_new)) on the oracle's scores. With that factor it reproduces the oracle's
O; with the factor dropped, or taken as e^(m_old - m_new), it misses O by
more than the dtype's parity tolerance, so a GPU kernel with either mistake
fails the GPU cases built from the same inputs."""
import math

import numpy as np
import pytest

import oracle
import rescale_cases as rc
from synth import TOL, decode


@pytest.mark.parametrize("n", range(len(rc.CASES)), ids=[c[0] for c in rc.CASES])
def test_case_takes_the_rescale_branch(n):
    assert rc.branch_fraction(n) >= rc.MIN_FRACTION


def _replay(S2, V, tile, factor):
    """O of the rows of one (batch, head) from scores S2 (log2 units) by a tiled
    online softmax with the lazy rule; factor(m_old, m_new) rescales."""
    Lq, Lkv = S2.shape
    O = np.zeros((Lq, V.shape[1]))
    for i in range(Lq):
        m, l, o = -np.inf, 0.0, np.zeros(V.shape[1])
        for t0 in range(0, Lkv, tile):
            s = S2[i, t0:t0 + tile]
            mt = s.max()
            if mt > m + rc.THRESH:
                a = factor(m, mt) if np.isfinite(m) else 0.0
                l, o, m = l * a, o * a, mt
            p = np.exp2(s - (m if np.isfinite(m) else 0.0))
            l += p.sum()
            o += p @ V[t0:t0 + tile]
        O[i] = o / l if l > 0 else 0.0
    return O


@pytest.mark.parametrize("n", [0, 1, 6, 8, 12, 20, 27], ids=lambda n: rc.CASES[n][0])
@pytest.mark.parametrize("tile", [32, 64])
def test_inputs_tell_a_wrong_rescale_from_the_right_one(n, tile):
    name, B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mk, path = rc.CASES[n]
    x, mask = rc.case_inputs(n)
    scale = 1.0 / math.sqrt(D)
    S2 = rc.scores_log2(x, dtype, scale, causal, window, mask)[0, 0]
    q, k, v = (decode(x[name], dtype)[:1, :1] for name in ("q", "k", "v"))  # batch 0, head 0 (kv head 0)
    bias = None if mask is None else oracle.logical_mask_bias(mask) if mask.dtype == np.bool_ else mask
    ref = oracle.forward(q, k, v, scale, causal, window, bias=bias)[0][0, 0]
    v = v[0, 0]

    def err(O):
        return np.abs(O - ref).max() / np.abs(ref).max()

    assert err(_replay(S2, v, tile, lambda m0, m1: 2.0 ** (m0 - m1))) < 1e-12
    assert err(_replay(S2, v, tile, lambda m0, m1: 1.0)) > 10 * TOL[dtype]
    assert err(_replay(S2, v, tile, lambda m0, m1: math.exp(m0 - m1))) > TOL[dtype]
