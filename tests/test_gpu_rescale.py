"""GPU parity on inputs that make the forward's lazy online-softmax rescale
fire (tests/rescale_cases.py): a later key tile's row maximum above the first
live tile's by more than 8 log2 units in most rows, asserted from the
oracle's scores before the GPU runs. Covers every forward instantiation:
16-bit tiled kernels in the 64/128/256/512 buckets, float32 kernels in the
32/64/96/128/256/512 buckets and the short-query kernels in the 64/128
buckets, each with and without a mask (float or bool), with causal,
windowed, cross-length (Lq != Lkv) and Dv != D shapes. Element-wise O, LSE,
Delta, dQ, dK and dV against the float64 oracle at the dtype's tolerance."""
import math

import pytest

import rescale_cases as rc
from parity_util import compare_given

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", range(len(rc.CASES)), ids=[c[0] for c in rc.CASES])
def test_rescale_parity(n):
    name, B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window, mk, path = rc.CASES[n]
    print(f"rescale case {n}: {rc.CASES[n]}", flush=True)
    x, mask = rc.case_inputs(n)
    frac = rc.branch_fraction(n, x, mask)
    assert frac >= rc.MIN_FRACTION, f"inputs take the rescale branch in only {frac:.2f} of the rows"
    compare_given(x, dtype, 1.0 / math.sqrt(D), causal, window, mask=mask)
