"""GPU parity of the 16-bit head-dim buckets 32 and 96 (head dim 32, the
smallest the calls take, and head dims from 72 to 96: the MLX pull request's test plan runs head dims 32, 64,
96 and 128, and mlx-bun supports 96). These buckets keep padded LDS rows for
the swizzle but run every product over 32 or 96 columns. The cases use query
lengths above 16 (the tiled kernels, not the short-query path): causal,
windowed, cross-length, head dims below the bucket's, a float and a bool mask, Dv != D
(the bucket is that of the larger head dim) and the causal key-block pairing
of dK/dV. Element-wise O, LSE, Delta, dQ, dK, dV against the float64 oracle."""
import numpy as np
import pytest

from parity_util import compare_full, compare_given
from synth import make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window
    (1, 4, 2, 300, 300, 32, 32, "bf16", True, 0),
    (2, 4, 1, 257, 257, 32, 32, "f16", True, 50),
    (1, 2, 2, 100, 333, 32, 32, "bf16", False, 0),
    (1, 8, 2, 200, 130, 32, 32, "f16", True, 0),
    (1, 4, 2, 333, 333, 96, 96, "bf16", True, 0),
    (2, 2, 1, 270, 270, 80, 80, "f16", True, 100),
    (1, 4, 4, 150, 400, 96, 96, "f16", False, 0),
    (1, 4, 2, 300, 200, 88, 88, "bf16", True, 0),
    (1, 4, 2, 190, 190, 96, 64, "bf16", True, 0),
    (1, 2, 1, 210, 210, 72, 96, "f16", False, 30),
    (1, 2, 2, 120, 120, 32, 32, "bf16", False, 7),
]


@pytest.mark.parametrize("n", range(len(CASES)), ids=["B{}_H{}:{}_L{}x{}_D{}_Dv{}_{}_c{}_w{}".format(*c) for c in CASES])
def test_bucket_parity(n):
    B, Hq, Hkv, Lq, Lkv, D, Dv, dtype, causal, window = CASES[n]
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 33000 + n, Dv=Dv)
    compare_given(x, dtype, 1.0 / np.sqrt(D), causal, window)


@pytest.mark.parametrize("D,dtype,kind", [(32, "bf16", "float"), (96, "f16", "bool"), (32, "f16", "bool"),
                                          (72, "bf16", "float")])
def test_bucket_parity_with_mask(D, dtype, kind):
    B, Hq, Hkv, Lq, Lkv = 1, 4, 2, 180, 230
    x = make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, 33100 + D)
    rng = np.random.default_rng(33200 + D)
    if kind == "float":
        m = (rng.standard_normal((Hq, Lq, Lkv)) * 1.5).astype(np.float32)
        m[rng.random((Hq, Lq, Lkv)) < 0.2] = -np.inf
    else:
        m = rng.random((Lq, Lkv)) >= 0.2
    compare_given(x, dtype, 1.0 / np.sqrt(D), True, 0, mask=m)


@pytest.mark.parametrize("D,dtype", [(96, "bf16"), (32, "f16")])
def test_bucket_key_block_pairing(D, dtype):
    # causal without window and 8 key blocks of 128 over 64 (batch, kv head)
    # groups: the dK/dV workgroups take key blocks p and 7 - p; ragged last block
    compare_full(8, 8, 8, 900, 900, D, dtype, True, 0, seed=33300 + D)
