"""The torch.autograd node (attention_fa_fwd_06_amd.autograd) on the GPU:
gradients from loss.backward() against the float64 oracle, identity with the
four C-ABI calls made directly, and non-contiguous inputs."""
import numpy as np
import pytest
import torch

import oracle
from attention_fa_fwd_06_amd.autograd import flash_attention
from parity_util import gpu_inputs, rel_err, run_gpu
from synth import TOL, decode, from_torch, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16", 2, 4, 2, 200, 128, True, 0),
    ("f16", 1, 4, 1, 130, 64, True, 48),
    ("f32", 1, 2, 2, 70, 32, False, 0),
    ("bf16", 1, 2, 1, 96, 256, True, 0),
    ("f16", 1, 3, 3, 40, 96, False, 16),
]


def _grads(t, scale, causal, window):
    q, k, v = (t[n].clone().requires_grad_() for n in ("q", "k", "v"))
    o = flash_attention(q, k, v, scale, causal, window)
    o.backward(t["do"])
    torch.cuda.synchronize()
    return o.detach(), q.grad, k.grad, v.grad


@pytest.mark.parametrize("dtype,B,Hq,Hkv,L,D,causal,window", CASES)
def test_backward_through_autograd_matches_oracle(dtype, B, Hq, Hkv, L, D, causal, window):
    seed = 7000 + L + D
    scale = 1.0 / np.sqrt(D)
    x = make_inputs(B, Hq, Hkv, L, L, D, dtype, seed)
    ref = oracle.backward(*(decode(x[n], dtype) for n in ("q", "k", "v", "do")), scale, causal, window)
    o, dq, dk, dv = _grads(gpu_inputs(x, dtype), scale, causal, window)
    errs = {key: rel_err(from_torch(val, dtype), ref[key])
            for key, val in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv))}
    assert all(e <= TOL[dtype] for e in errs.values()), errs


def test_autograd_node_is_the_c_abi_path():
    dtype, scale = "bf16", 1.0 / np.sqrt(128)
    x = make_inputs(1, 4, 2, 150, 150, 128, dtype, 7101)
    t = gpu_inputs(x, dtype)
    direct = run_gpu(t, scale, True, 0)
    o, dq, dk, dv = _grads(t, scale, True, 0)
    for name, got in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert torch.equal(got, direct[name]), name


def test_non_contiguous_inputs_and_lse_output():
    dtype, scale = "f16", 0.125
    x = make_inputs(2, 4, 4, 64, 64, 64, dtype, 7102)
    t = gpu_inputs(x, dtype)
    # the same values laid out [B, L, H, D] and viewed as [B, H, L, D]
    q, k, v = (t[n].transpose(1, 2).contiguous().transpose(1, 2).requires_grad_() for n in ("q", "k", "v"))
    assert not q.is_contiguous()
    o, lse = flash_attention(q, k, v, scale, True, 0, return_lse=True)
    assert not lse.requires_grad and lse.dtype == torch.float32 and tuple(lse.shape) == (2, 4, 64)
    o.backward(t["do"])
    o2, dq2, dk2, dv2 = _grads(t, scale, True, 0)
    assert torch.equal(o.detach(), o2)
    assert torch.equal(q.grad, dq2) and torch.equal(k.grad, dk2) and torch.equal(v.grad, dv2)
