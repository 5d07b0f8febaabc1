"""Pins of the oracle with a value head dim Dv different from the query/key
head dim D (O, dO and dV are [.., Dv]): brute force, finite differences and
torch's float64 autograd."""
import math

import numpy as np
import pytest
import torch

import oracle


def _case(B, Hq, Hkv, Lq, Lkv, D, Dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lkv, D))
    v = rng.standard_normal((B, Hkv, Lkv, Dv))
    do = rng.standard_normal((B, Hq, Lq, Dv))
    return q, k, v, do


@pytest.mark.parametrize("D,Dv,causal,window", [(4, 6, True, 0), (6, 3, False, 2), (5, 5, True, 3)])
def test_forward_matches_brute_force(D, Dv, causal, window):
    q, k, v, _ = _case(1, 2, 1, 5, 6, D, Dv, 31)
    O, L = oracle.forward(q, k, v, 0.8, causal, window)
    assert O.shape == (1, 2, 5, Dv)
    for h in range(2):
        for i in range(5):
            keys = [j for j in range(6) if oracle.allowed(i, j, causal, window)]
            s = {j: 0.8 * sum(q[0, h, i, d] * k[0, 0, j, d] for d in range(D)) for j in keys}
            den = sum(math.exp(x) for x in s.values())
            assert abs(L[0, h, i] - math.log(den)) < 1e-12
            for e in range(Dv):
                assert abs(O[0, h, i, e] - sum(math.exp(s[j]) / den * v[0, 0, j, e] for j in keys)) < 1e-12


def test_gradients_match_finite_differences():
    q, k, v, do = _case(1, 2, 1, 5, 6, 4, 7, 32)
    r = oracle.backward(q, k, v, do, 0.6, True, 0)
    assert r["dV"].shape == v.shape and r["dQ"].shape == q.shape and r["dK"].shape == k.shape

    def f(qq, kk, vv):
        return float((oracle.forward(qq, kk, vv, 0.6, True, 0)[0] * do).sum())

    for name, x in (("dQ", q), ("dK", k), ("dV", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + 1e-6
            fp = f(q, k, v)
            x[idx] = x0 - 1e-6
            fm = f(q, k, v)
            x[idx] = x0
            g[idx] = (fp - fm) / 2e-6
        assert np.abs(r[name] - g).max() / np.abs(g).max() < 1e-6, name


def test_matches_torch_autograd():
    q, k, v, do = _case(2, 4, 2, 7, 9, 8, 12, 33)
    r = oracle.backward(q, k, v, do, 0.35, False, 3)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
    s = 0.35 * tq @ kk.transpose(-1, -2)
    i = torch.arange(7)[:, None]
    j = torch.arange(9)[None, :]
    s = s.masked_fill((i >= j) & (i - j >= 3), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    (o * torch.tensor(do)).sum().backward()
    assert np.abs(r["O"] - o.detach().numpy()).max() < 1e-12
    for name, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        assert np.abs(r[name] - t.grad.numpy()).max() / np.abs(t.grad.numpy()).max() < 1e-12, name
    assert np.allclose(r["Delta"], (r["O"] * do).sum(-1), rtol=0, atol=1e-12)
