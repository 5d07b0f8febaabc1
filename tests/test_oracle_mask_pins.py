"""Pins of the oracle's additive mask (the `mask` argument of ggmlR's
ag_flash_attention: 0 attends, -Inf blocks; a finite value is added to the
scaled score), against brute force, closed forms, finite differences and
torch's float64 autograd, plus planted mistakes that these pins must catch."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa


def _case(B=1, Hq=2, Hkv=1, Lq=5, Lkv=6, D=4, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, Lkv, D))
    v = rng.standard_normal((B, Hkv, Lkv, D))
    do = rng.standard_normal((B, Hq, Lq, D))
    return q, k, v, do


def _bias(shape, seed, blocked=0.25):
    """Finite N(0,1) values with about `blocked` of the entries -inf."""
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(shape)
    b[rng.random(shape) < blocked] = -np.inf
    return b


def _brute(q, k, v, scale, causal, window, bias):
    """Pure-Python loops: each row's softmax over the keys that the flags allow
    and the mask does not block, score = scale * q.k + mask."""
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    bias = np.broadcast_to(bias, (B, Hq, Lq, Lkv))
    O = np.zeros_like(q)
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Lq):
                s = {}
                for j in range(Lkv):
                    if not oracle.allowed(i, j, causal, window) or bias[b, h, i, j] == -math.inf:
                        continue
                    s[j] = scale * sum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) + bias[b, h, i, j]
                if not s:
                    LSE[b, h, i] = -math.inf
                    continue
                den = sum(math.exp(x) for x in s.values())
                LSE[b, h, i] = math.log(den)
                for d in range(D):
                    O[b, h, i, d] = sum(math.exp(s[j]) / den * v[b, g, j, d] for j in s)
    return O, LSE


def _fd(q, k, v, do, scale, causal, window, bias, h=1e-6):
    def f(qq, kk, vv):
        O, _ = oracle.forward(qq, kk, vv, scale, causal, window, bias=bias)
        return float((O * do).sum())

    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            fp = f(*args)
            x[idx] = x0 - h
            fm = f(*args)
            x[idx] = x0
            g[idx] = (fp - fm) / (2 * h)
        out.append(g)
    return out


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("causal,window,Lq,Lkv", [(False, 0, 5, 6), (True, 0, 6, 6), (True, 2, 6, 6),
                                                  (False, 3, 6, 4)])
def test_masked_forward_matches_brute_force(causal, window, Lq, Lkv):
    q, k, v, _ = _case(Lq=Lq, Lkv=Lkv, seed=11)
    bias = _bias((1, 2, Lq, Lkv), 12)
    O, L = oracle.forward(q, k, v, 0.7, causal, window, bias=bias)
    Ob, Lb = _brute(q, k, v, 0.7, causal, window, bias)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    assert np.abs(L[fin] - Lb[fin]).max() < 1e-12
    assert np.abs(O - Ob).max() < 1e-12


def test_zero_mask_changes_nothing():
    q, k, v, do = _case(Lq=6, Lkv=7, seed=13)
    a = oracle.backward(q, k, v, do, 0.5, True, 3)
    b = oracle.backward(q, k, v, do, 0.5, True, 3, bias=np.zeros((6, 7)))
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_causal_shaped_mask_equals_causal_flag():
    q, k, v, do = _case(Lq=6, Lkv=6, seed=14)
    m = np.where(np.tril(np.ones((6, 6), dtype=bool)), 0.0, -np.inf)
    a = oracle.backward(q, k, v, do, 0.5, True, 0)
    b = oracle.backward(q, k, v, do, 0.5, False, 0, bias=m)
    for key in a:
        assert np.allclose(a[key], b[key], rtol=0, atol=1e-14), key


def test_logical_mask_closed_form():
    # .ag_flash_mask: TRUE (may attend) -> 0, FALSE -> -Inf, elementwise, any shape
    m = np.array([[True, False, True, True],
                  [False, False, True, False],
                  [True, True, True, True]])
    want = np.array([[0.0, -np.inf, 0.0, 0.0],
                     [-np.inf, -np.inf, 0.0, -np.inf],
                     [0.0, 0.0, 0.0, 0.0]])
    got = oracle.logical_mask_bias(m)
    assert got.dtype == np.float64 and got.shape == m.shape
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.logical_mask_bias(m[None, None]), want[None, None])


def test_logical_causal_mask_equals_causal_flag():
    # the lower-triangular logical mask (key j <= query i allowed) is the causal
    # rule, so forward and gradients agree with causal=True and no mask
    q, k, v, do = _case(Hq=2, Hkv=1, Lq=7, Lkv=7, seed=31)
    m = oracle.logical_mask_bias(np.tril(np.ones((7, 7), dtype=bool)))
    a = oracle.backward(q, k, v, do, 0.5, True, 0)
    b = oracle.backward(q, k, v, do, 0.5, False, 0, bias=m)
    for key in a:
        assert np.allclose(a[key], b[key], rtol=0, atol=1e-14), key


def test_logical_mask_matches_brute_force():
    q, k, v, do = _case(Lq=5, Lkv=6, seed=32)
    allowed_pairs = np.random.default_rng(33).random((5, 6)) > 0.3
    bias = oracle.logical_mask_bias(allowed_pairs)
    O, L = oracle.forward(q, k, v, 0.6, False, 0, bias=bias)
    Ob, Lb = _brute(q, k, v, 0.6, False, 0, bias)
    assert np.abs(O - Ob).max() <= 1e-12
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))


def test_planted_inverted_logical_mask_is_caught(monkeypatch):
    # reading TRUE as "blocked" must fail the closed form and the causal pin
    real = oa.logical_mask_bias
    monkeypatch.setattr(oracle, "logical_mask_bias", lambda m: real(~np.asarray(m, dtype=bool)))
    with pytest.raises(AssertionError):
        test_logical_mask_closed_form()
    with pytest.raises(AssertionError):
        test_logical_causal_mask_equals_causal_flag()


def test_row_constant_mask_shifts_only_the_lse():
    q, k, v, do = _case(Lq=5, Lkv=6, seed=15)
    c = np.array([0.5, -1.0, 2.0, 0.0, 3.5])
    a = oracle.backward(q, k, v, do, 0.4, False, 0)
    b = oracle.backward(q, k, v, do, 0.4, False, 0, bias=np.repeat(c[:, None], 6, axis=1))
    for key in ("O", "dQ", "dK", "dV", "Delta"):
        assert np.allclose(a[key], b[key], rtol=0, atol=1e-12), key
    assert np.allclose(b["LSE"], a["LSE"] + c, rtol=0, atol=1e-12)


def test_log_weights_give_a_weighted_softmax():
    # mask = log w_j: P_ij = w_j exp(s_ij) / sum_j w_j exp(s_ij)
    q, k, v, _ = _case(Hq=1, Lq=3, Lkv=4, seed=16)
    w = np.array([0.5, 2.0, 1.0, 0.25])
    O, _ = oracle.forward(q, k, v, 1.0, False, 0, bias=np.log(w)[None, :])
    e = np.exp(q[0, 0] @ k[0, 0].T) * w
    assert np.abs(O[0, 0] - (e / e.sum(axis=1, keepdims=True)) @ v[0, 0]).max() < 1e-13


def test_per_head_mask_broadcast():
    q, k, v, do = _case(B=2, Hq=2, Hkv=1, Lq=4, Lkv=5, seed=17)
    m = _bias((2, 1, 4, 5), 18, blocked=0.1)
    a = oracle.backward(q, k, v, do, 0.5, False, 0, bias=m)
    b = oracle.backward(q, k, v, do, 0.5, False, 0, bias=np.repeat(m, 2, axis=1))
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    # a mask that differs between the two heads changes only the second head
    m2 = np.repeat(m, 2, axis=1).copy()
    m2[:, 1] += 1.0 * np.arange(5)
    c = oracle.backward(q, k, v, do, 0.5, False, 0, bias=m2)
    assert np.array_equal(c["O"][:, 0], a["O"][:, 0]) and not np.allclose(c["O"][:, 1], a["O"][:, 1])


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 2)])
def test_masked_gradients_match_finite_differences(causal, window):
    q, k, v, do = _case(Lq=5, Lkv=6, seed=19)
    bias = _bias((5, 6), 20)
    r = oracle.backward(q, k, v, do, 0.6, causal, window, bias=bias)
    gq, gk, gv = _fd(q, k, v, do, 0.6, causal, window, bias)
    assert _rel(r["dQ"], gq) < 1e-6
    assert _rel(r["dK"], gk) < 1e-6
    assert _rel(r["dV"], gv) < 1e-6


def test_masked_matches_torch_autograd():
    q, k, v, do = _case(B=1, Hq=4, Hkv=2, Lq=7, Lkv=8, seed=21)
    bias = _bias((1, 4, 7, 8), 22, blocked=0.2)
    bias[0, 0, 3, :] = -np.inf  # one row with every key blocked
    r = oracle.backward(q, k, v, do, 0.3, False, 0, bias=bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(2, dim=1)
    vv = tv.repeat_interleave(2, dim=1)
    s = 0.3 * tq @ kk.transpose(-1, -2) + torch.tensor(bias)
    rowmax = torch.nan_to_num(s.max(dim=-1, keepdim=True).values, neginf=0.0)
    e = torch.exp(s - rowmax)
    den = e.sum(dim=-1, keepdim=True)
    p = torch.where(den > 0, e / torch.where(den > 0, den, torch.ones_like(den)), torch.zeros_like(e))
    o = p @ vv
    (o * torch.tensor(do)).sum().backward()
    assert np.abs(r["O"] - o.detach().numpy()).max() < 1e-12
    assert _rel(r["dQ"], tq.grad.numpy()) < 1e-12
    assert _rel(r["dK"], tk.grad.numpy()) < 1e-12
    assert _rel(r["dV"], tv.grad.numpy()) < 1e-12
    assert np.isneginf(r["LSE"][0, 0, 3]) and not r["O"][0, 0, 3].any() and not r["dQ"][0, 0, 3].any()


def test_nan_and_positive_infinity_are_rejected():
    q, k, v, _ = _case(Lq=2, Lkv=2)
    for bad in (np.nan, np.inf):
        with pytest.raises(ValueError):
            oracle.forward(q, k, v, 1.0, False, 0, bias=np.array([[0.0, bad], [0.0, 0.0]]))


# ---------------------------------------------------------------------------
# planted mistakes in the mask handling: each must fail these pins
# ---------------------------------------------------------------------------

def _mask_pins_pass():
    try:
        q, k, v, do = _case(Lq=5, Lkv=6, seed=23)
        bias = _bias((5, 6), 24)
        for causal, window in [(False, 0), (True, 2)]:
            O, L = oracle.forward(q, k, v, 0.7, causal, window, bias=bias)
            Ob, Lb = _brute(q, k, v, 0.7, causal, window, bias)
            if np.abs(O - Ob).max() > 1e-12 or not np.array_equal(np.isneginf(L), np.isneginf(Lb)):
                return False
            r = oracle.backward(q, k, v, do, 0.7, causal, window, bias=bias)
            gq, gk, gv = _fd(q, k, v, do, 0.7, causal, window, bias)
            if max(_rel(r["dQ"], gq), _rel(r["dK"], gk), _rel(r["dV"], gv)) > 1e-6:
                return False
        return True
    except Exception:
        return False


def test_mask_pins_pass_on_the_real_oracle():
    assert _mask_pins_pass()


@pytest.mark.parametrize("mistake", ["scaled_mask", "transposed_mask", "mask_forward_only"])
def test_planted_mask_mistakes_are_caught(monkeypatch, mistake):
    real_rf = oa.rows_forward
    if mistake == "scaled_mask":
        def rf(q_rows, K, V, rows, scale, causal, window, cols=None, bias_rows=None):
            b = None if bias_rows is None else np.asarray(bias_rows) * scale  # mask inside the scale
            return real_rf(q_rows, K, V, rows, scale, causal, window, cols, b)
        monkeypatch.setattr(oa, "rows_forward", rf)
    elif mistake == "transposed_mask":
        real_bias = oa._bias

        def tb(bias, B, Hq, Lq, Lkv):
            if bias is None:
                return None
            full = np.zeros((Lq, Lkv))
            m = np.asarray(bias)
            full[:min(Lq, Lkv), :min(Lq, Lkv)] = m.T[:min(Lq, Lkv), :min(Lq, Lkv)]  # keys read as rows
            return real_bias(full, B, Hq, Lq, Lkv)
        monkeypatch.setattr(oa, "_bias", tb)
    elif mistake == "mask_forward_only":
        real_bwd = oa.backward

        def bwd(q, k, v, do, scale, causal=False, window=0, bias=None):
            return real_bwd(q, k, v, do, scale, causal, window)  # gradient against the unmasked scores
        monkeypatch.setattr(oracle, "backward", bwd)
    assert not _mask_pins_pass()
