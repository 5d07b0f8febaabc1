"""Pins of the float64 oracle against things other than itself.

Every check here runs on the CPU. The oracle is pinned by:
  * hand-written mask tables (tests/golden/), from the pages' mask rule;
  * pure-Python triple loops of textbook softmax attention on tiny inputs;
  * torch float64 autograd of a materialised attention (a library routine);
  * central finite differences of f = sum(dO * O) for dQ, dK, dV;
  * closed forms (constant V, zero scale, one key, diagonal-only window);
  * invariants (softmax rows sum to 1, LSE identity, sum_j dK_j = 0,
    sum_j dS_ij = 0, Delta = rowsum(P * dP), dV = P^T dO, GQA = repeated MHA);
  * the row/key sampling entry points against the full computation;
  * planted mistakes in the oracle, each of which one of the pins must catch.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
from synth import decode, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, rng, s=1.0):
    return rng.standard_normal(shape) * s


def _case(B=1, Hq=4, Hkv=2, Lq=6, Lkv=6, D=4, seed=0):
    rng = np.random.default_rng(seed)
    q = _rand((B, Hq, Lq, D), rng)
    k = _rand((B, Hkv, Lkv, D), rng)
    v = _rand((B, Hkv, Lkv, D), rng)
    do = _rand((B, Hq, Lq, D), rng)
    return q, k, v, do


def _load_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=bool)


# ---------------------------------------------------------------------------
# mask semantics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize(
    "name,Lq,Lkv,causal,window",
    [
        ("mask_causal_L6.txt", 6, 6, True, 0),
        ("mask_causal_w3_L6.txt", 6, 6, True, 3),
        ("mask_causal_w1_L6.txt", 6, 6, True, 1),
        ("mask_window3_noncausal_L6.txt", 6, 6, False, 3),
        ("mask_causal_w2_Lq6_Lkv3.txt", 6, 3, True, 2),
    ],
)
def test_mask_tables(name, Lq, Lkv, causal, window):
    want = _load_mask(name)
    got = oracle.mask_matrix(np.arange(Lq), Lkv, causal, window)
    assert got.shape == want.shape
    assert (got == want).all()
    for i in range(Lq):
        for j in range(Lkv):
            assert oracle.allowed(i, j, causal, window) == want[i, j]


def test_window_at_least_length_is_plain_causal():
    for L in (1, 5, 9):
        a = oracle.mask_matrix(np.arange(L), L, True, L)
        b = oracle.mask_matrix(np.arange(L), L, True, 0)
        assert (a == b).all()


# ---------------------------------------------------------------------------
# brute force: textbook softmax attention in pure-Python loops
# ---------------------------------------------------------------------------

def _brute_forward(q, k, v, scale, causal, window):
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    reps = Hq // Hkv
    O = np.zeros_like(q)
    LSE = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // reps
            for i in range(Lq):
                keys = [j for j in range(Lkv) if oracle.allowed(i, j, causal, window)]
                if not keys:
                    LSE[b, h, i] = -math.inf
                    continue
                s = {}
                for j in keys:
                    dot = 0.0
                    for d in range(D):
                        dot += q[b, h, i, d] * k[b, g, j, d]
                    s[j] = dot * scale
                den = sum(math.exp(s[j]) for j in keys)
                LSE[b, h, i] = math.log(den)
                for d in range(D):
                    O[b, h, i, d] = sum(math.exp(s[j]) / den * v[b, g, j, d] for j in keys)
    return O, LSE


@pytest.mark.parametrize("causal,window,Lq,Lkv", [(False, 0, 5, 5), (True, 0, 6, 6), (True, 3, 6, 6),
                                                   (False, 2, 5, 6), (True, 2, 6, 3), (True, 0, 4, 6)])
def test_forward_matches_brute_force(causal, window, Lq, Lkv):
    q, k, v, _ = _case(Lq=Lq, Lkv=Lkv, seed=1)
    scale = 0.7
    O, LSE = oracle.forward(q, k, v, scale, causal, window)
    Ob, LSEb = _brute_forward(q, k, v, scale, causal, window)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(LSEb)
    assert (np.isfinite(LSE) == fin).all()
    np.testing.assert_allclose(LSE[fin], LSEb[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# torch float64 autograd of a materialised attention (independent library path)
# ---------------------------------------------------------------------------

def _torch_attention(q, k, v, scale, causal, window):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    reps = q.shape[1] // k.shape[1]
    kr = kt.repeat_interleave(reps, dim=1)
    vr = vt.repeat_interleave(reps, dim=1)
    Lq, Lkv = q.shape[2], k.shape[2]
    i = torch.arange(Lq)[:, None]
    j = torch.arange(Lkv)[None, :]
    ok = torch.ones(Lq, Lkv, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window:
        ok &= ~((i >= j) & (i - j >= window))
    s = torch.matmul(qt, kr.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~ok, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p, vr)
    return qt, kt, vt, o, lse


@pytest.mark.parametrize("causal,window,Hq,Hkv,Lq,Lkv", [(False, 0, 2, 2, 7, 7), (True, 0, 4, 2, 9, 9),
                                                         (True, 4, 8, 2, 11, 11), (False, 3, 4, 1, 6, 8),
                                                         (True, 0, 3, 1, 5, 9)])
def test_matches_torch_autograd(causal, window, Hq, Hkv, Lq, Lkv):
    q, k, v, do = _case(B=2, Hq=Hq, Hkv=Hkv, Lq=Lq, Lkv=Lkv, D=8, seed=2)
    scale = 1 / math.sqrt(8)
    qt, kt, vt, o, lse = _torch_attention(q, k, v, scale, causal, window)
    (o * torch.tensor(do)).sum().backward()
    r = oracle.backward(q, k, v, do, scale, causal, window)
    np.testing.assert_allclose(r["O"], o.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["LSE"], lse.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dQ"], qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["dK"], kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(r["dV"], vt.grad.numpy(), rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# central finite differences of f = sum(dO * O)
# ---------------------------------------------------------------------------

def _fd_grads(q, k, v, do, scale, causal, window, h=1e-6):
    def f(qq, kk, vv):
        O, _ = oracle.forward(qq, kk, vv, scale, causal, window)
        return float((O * do).sum())

    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
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


FD_CASES = [(False, 0, 6, 6), (True, 0, 6, 6), (True, 3, 6, 6), (False, 2, 5, 6), (True, 2, 6, 3)]


@pytest.mark.parametrize("causal,window,Lq,Lkv", FD_CASES)
def test_gradients_match_finite_differences(causal, window, Lq, Lkv):
    q, k, v, do = _case(Lq=Lq, Lkv=Lkv, seed=3)
    scale = 0.6
    r = oracle.backward(q, k, v, do, scale, causal, window)
    gq, gk, gv = _fd_grads(q, k, v, do, scale, causal, window)
    assert _rel(r["dQ"], gq) < 1e-6
    assert _rel(r["dK"], gk) < 1e-6
    assert _rel(r["dV"], gv) < 1e-6


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_constant_v_gives_constant_o_and_zero_dq_dk():
    q, k, v, do = _case(Lq=7, Lkv=7, seed=4)
    v[...] = 1.25
    r = oracle.backward(q, k, v, do, 0.5, True, 3)
    np.testing.assert_allclose(r["O"], 1.25, rtol=0, atol=1e-14)
    assert np.abs(r["dQ"]).max() < 1e-13
    assert np.abs(r["dK"]).max() < 1e-13


def test_zero_scale_gives_prefix_mean():
    q, k, v, _ = _case(Lq=6, Lkv=6, seed=5)
    O, LSE = oracle.forward(q, k, v, 0.0, True, 0)
    reps = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        for i in range(6):
            np.testing.assert_allclose(O[0, h, i], v[0, h // reps, : i + 1].mean(axis=0), atol=1e-14)
            assert abs(LSE[0, h, i] - math.log(i + 1)) < 1e-14


def test_zero_q_gives_window_mean():
    q, k, v, _ = _case(Lq=8, Lkv=8, seed=6)
    q[...] = 0
    O, _ = oracle.forward(q, k, v, 0.3, True, 3)
    for i in range(8):
        lo = max(0, i - 2)
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, lo: i + 1].mean(axis=0), atol=1e-14)


def test_single_key():
    q, k, v, _ = _case(Lq=5, Lkv=1, seed=7)
    O, LSE = oracle.forward(q, k, v, 0.9, False, 0)
    reps = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        np.testing.assert_allclose(O[0, h], np.broadcast_to(v[0, h // reps, 0], O[0, h].shape), atol=1e-14)
        np.testing.assert_allclose(LSE[0, h], 0.9 * q[0, h] @ k[0, h // reps, 0], atol=1e-14)


def test_diagonal_window_gives_v_itself():
    q, k, v, _ = _case(Lq=6, Lkv=6, seed=8)
    O, _ = oracle.forward(q, k, v, 1.0, True, 1)
    reps = q.shape[1] // k.shape[1]
    for h in range(q.shape[1]):
        np.testing.assert_allclose(O[0, h], v[0, h // reps], atol=1e-14)


def test_fully_masked_rows_are_zero():
    q, k, v, do = _case(Lq=6, Lkv=3, seed=9)
    r = oracle.backward(q, k, v, do, 0.5, True, 2)
    assert np.all(r["O"][:, :, 4:] == 0)
    assert np.all(np.isneginf(r["LSE"][:, :, 4:]))
    assert np.all(r["dQ"][:, :, 4:] == 0)
    assert np.isfinite(r["dK"]).all() and np.isfinite(r["dV"]).all()


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_lse_identity():
    q, k, v, _ = _case(Lq=9, Lkv=9, D=5, seed=10)
    rows = np.arange(9)
    for causal, window in [(False, 0), (True, 0), (True, 4)]:
        S, P, O, lse = oracle.rows_forward(q[0, 1], k[0, 0], v[0, 0], rows, 0.4, causal, window)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        ok = oracle.mask_matrix(rows, 9, causal, window)
        assert np.all(P[~ok] == 0)
        raw = 0.4 * (q[0, 1] @ k[0, 0].T)
        direct = np.log(np.where(ok, np.exp(raw), 0).sum(axis=1))  # no max shift
        np.testing.assert_allclose(lse, direct, rtol=0, atol=1e-12)
        np.testing.assert_allclose(O, np.where(ok, np.exp(raw - direct[:, None]), 0) @ v[0, 0], atol=1e-12)


def test_gradient_identities():
    q, k, v, do = _case(B=2, Hq=6, Hkv=2, Lq=10, Lkv=10, D=6, seed=11)
    scale = 0.45
    for causal, window in [(False, 0), (True, 0), (True, 3)]:
        r = oracle.backward(q, k, v, do, scale, causal, window)
        # softmax shift invariance: adding a constant to every key of a row changes nothing,
        # so the key gradients of each (b, g) sum to zero
        np.testing.assert_allclose(r["dK"].sum(axis=2), 0, atol=1e-12)
        rows = np.arange(10)
        for b in range(2):
            for h in range(6):
                g = h // 3
                _, P, O, _ = oracle.rows_forward(q[b, h], k[b, g], v[b, g], rows, scale, causal, window)
                dP = do[b, h] @ v[b, g].T
                np.testing.assert_allclose(r["Delta"][b, h], (P * dP).sum(axis=1), atol=1e-12)
                dS = P * (dP - r["Delta"][b, h][:, None])
                np.testing.assert_allclose(dS.sum(axis=1), 0, atol=1e-12)
        # dV = P^T dO summed over the group, as one explicit product over stacked heads
        for b in range(2):
            for g in range(2):
                Ps, dOs = [], []
                for h in range(3 * g, 3 * g + 3):
                    _, P, _, _ = oracle.rows_forward(q[b, h], k[b, g], v[b, g], rows, scale, causal, window)
                    Ps.append(P)
                    dOs.append(do[b, h])
                np.testing.assert_allclose(r["dV"][b, g], np.vstack(Ps).T @ np.vstack(dOs), atol=1e-12)


def test_gqa_equals_repeated_mha():
    q, k, v, do = _case(B=1, Hq=8, Hkv=2, Lq=7, Lkv=7, D=4, seed=12)
    g = oracle.backward(q, k, v, do, 0.5, True, 0)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    m = oracle.backward(q, kr, vr, do, 0.5, True, 0)
    np.testing.assert_allclose(g["O"], m["O"], atol=1e-14)
    np.testing.assert_allclose(g["dQ"], m["dQ"], atol=1e-14)
    np.testing.assert_allclose(g["dK"], m["dK"].reshape(1, 2, 4, 7, 4).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(g["dV"], m["dV"].reshape(1, 2, 4, 7, 4).sum(axis=2), atol=1e-13)


def test_sampling_entry_points_match_full():
    q, k, v, do = _case(B=2, Hq=4, Hkv=2, Lq=13, Lkv=13, D=4, seed=13)
    for causal, window in [(False, 0), (True, 0), (True, 4), (False, 3)]:
        r = oracle.backward(q, k, v, do, 0.5, causal, window)
        rows = [0, 5, 12]
        s = oracle.sample_rows(q, k, v, do, 0.5, causal, window, 1, 3, rows)
        for key in ("O", "LSE", "Delta", "dQ"):
            np.testing.assert_allclose(s[key], r[key][1, 3, rows], atol=1e-13)
        keys = [0, 7, 12]
        s = oracle.sample_keys(q, k, v, do, 0.5, causal, window, 1, 1, keys)
        np.testing.assert_allclose(s["dK"], r["dK"][1, 1, keys], atol=1e-13)
        np.testing.assert_allclose(s["dV"], r["dV"][1, 1, keys], atol=1e-13)


def test_bwd_preprocess_definition():
    rng = np.random.default_rng(14)
    o, do = rng.standard_normal((3, 5, 8)), rng.standard_normal((3, 5, 8))
    want = np.einsum("abd,abd->ab", o, do)
    np.testing.assert_allclose(oracle.bwd_preprocess(o, do), want, atol=1e-13)


def test_synth_inputs_are_exact_storage_values():
    x = make_inputs(1, 2, 1, 5, 5, 8, "bf16", 1234)
    q = decode(x["q"], "bf16")
    # bf16 values have at most 8 significant bits
    m, e = np.frexp(q)
    assert np.all(m * 256 == np.round(m * 256))
    t = torch.from_numpy(x["q"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(t, q)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def _pins_pass():
    """Run the strongest pins on one small case; True when all pass."""
    q, k, v, do = _case(Lq=6, Lkv=6, seed=3)
    try:
        for causal, window in [(True, 3), (False, 0)]:
            r = oracle.backward(q, k, v, do, 0.6, causal, window)
            gq, gk, gv = _fd_grads(q, k, v, do, 0.6, causal, window)
            if max(_rel(r["dQ"], gq), _rel(r["dK"], gk), _rel(r["dV"], gv)) > 1e-6:
                return False
            Ob, Lb = _brute_forward(q, k, v, 0.6, causal, window)
            if np.abs(r["O"] - Ob).max() > 1e-12 or np.abs(r["LSE"] - Lb).max() > 1e-12:
                return False
            if (oracle.mask_matrix(np.arange(6), 6, True, 3) != _load_mask("mask_causal_w3_L6.txt")).any():
                return False
        return True
    except Exception:
        return False


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("mistake", ["delta_zero", "window_off_by_one", "dk_transposed_q", "no_scale_in_dq",
                                     "lse_log2", "kv_head_modulo"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "delta_zero":
        monkeypatch.setattr(oa, "bwd_preprocess", lambda o, do: np.zeros(np.shape(o)[:-1]))
    elif mistake == "window_off_by_one":
        real = oa.mask_matrix

        def mm(rows, Lkv, causal, window, cols=None):
            return real(rows, Lkv, causal, window + 1 if window else 0, cols)
        monkeypatch.setattr(oa, "mask_matrix", mm)
    elif mistake == "dk_transposed_q":
        real_bwd = oa.backward

        def bwd(q, k, v, do, scale, causal=False, window=0):
            r = real_bwd(q, k, v, do, scale, causal, window)
            r["dK"] = r["dK"][:, :, ::-1]  # keys reversed: a wrong index
            return r
        monkeypatch.setattr(oracle, "backward", bwd)
    elif mistake == "no_scale_in_dq":
        real_bwd = oa.backward

        def bwd(q, k, v, do, scale, causal=False, window=0):
            r = real_bwd(q, k, v, do, scale, causal, window)
            r["dQ"] = r["dQ"] / scale
            return r
        monkeypatch.setattr(oracle, "backward", bwd)
    elif mistake == "lse_log2":
        real_rf = oa.rows_forward

        def rf(*a, **kw):
            S, P, O, lse = real_rf(*a, **kw)
            return S, P, O, lse / math.log(2)
        monkeypatch.setattr(oa, "rows_forward", rf)
    elif mistake == "kv_head_modulo":
        monkeypatch.setattr(oa, "_kv_head", lambda h, Hq, Hkv: h % Hkv)
    assert not _pins_pass()


def test_sampling_with_cross_lengths_and_empty_rows():
    # Lq > Lkv with causal + window leaves rows with no allowed key at all
    q, k, v, do = _case(B=1, Hq=4, Hkv=2, Lq=12, Lkv=5, D=4, seed=15)
    for causal, window in [(True, 2), (True, 0), (False, 3)]:
        r = oracle.backward(q, k, v, do, 0.5, causal, window)
        rows = list(range(12))
        s = oracle.sample_rows(q, k, v, do, 0.5, causal, window, 0, 1, rows)
        for key in ("O", "Delta", "dQ"):
            np.testing.assert_allclose(s[key], r[key][0, 1, rows], atol=1e-13)
        assert np.array_equal(np.isneginf(s["LSE"]), np.isneginf(r["LSE"][0, 1]))
        fin = np.isfinite(s["LSE"])
        np.testing.assert_allclose(s["LSE"][fin], r["LSE"][0, 1][fin], atol=1e-13)
        keys = list(range(5))
        s = oracle.sample_keys(q, k, v, do, 0.5, causal, window, 0, 1, keys)
        np.testing.assert_allclose(s["dK"], r["dK"][0, 1, keys], atol=1e-13)
        np.testing.assert_allclose(s["dV"], r["dV"][0, 1, keys], atol=1e-13)


def test_key_span_holds_every_allowed_key():
    for Lq, Lkv, causal, window in [(9, 9, True, 3), (9, 4, True, 2), (6, 9, False, 2), (7, 7, False, 0)]:
        ok = oracle.mask_matrix(np.arange(Lq), Lkv, causal, window)
        for i in range(Lq):
            span = oracle.key_span([i], Lkv, causal, window)
            assert set(np.nonzero(ok[i])[0]) <= set(span.tolist())


# ---------------------------------------------------------------------------
# row-blocked key gradients (used for the 32768-token workload's dK/dV)
# ---------------------------------------------------------------------------

KEY_GRAD_SHAPES = [
    # B, Hq, Hkv, Lq, Lkv, causal, window
    (2, 4, 2, 37, 37, True, 0),
    (1, 6, 2, 40, 40, True, 5),
    (1, 4, 1, 20, 33, False, 0),
    (2, 4, 2, 30, 12, True, 3),  # rows with no allowed key
    (1, 2, 2, 25, 25, False, 7),
]


def _key_grads_agree():
    """key_grads against the full backward (whole score matrices, no blocking) on
    small shapes, for every kv head, all keys and a scattered subset, with row
    blocks of 1, 5 and 64 rows and 1 or 3 threads; True when all agree to 1e-12
    (an exception counts as disagreement)."""
    try:
        return _key_grads_agree_or_raise()
    except Exception:
        return False


def _key_grads_agree_or_raise():
    for n, (B, Hq, Hkv, Lq, Lkv, causal, window) in enumerate(KEY_GRAD_SHAPES):
        q, k, v, do = _case(B, Hq, Hkv, Lq, Lkv, 5, seed=40 + n)
        r = oracle.backward(q, k, v, do, 0.45, causal, window)
        for keys in (np.arange(Lkv), np.array([Lkv - 1, 0, Lkv // 2, 1])):
            for row_block, workers in ((1, 1), (5, 3), (64, 1)):
                for b in range(B):
                    for g in range(Hkv):
                        s = oracle.key_grads(q, k, v, do, 0.45, causal, window, b, g, keys, row_block, workers)
                        if np.abs(s["dK"] - r["dK"][b, g, keys]).max() > 1e-12:
                            return False
                        if np.abs(s["dV"] - r["dV"][b, g, keys]).max() > 1e-12:
                            return False
    return True


def test_key_grads_match_the_full_backward():
    assert _key_grads_agree()


@pytest.mark.parametrize("mistake", ["span_short_by_one", "rows_of_one_head"])
def test_key_grads_planted_mistakes_are_caught(monkeypatch, mistake):
    if mistake == "span_short_by_one":
        # each row block's LSE taken without the first key of its span
        real = oa.key_span
        monkeypatch.setattr(oa, "key_span", lambda rows, Lkv, causal, window: real(rows, Lkv, causal, window)[1:])
    elif mistake == "rows_of_one_head":
        # every query head of the group handled with the rows of the group's first head
        real_kg = oa.key_grads

        def kg(q, k, v, do, scale, causal, window, b, g, keys, row_block=256, workers=1):
            reps = q.shape[1] // k.shape[1]
            q1 = q.copy()
            q1[:, g * reps:(g + 1) * reps] = q[:, g * reps:g * reps + 1]
            return real_kg(q1, k, v, do, scale, causal, window, b, g, keys, row_block, workers)
        monkeypatch.setattr(oracle, "key_grads", kg)
    assert not _key_grads_agree()
