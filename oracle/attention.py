"""Float64 CPU oracle for scaled-dot-product attention and its gradients.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library.

What it computes is the plain definition of attention, written out with
matrix products and no blocking, fusion or online rescaling:

  S   = scale * Q K^T                      per batch b and query head h, with
                                           K, V taken from kv head g = h // (Hq/Hkv)
  S_ij = -inf where the mask forbids (i, j)
  LSE_i = log sum_j exp(S_ij)              natural log
  P   = exp(S - LSE)                       exactly 0 at masked entries
  O   = P V
  dP  = dO V^T,   Delta_i = sum_d dO_id O_id,   dS = P * (dP - Delta)
  dQ  = scale * dS K,  dK_g = scale * sum_{h in g} dS^T Q,  dV_g = sum_{h in g} P^T dO

Sources (the pages this follows):
  * mlx-bun flash-attention.ts, `manualSdpa`: materialised GQA attention,
    q reshaped to [B, Hkv, reps, T, D] so consecutive query heads share one kv
    head; scores times scale, masked, softmax, times V.
  * mlx-bun flash-attention.ts, forward shader: the mask rule (causal
    `kpos > q_row`; window `W != 0 and q_row >= kpos and q_row - kpos >= W`),
    the scale applied to the dot product before masking, and the natural-log
    LSE `m + log(l)` handed to the backward.
  * mlx-bun flash-attention.ts, D pre-pass and dK/dV / dQ shaders: Delta as
    the row sum of O*dO, p = exp(s - L), ds = p * (dp - Delta), dV += p dO,
    dK += ds q scale, dQ += ds k scale.
  * ggmlR R/ag_flash_attn.R, `.ag_flash_mask`: causal means query j attends to
    keys 1..j (top-left alignment).
  * ggmlR R/ag_flash_attn.R, `ag_flash_attention` (`mask` argument) and
    `.ag_flash_mask`: an optional numeric mask per (query, key), 0 to attend
    and -Inf to block, the same mask for the forward and the gradient. Here
    it is the `bias` argument, indexed [.., query, key]; a finite value is
    added to the scaled score (the reading under which 0 leaves a score alone
    and -Inf removes it), and it carries no gradient.
  * ggmlR R/ag_flash_attn.R, `.ag_flash_mask`: a logical mask is TRUE where
    attention is allowed and stands for the numeric mask with 0 there and
    -Inf elsewhere (`logical_mask_bias`).

Readings where the pages are silent or disagree (each listed in the design notes):
  * a row whose every key is masked gets O = 0, LSE = -inf and contributes no
    gradient (the forward shader would divide 0 by 0 there);
  * masked probabilities are exactly 0 (true -inf, no clamp of the exponent);
  * the window counts keys including the query itself: allowed keys are
    (i - W, i]; without causal it trims only the past, as the shader does.

Pins: every function here is checked in tests/test_oracle_pins.py against
central finite differences, torch's float64 autograd of a materialised
attention, closed forms, invariants and brute-force loops on tiny inputs.
"""
from __future__ import annotations

import numpy as np


def allowed(i: int, j: int, causal: bool, window: int) -> bool:
    """Mask rule for query row i and key j (forward shader of mlx-bun flash-attention.ts)."""
    if causal and j > i:
        return False
    if window != 0 and i >= j and i - j >= window:
        return False
    return True


def mask_matrix(rows, Lkv: int, causal: bool, window: int, cols=None) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: True where query row i may attend key j.

    cols defaults to all keys 0..Lkv-1.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = (np.arange(Lkv, dtype=np.int64) if cols is None else np.asarray(cols, dtype=np.int64))[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        ok &= j <= i
    if window != 0:
        ok &= ~((i >= j) & (i - j >= window))
    return ok


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def rows_forward(q_rows, K, V, rows, scale, causal, window, cols=None, bias_rows=None):
    """Forward for a set of query rows of one (b, h).

    q_rows [R, D], K and V [Lkv, D], rows = the R absolute row indices.
    cols (optional) = absolute key indices to evaluate; it must contain every
    allowed key of every row, and then the result is exact, because masked
    probabilities are exactly 0 (the returned S and P cover only cols).
    bias_rows (optional) [R, Lkv]: additive mask of these rows over all keys
    (finite or -inf), added to the scaled scores.
    Returns S (masked, -inf where forbidden), P, O [R, D], LSE [R].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    if cols is None:
        cols = np.arange(K.shape[0])
        Kc, Vc = K, V
    else:
        cols = np.asarray(cols)
        Kc, Vc = K[cols], V[cols]
    S = scale * (q_rows @ Kc.T)
    ok = mask_matrix(rows, K.shape[0], causal, window, cols=cols)
    if bias_rows is not None:
        bias = np.asarray(bias_rows, dtype=np.float64)[:, cols]
        if np.isnan(bias).any() or np.isposinf(bias).any():
            raise ValueError("mask values must be finite or -inf")
        ok = ok & np.isfinite(bias)
        S = S + np.where(np.isfinite(bias), bias, 0.0)
    S = np.where(ok, S, -np.inf)
    m = S.max(axis=1)
    live = np.isfinite(m)
    m0 = np.where(live, m, 0.0)
    with np.errstate(under="ignore"):
        total = np.exp(S - m0[:, None]).sum(axis=1)
    lse = np.where(live, m0 + np.log(np.where(live, total, 1.0)), -np.inf)
    lse0 = np.where(live, lse, 0.0)
    with np.errstate(under="ignore"):
        P = np.where(ok & live[:, None], np.exp(S - lse0[:, None]), 0.0)
    O = P @ Vc
    return S, P, O, lse


def key_span(rows, Lkv, causal, window):
    """Smallest contiguous key range [lo, hi] holding every allowed key of the rows
    (from the mask rule: causal caps keys at the row, a window floors them)."""
    rows = np.asarray(rows)
    lo = max(0, int(rows.min()) - window + 1) if window else 0
    hi = min(Lkv - 1, int(rows.max())) if causal else Lkv - 1
    return np.arange(lo, hi + 1) if hi >= lo else np.arange(0)


def logical_mask_bias(allowed_pairs) -> np.ndarray:
    """The numeric mask a logical mask stands for (ggmlR R/ag_flash_attn.R,
    `.ag_flash_mask`): 0 where the entry is TRUE (attention allowed), -Inf where
    it is FALSE. Any shape; float64 of the same shape, usable as `bias`."""
    m = np.asarray(allowed_pairs, dtype=bool)
    return np.where(m, 0.0, -np.inf)


def _bias(bias, B, Hq, Lq, Lkv):
    """The additive mask broadcast to [B, Hq, Lq, Lkv], or None."""
    if bias is None:
        return None
    return np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, Lq, Lkv))


def forward(q, k, v, scale, causal=False, window=0, bias=None):
    """O [B,Hq,Lq,Dv] and natural-log LSE [B,Hq,Lq] for float64 inputs (v: [B,Hkv,Lkv,Dv]).

    bias: optional additive mask broadcastable to [B, Hq, Lq, Lkv]."""
    B, Hq, Lq, D = q.shape
    Hkv = k.shape[1]
    bias = _bias(bias, B, Hq, Lq, k.shape[2])
    O = np.zeros((B, Hq, Lq, v.shape[3]))
    LSE = np.zeros((B, Hq, Lq))
    rows = np.arange(Lq)
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            _, _, O[b, h], LSE[b, h] = rows_forward(q[b, h], k[b, g], v[b, g], rows, scale, causal, window,
                                                    bias_rows=None if bias is None else bias[b, h])
    return O, LSE


def bwd_preprocess(o, do):
    """Delta [.., L] = sum over the last axis of dO * O (mlx-bun flash-attention.ts, D pre-pass)."""
    return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-1)


def backward(q, k, v, do, scale, causal=False, window=0, bias=None):
    """Gradients of f = sum(dO * O) with respect to q, k, v.

    bias: optional additive mask broadcastable to [B, Hq, Lq, Lkv] (no gradient).
    Returns dict with O, LSE, Delta, dQ, dK, dV (all float64).
    """
    B, Hq, Lq, D = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    bias = _bias(bias, B, Hq, Lq, Lkv)
    O = np.zeros((B, Hq, Lq, v.shape[3]))
    LSE = np.zeros((B, Hq, Lq))
    Delta = np.zeros((B, Hq, Lq))
    dQ = np.zeros_like(q, dtype=np.float64)
    dK = np.zeros((B, Hkv, Lkv, D))
    dV = np.zeros((B, Hkv, Lkv, v.shape[3]))
    rows = np.arange(Lq)
    for b in range(B):
        for h in range(Hq):  # heads of one group summed in increasing h
            g = _kv_head(h, Hq, Hkv)
            Kg, Vg = k[b, g], v[b, g]
            _, P, Oh, lse = rows_forward(q[b, h], Kg, Vg, rows, scale, causal, window,
                                         bias_rows=None if bias is None else bias[b, h])
            dOh = do[b, h]
            dP = dOh @ Vg.T
            delta = bwd_preprocess(Oh, dOh)
            dS = P * (dP - delta[:, None])
            dQ[b, h] = scale * (dS @ Kg)
            dK[b, g] += scale * (dS.T @ q[b, h])
            dV[b, g] += P.T @ dOh
            O[b, h], LSE[b, h], Delta[b, h] = Oh, lse, delta
    return {"O": O, "LSE": LSE, "Delta": Delta, "dQ": dQ, "dK": dK, "dV": dV}


# ---------------------------------------------------------------------------
# Row / key subsets of the same definition, for shapes too large to
# materialise whole (e.g. L = 32768): each output element needs only its own
# row of scores (O, LSE, dQ) or the rows that attend its key (dK, dV).
# ---------------------------------------------------------------------------

def sample_rows(q, k, v, do, scale, causal, window, b, h, rows):
    """O, LSE, Delta, dQ for the given query rows of (b, h), one row at a time
    over that row's allowed key span."""
    Hq, Hkv, Lkv = q.shape[1], k.shape[1], k.shape[2]
    g = _kv_head(h, Hq, Hkv)
    Kg, Vg = k[b, g], v[b, g]
    out = {"O": [], "LSE": [], "Delta": [], "dQ": []}
    for i in np.asarray(rows):
        cols = key_span([i], Lkv, causal, window)
        if len(cols) == 0:
            cols = np.arange(1)  # every key masked: a single masked column gives O = 0, LSE = -inf
        _, P, O, lse = rows_forward(q[b, h, [i]], Kg, Vg, [i], scale, causal, window, cols)
        dOr = do[b, h, [i]]
        delta = bwd_preprocess(O, dOr)
        dS = P * (dOr @ Vg[cols].T - delta[:, None])
        out["O"].append(O[0])
        out["LSE"].append(lse[0])
        out["Delta"].append(delta[0])
        out["dQ"].append(scale * (dS @ Kg[cols])[0])
    return {key: np.array(val) for key, val in out.items()}


def sample_keys(q, k, v, do, scale, causal, window, b, g, keys):
    """dK, dV for the given keys of kv head g in batch b, one key at a time.

    Every query row that may attend the key contributes, for every query head
    of the group; each such row's LSE and Delta come from its own scores over
    the key span that holds all of that row's allowed keys.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    Lq, Lkv = q.shape[2], k.shape[2]
    reps = Hq // Hkv
    Kg, Vg = k[b, g], v[b, g]
    keys = np.asarray(keys)
    dK = np.zeros((len(keys), Kg.shape[1]))
    dV = np.zeros((len(keys), Vg.shape[1]))
    for n, j in enumerate(keys):
        rows = np.nonzero(mask_matrix(np.arange(Lq), Lkv, causal, window, cols=[j])[:, 0])[0]
        if len(rows) == 0:
            continue
        cols = key_span(rows, Lkv, causal, window)
        jc = int(np.nonzero(cols == j)[0][0])
        for r in range(reps):
            h = g * reps + r
            _, P, O, _ = rows_forward(q[b, h, rows], Kg, Vg, rows, scale, causal, window, cols)
            dOr = do[b, h, rows]
            delta = bwd_preprocess(O, dOr)
            dS = P * (dOr @ Vg[cols].T - delta[:, None])
            dK[n] += scale * (dS[:, jc] @ q[b, h, rows])
            dV[n] += P[:, jc] @ dOr
    return {"dK": dK, "dV": dV}


def key_grads(q, k, v, do, scale, causal, window, b, g, keys, row_block=256, workers=1):
    """dK, dV [len(keys), D] of the given keys of kv head g in batch b, over query-row blocks.

    For each query head h of the group (increasing h) and each block of up to
    row_block consecutive query rows among those that may attend one of the
    keys: the rows' scores over the key span that holds all of their allowed
    keys (exact, since masked probabilities are 0), their LSE, P, O and
    Delta = rowsum(dO * O); then, for the requested keys, dP = dO V^T,
    dS = P (dP - Delta) and the contributions scale * dS^T Q to dK and P^T dO
    to dV. The contributions are added in (head, block) order whatever
    `workers` is; workers > 1 evaluates the blocks on that many threads (the
    matrix products and ufuncs release the interpreter lock), with the BLAS
    library held to one thread each.
    """
    Hq, Hkv, Lq, Lkv = q.shape[1], k.shape[1], q.shape[2], k.shape[2]
    reps = Hq // Hkv
    _kv_head(g * reps, Hq, Hkv)  # checks Hq % Hkv
    keys = np.asarray(keys, dtype=np.int64)
    Kg, Vg = k[b, g], v[b, g]
    sees = mask_matrix(np.arange(Lq), Lkv, causal, window, cols=keys).any(axis=1)
    rows_any = np.nonzero(sees)[0]
    blocks = [rows_any[i:i + row_block] for i in range(0, len(rows_any), row_block)]
    tasks = [(h, rows) for h in range(g * reps, (g + 1) * reps) for rows in blocks]

    def contribution(task):
        h, rows = task
        cols = key_span(rows, Lkv, causal, window)  # contiguous keys cols[0] .. cols[-1]
        _, P, O, _ = rows_forward(q[b, h, rows], Kg, Vg, rows, scale, causal, window, cols)
        dOr = np.asarray(do[b, h, rows], dtype=np.float64)
        delta = bwd_preprocess(O, dOr)
        pos = keys - cols[0]
        inside = (pos >= 0) & (pos < len(cols))
        Pk = np.zeros((len(rows), len(keys)))
        Pk[:, inside] = P[:, pos[inside]]  # keys outside the span are masked for every row
        dS = Pk * (dOr @ Vg[keys].T - delta[:, None])
        return scale * (dS.T @ q[b, h, rows]), Pk.T @ dOr

    dK = np.zeros((len(keys), Kg.shape[1]))
    dV = np.zeros((len(keys), Vg.shape[1]))
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
            parts = list(ex.map(contribution, tasks))
    else:
        parts = map(contribution, tasks)
    for pk, pv in parts:
        dK += pk
        dV += pv
    return {"dK": dK, "dV": dV}
