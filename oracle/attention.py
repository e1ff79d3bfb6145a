"""Plain float64 CPU definition of ragged grouped-query attention and its VJP.

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP path is
checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library never does, and it shares no
code with the library.

What is computed (sources are the pages' own words, restated):

* Page "Noncausal Global Extreme-GQA Ragged Attention Full VJP", section
  "What You Have": packed ragged sequences addressed by cumulative offsets
  ``cu_q``/``cu_k``; Q has Hq heads, K/V have Hkv heads (one on the page);
  the logit of query i and key j in a sequence is the dot product scaled by
  ``scale_multiplier / sqrt(head_dim)`` (0.75 on the page), passed through the
  soft cap ``c * tanh(x / c)`` (c = 3 on the page), then shifted by the ALiBi
  term ``-slope[b, h] * |i + Lk - Lq - j|`` with positions local to the
  sequence, and normalised by a softmax over that sequence's keys.  The page's
  cases are all noncausal with no window; its signature still carries
  ``causal``, ``window_left`` and ``window_right``.
* Same page, section "Hard Constraints": order of the logit steps is tanh
  cap first, then the ALiBi bias, then the mask; dK and dV collect the
  contributions of all query heads mapped to their K/V head; the results are
  (out, dq, dk, dv), shaped and typed like the packed inputs.
* Page "python-20261012-ragged-flash-attention-gradient-recompute", section
  "Root causes addressed": the stored row statistic is L = m + log l
  (natural log); a row with no keys has L = -inf, output 0 and gradient 0.

Readings taken where the pages are silent:
  - ``softcap == 0`` means no cap (identity); the pages always use 3.
  - head_dim in the scale is the logical feature count D (160), never the
    padded buffer width.
  - the query-head to K/V-head map is g = h // (Hq // Hkv).
  - the backward is the exact chain rule of the forward above:
        dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,  dA = P * (dP - Delta),
        dS = dA * (1 - tanh^2(S / c)),  dQ = sigma dS K,
        dK = sigma sum_h dS^T Q,  dV = sum_h P^T dO.

  - dropout (page "python-20261012-ragged-flash-attention-gradient-
    recompute", section "Root causes addressed"): the keep mask M and the
    scale 1 / (1 - p) come from oracle/dropout.py; with D = M / (1 - p) per
    row, out = (P * D) V, the statistic L is that of P (before dropout), and
    the chain rule gives dV = sum_h (P * D)^T dO, dP = (dO V^T) * D,
    Delta = rowsum(P * dP) = rowsum(dO * out), then dA, dS, dQ, dK as below.
  - masks (the pages name the arguments but never define them): key j of
    query row i is kept iff i + Lk - Lq - window_left <= j <= i + Lk - Lq +
    window_right, a negative bound meaning no limit on that side; ``causal``
    sets window_right = 0 (alignment at the bottom right, like the ALiBi
    centre).  Masking drops keys from the softmax; the cap and ALiBi are
    unchanged for the kept keys.  A row that keeps no key is a row with no
    keys (L = -inf, output and gradients 0).

Everything is dense per (sequence, head): no tiling, no online softmax, no
fusion.  Rows may be processed in chunks to bound memory; each row's softmax
still spans all of its sequence's keys, so the arithmetic is unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from . import dropout as _dropout

__all__ = ["sequence_vjp", "forward", "vjp", "rows_vjp", "window_bounds"]


def window_bounds(causal=False, window_left=-1, window_right=-1):
    """(left, right) key bounds relative to a row's centre i + Lk - Lq; -1 = none."""
    wl = int(window_left) if window_left is not None and window_left >= 0 else -1
    wr = 0 if causal else (int(window_right) if window_right is not None and window_right >= 0 else -1)
    return wl, wr


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _head_rows(Qh, K, V, dOh, i_pos, Lq, Lk, slope, softcap, sigma, want_kv, window=(-1, -1),
               drop=None):
    """Forward and VJP for one head of one sequence, rows at query positions ``i_pos``.

    Qh [n, D], dOh [n, D] (or None), K/V [Lk, D]; ``i_pos`` are the local
    query positions of those n rows.  ``drop``: None, or the dropout factors
    [n, Lk] (1 / (1 - p) where a key is kept, 0 where it is dropped).  Returns
    out, lse, and, when dOh is given, dq, delta and (if ``want_kv``) this
    head's dK/dV contributions.
    """
    n, D = Qh.shape
    out = np.zeros((n, D))
    lse = np.full(n, -np.inf)
    if dOh is None:
        res = {"out": out, "lse": lse}
    else:
        res = {"out": out, "lse": lse, "dq": np.zeros((n, D)), "delta": np.zeros(n)}
        if want_kv:
            res["dk"] = np.zeros((Lk, D))
            res["dv"] = np.zeros((Lk, D))
    if n == 0 or Lk == 0:
        # A row with no keys: L = -inf, output and gradients stay exactly zero.
        return res

    # scaled dot product
    S = sigma * (Qh @ K.T)                                   # [n, Lk]
    # soft cap before ALiBi
    if softcap > 0.0:
        U = np.tanh(S / softcap)
        T = softcap * U
    else:
        U = None
        T = S
    # ALiBi: -slope * |q_position + key_length - query_length - k_position|
    dist = np.abs(i_pos[:, None] + (Lk - Lq) - np.arange(Lk)[None, :]).astype(np.float64)
    A = T - slope * dist
    # mask: keys outside [centre - window_left, centre + window_right] leave
    # the softmax (a negative bound is no bound)
    wl, wr = window
    centre = i_pos[:, None] + (Lk - Lq)
    j = np.arange(Lk)[None, :]
    keep = np.ones((n, Lk), dtype=bool)
    if wl >= 0:
        keep &= j >= centre - wl
    if wr >= 0:
        keep &= j <= centre + wr
    A = np.where(keep, A, -np.inf)
    has = keep.any(axis=1)
    # softmax over the kept keys; a row that keeps none stays at zero
    m = np.where(has, A.max(axis=1), 0.0)[:, None]
    E = np.exp(A - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / np.where(l > 0.0, l, 1.0)
    # dropout acts on the normalised weights; L keeps the undropped statistic
    Pd = P if drop is None else P * drop
    res["out"] = Pd @ V
    res["lse"] = np.where(has, (m + np.log(np.where(l > 0.0, l, 1.0)))[:, 0], -np.inf)
    if dOh is None:
        return res

    dP = dOh @ V.T                                           # [n, Lk]
    if drop is not None:
        dP = dP * drop                                       # d out / d P of the dropped weights
    delta = (P * dP).sum(axis=1)                             # = rowsum(dO * O)
    dA = P * (dP - delta[:, None])
    dS = dA * (1.0 - U * U) if U is not None else dA
    res["dq"] = sigma * (dS @ K)
    res["delta"] = delta
    if want_kv:
        res["dk"] = sigma * (dS.T @ Qh)
        res["dv"] = Pd.T @ dOh
    return res


def sequence_vjp(Q, K, V, dO, slopes, softcap, scale_multiplier, row_chunk=4096, window=(-1, -1),
                 dropout=None):
    """Forward and full VJP of one sequence.

    Q, dO: [Lq, Hq, D]; K, V: [Lk, Hkv, D]; slopes: [Hq].  ``dO`` may be None
    (forward only).  ``dropout``: None or (seed, b, rates) with b the
    sequence's index in the batch and rates float32 [Lq, Hq] (see
    oracle/dropout.py).  Returns a dict with out [Lq,Hq,D], lse [Lq,Hq] and,
    with dO, dq [Lq,Hq,D], delta [Lq,Hq], dk/dv [Lk,Hkv,D].
    """
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    Lq, Hq, D = Q.shape
    Lk, Hkv = K.shape[0], K.shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    sigma = scale_multiplier / math.sqrt(D)
    out = np.zeros((Lq, Hq, D))
    lse = np.full((Lq, Hq), -np.inf)
    res = {"out": out, "lse": lse}
    if dO is not None:
        dO = _as_f64(dO)
        res.update(dq=np.zeros((Lq, Hq, D)), delta=np.zeros((Lq, Hq)),
                   dk=np.zeros((Lk, Hkv, D)), dv=np.zeros((Lk, Hkv, D)))
    for h in range(Hq):
        g = h // group
        for r0 in range(0, Lq, row_chunk):
            r1 = min(Lq, r0 + row_chunk)
            drop = None
            if dropout is not None:
                seed, b, rates = dropout
                drop = _dropout.keep_scale(seed, b, h, np.arange(r0, r1), Lk, rates[r0:r1, h])
            part = _head_rows(Q[r0:r1, h], K[:, g], V[:, g],
                              None if dO is None else dO[r0:r1, h],
                              np.arange(r0, r1), Lq, Lk, float(slopes[h]),
                              softcap, sigma, want_kv=True, window=window, drop=drop)
            out[r0:r1, h] = part["out"]
            lse[r0:r1, h] = part["lse"]
            if dO is not None:
                res["dq"][r0:r1, h] = part["dq"]
                res["delta"][r0:r1, h] = part["delta"]
                if "dk" in part:
                    # K/V gradients sum over every query head sharing K/V head g
                    res["dk"][:, g] += part["dk"]
                    res["dv"][:, g] += part["dv"]
    return res


def _rates(dropout_p, Tq, Hq):
    """Per-row float32 rates [Tq, Hq] from a scalar or an array, or None when
    there is no dropout (a scalar 0)."""
    if np.ndim(dropout_p) == 0:
        if float(dropout_p) == 0.0:
            return None
        return np.full((Tq, Hq), dropout_p, dtype=np.float32)
    r = np.asarray(dropout_p, dtype=np.float32)
    assert r.shape == (Tq, Hq), "per-row dropout rates must be [total_q, hq]"
    return r


def _run(q, k, v, cu_q, cu_k, alibi_slopes, dout, softcap, scale_multiplier, window=(-1, -1),
         dropout_p=0.0, dropout_seed=0):
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    slopes = _as_f64(alibi_slopes)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = k.shape
    B = len(cu_q) - 1
    assert len(cu_k) == B + 1 and slopes.shape == (B, Hq)
    rates = _rates(dropout_p, Tq, Hq)
    res = {"out": np.zeros((Tq, Hq, D)), "lse": np.full((Tq, Hq), -np.inf)}
    if dout is not None:
        dout = _as_f64(dout)
        res.update(dq=np.zeros((Tq, Hq, D)), delta=np.zeros((Tq, Hq)),
                   dk=np.zeros((Tk, Hkv, D)), dv=np.zeros((Tk, Hkv, D)))
    for b in range(B):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        part = sequence_vjp(q[q0:q1], k[k0:k1], v[k0:k1],
                            None if dout is None else dout[q0:q1],
                            slopes[b], softcap, scale_multiplier, window=window,
                            dropout=None if rates is None else (dropout_seed, b, rates[q0:q1]))
        res["out"][q0:q1] = part["out"]
        res["lse"][q0:q1] = part["lse"]
        if dout is not None:
            res["dq"][q0:q1] = part["dq"]
            res["delta"][q0:q1] = part["delta"]
            res["dk"][k0:k1] = part["dk"]
            res["dv"][k0:k1] = part["dv"]
    return res


def forward(q, k, v, cu_q, cu_k, alibi_slopes, softcap, scale_multiplier, causal=False,
            window_left=-1, window_right=-1, dropout_p=0.0, dropout_seed=0):
    """out [Tq,Hq,D] and lse [Tq,Hq] (natural log) for a packed ragged batch.
    dropout_p: a float32 rate in [0, 1) or per-row rates [Tq, Hq]."""
    res = _run(q, k, v, cu_q, cu_k, alibi_slopes, None, softcap, scale_multiplier,
               window_bounds(causal, window_left, window_right), dropout_p, dropout_seed)
    return res["out"], res["lse"]


def vjp(q, k, v, cu_q, cu_k, alibi_slopes, dout, softcap, scale_multiplier, causal=False,
        window_left=-1, window_right=-1, dropout_p=0.0, dropout_seed=0):
    """Forward plus full VJP; dict with out, dq, dk, dv, lse, delta (float64)."""
    return _run(q, k, v, cu_q, cu_k, alibi_slopes, dout, softcap, scale_multiplier,
                window_bounds(causal, window_left, window_right), dropout_p, dropout_seed)


def rows_vjp(Q, K, V, dO, slopes, softcap, scale_multiplier, tokens, heads, causal=False,
             window_left=-1, window_right=-1, dropout=None):
    """out, lse, dq, delta for selected rows of one sequence.

    Each row's result depends only on its own q/dout row and the sequence's
    K/V, so a sample of rows can be checked at any sequence length.  ``tokens``
    and ``heads`` are equal-length integer arrays of local query positions and
    head indices.  ``dropout`` as in sequence_vjp.  Returns arrays shaped
    [n, D] / [n].
    """
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    dO = _as_f64(dO)
    Lq, Hq, D = Q.shape
    Lk, Hkv = K.shape[0], K.shape[1]
    group = Hq // Hkv
    sigma = scale_multiplier / math.sqrt(D)
    tokens = np.asarray(tokens, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    n = len(tokens)
    res = {"out": np.zeros((n, D)), "lse": np.full(n, -np.inf),
           "dq": np.zeros((n, D)), "delta": np.zeros(n)}
    for h in np.unique(heads):
        sel = np.nonzero(heads == h)[0]
        g = int(h) // group
        drop = None
        if dropout is not None:
            seed, b, rates = dropout
            drop = _dropout.keep_scale(seed, b, int(h), tokens[sel], Lk, rates[tokens[sel], h])
        part = _head_rows(Q[tokens[sel], h], K[:, g], V[:, g], dO[tokens[sel], h],
                          tokens[sel], Lq, Lk, float(slopes[h]), softcap, sigma,
                          want_kv=False,
                          window=window_bounds(causal, window_left, window_right), drop=drop)
        for key in res:
            res[key][sel] = part[key]
    return res

