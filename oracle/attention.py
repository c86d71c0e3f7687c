"""Oracle attention over a packed trie: naive masked softmax attention and its
closed-form gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed ([TT] packing figure: every token attends only to itself and
its ancestors; [DTA] §3 问题形式化: a prefix shared by several sequences is
processed once forward, and the gradients of all sequences through it are
accumulated into it):

    S[i, j] = scale * q_i . k_j            for j in A(i), else masked
    P[i, :] = softmax(S[i, :]);  O_i = sum_j P[i, j] v_j
    LSE_i   = ln sum_{j in A(i)} exp S[i, j]

with grouped-query heads: query head h reads key/value head h // (Hq / Hkv)
(consecutive grouping; the pages never mention GQA -- a reading).  A row with
no visible key (a pad) has O = 0 and LSE = -inf.  Backward, with
Delta_i = dO_i . O_i:

    dV_j = sum_i P[i, j] dO_i          dP[i, j] = dO_i . v_j
    dS[i, j] = P[i, j] (dP[i, j] - Delta_i)
    dQ_i = scale sum_j dS[i, j] k_j    dK_j = scale sum_i dS[i, j] q_i

dK and dV of a key/value head sum over the query heads of its group.  Shared
prefix gradients are summed over all descendant sequences automatically,
because a shared token is one row/column of the packed problem.

Rows are processed in chunks, and each chunk takes only the key columns some
row of it can see (plain column selection; no tiling logic).  Inputs are
expected already rounded to the kernel dtype and upcast; ``dtype`` selects
the arithmetic (float64 for self-checks, float32 at large sizes).
"""

from __future__ import annotations

import numpy as np


def _heads(q, k):
    L, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return L, hq, hkv, hq // hkv, d


def attention_forward(q, k, v, mask, scale, dtype=np.float64, row_chunk=256):
    """Masked softmax attention.  q [L,Hq,D], k/v [L,Hkv,D], mask bool [L,L]
    (query, key).  Returns o [L,Hq,D] and lse [Hq,L] (natural log)."""
    q = np.asarray(q, dtype)
    k = np.asarray(k, dtype)
    v = np.asarray(v, dtype)
    L, hq, hkv, g, d = _heads(q, k)
    o = np.zeros((L, hq, d), dtype)
    lse = np.full((hq, L), -np.inf, dtype)
    for r0 in range(0, L, row_chunk):
        r1 = min(L, r0 + row_chunk)
        mm = mask[r0:r1]
        cols = np.nonzero(mm.any(axis=0))[0]
        if cols.size == 0:
            continue
        mm = mm[:, cols]
        live = mm.any(axis=1)
        for h in range(hq):
            kv = h // g
            s = scale * (q[r0:r1, h] @ k[cols, kv].T)
            s = np.where(mm, s, -np.inf)
            mx = np.where(live, s.max(axis=1), 0.0)
            e = np.exp(s - mx[:, None])
            tot = e.sum(axis=1)
            p = e / np.where(live, tot, 1.0)[:, None]
            o[r0:r1, h] = p @ v[cols, kv]
            with np.errstate(divide="ignore"):
                lse[h, r0:r1] = np.where(live, mx + np.log(np.where(live, tot, 1.0)), -np.inf)
    return o, lse


def attention_backward(q, k, v, o, lse, do, mask, scale, dtype=np.float64, row_chunk=256):
    """Closed-form gradients of :func:`attention_forward`.  ``o``/``lse`` are
    the forward's outputs; dO on rows with no visible key has no effect.
    Returns dq [L,Hq,D], dk/dv [L,Hkv,D]."""
    q = np.asarray(q, dtype)
    k = np.asarray(k, dtype)
    v = np.asarray(v, dtype)
    o = np.asarray(o, dtype)
    do = np.asarray(do, dtype)
    lse = np.asarray(lse, dtype)
    L, hq, hkv, g, d = _heads(q, k)
    dq = np.zeros((L, hq, d), dtype)
    dk = np.zeros((L, hkv, d), dtype)
    dv = np.zeros((L, hkv, d), dtype)
    for r0 in range(0, L, row_chunk):
        r1 = min(L, r0 + row_chunk)
        mm = mask[r0:r1]
        cols = np.nonzero(mm.any(axis=0))[0]
        if cols.size == 0:
            continue
        mm = mm[:, cols]
        for h in range(hq):
            kv = h // g
            s = scale * (q[r0:r1, h] @ k[cols, kv].T)
            lrow = lse[h, r0:r1]
            finite = np.isfinite(lrow)
            p = np.where(mm, np.exp(s - np.where(finite, lrow, 0.0)[:, None]), 0.0)
            dv[cols, kv] += p.T @ do[r0:r1, h]
            dp = do[r0:r1, h] @ v[cols, kv].T
            delta = (do[r0:r1, h] * o[r0:r1, h]).sum(axis=1)
            ds = p * (dp - delta[:, None])
            dq[r0:r1, h] = scale * (ds @ k[cols, kv])
            dk[cols, kv] += scale * (ds.T @ q[r0:r1, h])
    return dq, dk, dv


def attention_delta(o, do, dtype=np.float64):
    """The backward's row term Delta_i = dO_i . O_i for every token and
    query head, laid out [Hq, L] like LSE.  It is the quantity the closed-form
    gradient subtracts from dP (dS = P (dP - Delta)); by the softmax identity
    it equals sum_j P[i, j] dP[i, j].  Pads (O = 0) give 0."""
    o = np.asarray(o, dtype)
    do = np.asarray(do, dtype)
    return (o * do).sum(axis=2).T.copy()


# ---------------------------------------------------------------------------
# one-row / one-column forms, for sampled checks at sizes where the dense
# problem does not fit a CPU budget.  Same definitions, one output at a time.
# ---------------------------------------------------------------------------
def _row(q, k, v, i, h, g, cols, scale, dtype):
    s = scale * (k[cols, h // g].astype(dtype) @ q[i, h].astype(dtype))
    mx = s.max()
    e = np.exp(s - mx)
    tot = e.sum()
    p = e / tot
    return s, p, p @ v[cols, h // g].astype(dtype), mx + np.log(tot)


def attention_forward_rows(q, k, v, rows, anc, scale, dtype=np.float64):
    """O and LSE of the listed rows, every head.  ``anc[t]`` is the index
    array of keys row ``rows[t]`` may see.  Returns o [n,Hq,D], lse [Hq,n]."""
    L, hq, hkv, g, d = _heads(q, k)
    o = np.zeros((len(rows), hq, d), dtype)
    lse = np.full((hq, len(rows)), -np.inf, dtype)
    for t, i in enumerate(rows):
        cols = anc[t]
        if len(cols) == 0:
            continue
        for h in range(hq):
            _, _, o[t, h], lse[h, t] = _row(q, k, v, i, h, g, cols, scale, dtype)
    return o, lse


def attention_dq_rows(q, k, v, do, rows, anc, scale, dtype=np.float64):
    """dQ of the listed rows, every head (Delta from the row's own O)."""
    L, hq, hkv, g, d = _heads(q, k)
    dq = np.zeros((len(rows), hq, d), dtype)
    for t, i in enumerate(rows):
        cols = anc[t]
        if len(cols) == 0:
            continue
        for h in range(hq):
            _, p, oi, _ = _row(q, k, v, i, h, g, cols, scale, dtype)
            doi = do[i, h].astype(dtype)
            dp = v[cols, h // g].astype(dtype) @ doi
            ds = p * (dp - doi @ oi)
            dq[t, h] = scale * (ds @ k[cols, h // g].astype(dtype))
    return dq


def attention_dkdv_cols(q, k, v, do, cols, desc, anc_fn, scale, dtype=np.float64):
    """dK and dV of the listed keys, every key/value head.  ``desc[t]`` lists
    the rows that see key ``cols[t]``; ``anc_fn(i)`` returns the keys row i
    sees (needed for that row's softmax).  Returns dk, dv [n,Hkv,D]."""
    L, hq, hkv, g, d = _heads(q, k)
    dk = np.zeros((len(cols), hkv, d), dtype)
    dv = np.zeros((len(cols), hkv, d), dtype)
    for t, j in enumerate(cols):
        for i in desc[t]:
            a = anc_fn(int(i))
            pos = int(np.searchsorted(a, j))
            for h in range(hq):
                kv = h // g
                _, p, oi, _ = _row(q, k, v, int(i), h, g, a, scale, dtype)
                doi = do[i, h].astype(dtype)
                pij = p[pos]
                dpij = doi @ v[j, kv].astype(dtype)
                dsij = pij * (dpij - doi @ oi)
                dv[t, kv] += pij * doi
                dk[t, kv] += scale * dsij * q[i, h].astype(dtype)
    return dk, dv
