"""Oracle: depth-first (DTA) execution of tree attention over one packed
trie.  TEST INFRASTRUCTURE ONLY (see the package docstring).

[DTA] §3.1 (前缀树的深度优先搜索遍历): the trie is walked depth first while a
stack holds the current root-to-node path -- its tokens and their key/value
cache.  Entering an internal node pushes it: its tokens are run forward
against the keys on the stack and their keys/values are appended.  At a leaf
(a whole sequence) the forward is finished and the loss gradient is injected
at once, so the branch's backward starts immediately.  Leaving a node pops
it: its backward runs, the gradients of every sequence below it having been
accumulated into its keys while the branches were visited, and then its
tokens leave the stack.  [DTA] §3.2 (系统优化): the forward/backward of a long
node is cut into chunks of at most ``chunk`` tokens (2048 in the notes), and
a leaf's keys/values are never kept on the stack (only a prefix can be
attended to later).

Attention alone (one layer, Q/K/V/dO given per packed token) is what this
computes, with the pages' attention semantics: a token attends to the keys
of its ancestors (the stack) and to its own node's tokens up to itself.  The
results are therefore exactly those of :mod:`oracle.attention` on the dense
ancestor mask -- a different route to the same numbers, which is what pins
this module.  It also reports the schedule's quantities that depend only on
the trie: the peak number of tokens on the stack (the longest root-to-node
path over internal nodes) and the number of forward and backward chunks.

Reading (the notes leave it open): children are visited in the trie's
pre-order (insertion order); the notes' greedy ordering heuristic is not
modelled.  Backward chunks of a node run in the same order as its forward
chunks.  The forward of an internal node runs when it is pushed; its backward
when it is popped.
"""

from __future__ import annotations

import numpy as np


def _children(p):
    kids = [[] for _ in range(p.n_nodes)]
    roots = []
    for v in range(p.n_nodes):  # node indices are pre-order, so lists stay ordered
        par = int(p.node_parent[v])
        (roots if par < 0 else kids[par]).append(v)
    return roots, kids


def _attend(q, k, v, do, o_rows, lse_rows, rows, keys, scale, dtype, backward):
    """Forward (backward=False) or backward of query ``rows`` (a contiguous
    run of one node) over ``keys`` (stack keys, then the node's own rows up
    to each query).  Returns (o, lse) or (dq, dk, dv contributions)."""
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    own0 = int(rows[0])
    n_anc = int(np.sum(keys < own0))
    # query t (row rows[t]) sees every ancestor key and own keys <= rows[t]
    vis = np.ones((len(rows), len(keys)), bool)
    vis[:, n_anc:] = keys[None, n_anc:] <= rows[:, None]
    out = []
    if not backward:
        o = np.zeros((len(rows), hq, q.shape[2]), dtype)
        lse = np.zeros((hq, len(rows)), dtype)
        for h in range(hq):
            s = scale * (q[rows, h] @ k[keys, h // g].T)
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1)
            e = np.exp(s - mx[:, None])
            tot = e.sum(axis=1)
            o[:, h] = (e / tot[:, None]) @ v[keys, h // g]
            lse[h] = mx + np.log(tot)
        return o, lse
    dq = np.zeros((len(rows), hq, q.shape[2]), dtype)
    dk = np.zeros((len(keys), hkv, q.shape[2]), dtype)
    dv = np.zeros((len(keys), hkv, q.shape[2]), dtype)
    for h in range(hq):
        kv = h // g
        s = scale * (q[rows, h] @ k[keys, kv].T)
        pr = np.where(vis, np.exp(s - lse_rows[h][:, None]), 0.0)
        dp = do[rows, h] @ v[keys, kv].T
        delta = (do[rows, h] * o_rows[:, h]).sum(axis=1)
        ds = pr * (dp - delta[:, None])
        dq[:, h] = scale * (ds @ k[keys, kv])
        dk[:, kv] += scale * (ds.T @ q[rows, h])
        dv[:, kv] += pr.T @ do[rows, h]
    out = (dq, dk, dv)
    return out


def dfs_attention(p, q, k, v, do, scale, chunk: int = 2048, dtype=np.float64):
    """Tree attention forward and backward of trie ``p`` by depth-first
    execution.  q / do [L, Hq, D], k / v [L, Hkv, D] (rounded inputs,
    upcast).  Returns (o, lse, dq, dk, dv, stats) with the layouts of
    :mod:`oracle.attention`; stats = {"peak_stack_tokens", "fwd_chunks",
    "bwd_chunks", "max_path_tokens"}."""
    q, k, v, do = (np.asarray(x, dtype) for x in (q, k, v, do))
    L, hq, d = q.shape
    hkv = k.shape[1]
    o = np.zeros((L, hq, d), dtype)
    lse = np.full((hq, L), -np.inf, dtype)
    dq = np.zeros((L, hq, d), dtype)
    dk = np.zeros((L, hkv, d), dtype)
    dv = np.zeros((L, hkv, d), dtype)
    roots, kids = _children(p)
    stack: list[int] = []  # nodes on the current path whose keys are kept
    st = {"peak_stack_tokens": 0, "fwd_chunks": 0, "bwd_chunks": 0, "max_path_tokens": 0}

    def stack_keys():
        if not stack:
            return np.zeros(0, np.int64)
        return np.concatenate([np.arange(int(p.node_start[u]), int(p.node_end[u]) + 1) for u in stack])

    def chunks(vn):
        a, b = int(p.node_start[vn]), int(p.node_end[vn]) + 1
        return [np.arange(c, min(c + chunk, b)) for c in range(a, b, chunk)]

    def forward(vn, anc):
        own = np.arange(int(p.node_start[vn]), int(p.node_end[vn]) + 1)
        for rows in chunks(vn):
            keys = np.concatenate([anc, own[own <= rows[-1]]])
            o[rows], lse[:, rows] = _attend(q, k, v, do, None, None, rows, keys, scale, dtype, False)
            st["fwd_chunks"] += 1

    def backward(vn, anc):
        own = np.arange(int(p.node_start[vn]), int(p.node_end[vn]) + 1)
        for rows in chunks(vn):
            keys = np.concatenate([anc, own[own <= rows[-1]]])
            gq, gk, gv = _attend(q, k, v, do, o[rows], lse[:, rows], rows, keys, scale, dtype, True)
            dq[rows] = gq
            dk[keys] += gk  # accumulated into the keys' gradients (stack and own)
            dv[keys] += gv
            st["bwd_chunks"] += 1

    def visit(vn):
        anc = stack_keys()
        n_own = int(p.node_end[vn]) - int(p.node_start[vn]) + 1
        st["max_path_tokens"] = max(st["max_path_tokens"], len(anc) + n_own)
        forward(vn, anc)
        if not kids[vn]:  # leaf: inject the gradient now; its keys are never pushed
            backward(vn, anc)
            return
        stack.append(vn)  # push: its keys/values join the path
        st["peak_stack_tokens"] = max(st["peak_stack_tokens"], len(anc) + n_own)
        for c in kids[vn]:
            visit(c)
        backward(vn, anc)  # every descendant's gradient is in; backprop the node
        stack.pop()

    for r in roots:
        visit(r)
    return o, lse, dq, dk, dv, st
