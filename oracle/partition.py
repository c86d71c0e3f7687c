"""Oracle: load-balanced partition of a rollout batch over K data-parallel
workers in DFS order.  TEST INFRASTRUCTURE ONLY (see the package docstring).

[DTA] section 4 (负载均衡并行化): N sequences are split into K disjoint
groups, each processed as one prefix tree T_j, minimising the largest cost
C(T_j), where C(T) is the number of tokens in the tree.  The sequences are
put in lexicographic order (the DFS order of the single tree over all of
them), so that each group is a contiguous run and loses little sharing --
at most (K - 1) times the longest sequence in extra tokens.  The smallest
feasible maximum cost tau is found by binary search between the largest
single sequence and the total, each candidate checked by a greedy scan that
opens a new group whenever the next sequence would push the current one
past tau; a group's cost is kept incrementally as sequences are added.

[TT] section 打包数据的生成 (DP 树数同步): workers synchronise their tree
counts with an all-reduce of the maximum, and a worker with fewer trees
appends empty ones.

Readings (the pages leave these open):
  - lexicographic order compares token ids as integers, a proper prefix
    first; equal sequences keep batch-row order;
  - the partition is the greedy scan at the optimal tau, so groups fill
    from the left; when it needs fewer than K groups the last ones are
    empty;
  - the tree of a group is the trie of its sequences (no token budget), so
    C(T) counts its distinct non-empty prefixes.
"""

from __future__ import annotations

import numpy as np

from .packing import OracleTrie, extract_sequences


def dfs_order(seqs: list[list[int]]) -> list[int]:
    """Indices of `seqs` in lexicographic (DFS) order, ties by index."""
    return sorted(range(len(seqs)), key=lambda i: (list(seqs[i]), i))


def tree_cost(seqs: list[list[int]]) -> int:
    """C(T): tokens of the prefix tree of `seqs`, counted by building it."""
    t = OracleTrie()
    for k, s in enumerate(seqs):
        t.insert(list(s), k)
    return t.num_tokens


def _lcp(a, b) -> int:
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


def _greedy(ordered: list[list[int]], tau: int) -> list[int] | None:
    """Group index of each sequence (in the given order) from the greedy
    scan under maximum cost tau; None if a single sequence exceeds tau."""
    groups, g, cost, prev = [], -1, 0, None
    for s in ordered:
        add = len(s) - (_lcp(s, prev) if prev is not None else 0)
        if g < 0 or cost + add > tau:
            g += 1
            cost = len(s)  # a fresh group shares nothing yet
            if cost > tau:
                return None
        else:
            cost += add
        groups.append(g)
        prev = s
    return groups


def partition(seqs: list[list[int]], K: int) -> tuple[list[int], int]:
    """(group of each sequence, optimal max cost) for K workers."""
    if K <= 0:
        raise ValueError("K must be positive")
    if not seqs:
        return [], 0
    order = dfs_order(seqs)
    ordered = [list(seqs[i]) for i in order]
    lo = max(len(s) for s in ordered)
    hi = tree_cost(ordered)
    while lo < hi:  # smallest tau whose greedy scan needs <= K groups
        mid = (lo + hi) // 2
        g = _greedy(ordered, mid)
        if g is not None and g[-1] + 1 <= K:
            hi = mid
        else:
            lo = mid + 1
    g = _greedy(ordered, lo)
    out = [0] * len(seqs)
    for pos, i in enumerate(order):
        out[i] = g[pos]
    return out, lo


def partition_batch(ids, mask, K: int) -> tuple[np.ndarray, int]:
    """partition() over the rows of a padded batch."""
    g, tau = partition(extract_sequences(np.asarray(ids), np.asarray(mask)), K)
    return np.asarray(g, dtype=np.int32), int(tau)


def dummy_tries(counts: list[int]) -> list[int]:
    """Empty tries each worker appends so all hold max(counts) (the
    all-reduce of the maximum, then padding)."""
    m = max(counts) if counts else 0
    return [m - c for c in counts]
