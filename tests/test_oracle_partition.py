"""Pins of the oracle's DFS-order load-balanced partition against things
other than itself:

* brute force -- on small batches, the optimal maximum cost equals the
  minimum over every split of the DFS-ordered list into at most K
  contiguous runs (all compositions enumerated), and the returned groups are
  contiguous, at most K, and each within that cost;
* the cost model -- C(T) of a group counted by building its trie equals the
  number of distinct non-empty prefixes (a set of tuples);
* the pages' bounds -- K = 1 costs the whole tree; the groups' trees hold at
  most (K - 1) * (longest sequence) more tokens than the single tree; the
  optimum is at least max(longest sequence, total / K);
* the order -- Python's lexicographic list order, a proper prefix first;
* dummy tries pad every worker to the maximum count.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads


def _seqs(seed, n, vocab=3, max_len=9):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        if out and rng.random() < 0.6:
            base = out[int(rng.integers(len(out)))]
            cut = int(rng.integers(0, len(base) + 1))
            s = list(base[:cut]) + list(rng.integers(0, vocab, int(rng.integers(0 if cut else 1, max_len))))
        else:
            s = list(rng.integers(0, vocab, int(rng.integers(1, max_len))))
        out.append([int(x) for x in (s or [0])])
    return out


def _prefixes(group):
    return len({tuple(s[:k]) for s in group for k in range(1, len(s) + 1)})


def _brute(ordered, K):
    n = len(ordered)
    best = None
    for k in range(1, min(K, n) + 1):
        for cuts in itertools.combinations(range(1, n), k - 1):
            b = (0,) + cuts + (n,)
            c = max(_prefixes(ordered[b[i]:b[i + 1]]) for i in range(k))
            best = c if best is None else min(best, c)
    return best


@pytest.mark.parametrize("seed", range(30))
def test_optimal_against_brute_force(seed):
    seqs = _seqs(seed, n=int(np.random.default_rng(seed).integers(2, 9)))
    K = 1 + seed % 4
    groups, tau = oracle.partition(seqs, K)
    order = oracle.dfs_order(seqs)
    ordered = [seqs[i] for i in order]
    assert tau == _brute(ordered, K)
    g_sorted = [groups[i] for i in order]
    assert g_sorted == sorted(g_sorted) and g_sorted[0] == 0 and max(g_sorted) < K
    assert all(b - a <= 1 for a, b in zip(g_sorted, g_sorted[1:]))  # contiguous runs
    for g in set(groups):
        assert _prefixes([seqs[i] for i in range(len(seqs)) if groups[i] == g]) <= tau


def test_cost_model_and_bounds():
    for seed in range(10):
        seqs = _seqs(100 + seed, n=25, vocab=4, max_len=20)
        assert oracle.tree_cost(seqs) == _prefixes(seqs)
        total = oracle.tree_cost(seqs)
        longest = max(len(s) for s in seqs)
        _, t1 = oracle.partition(seqs, 1)
        assert t1 == total
        for K in (2, 3, 5):
            groups, tau = oracle.partition(seqs, K)
            sizes = [oracle.tree_cost([s for s, g in zip(seqs, groups) if g == j]) for j in range(K)]
            assert max(sizes) == tau  # greedy is exact at the optimum
            assert tau >= max(longest, -(-total // K))
            assert sum(sizes) <= total + (K - 1) * longest


def test_dfs_order_is_lexicographic():
    seqs = [[2, 1], [1, 2, 3], [1, 2], [1], [2], [1, 2, 3], [0, 5]]
    assert oracle.dfs_order(seqs) == [6, 3, 2, 1, 5, 4, 0]


def test_grpo_groups_stay_together():
    # config-2 shapes: a group's 8 samples share their prompt; partitioned in
    # DFS order, a group is split at most at a segment boundary, so the K
    # trees hold nearly the single tree's tokens
    w = workloads.make_workload("2")
    seqs = oracle.extract_sequences(w.ids, w.mask)
    total = oracle.tree_cost(seqs)
    for K in (2, 4, 8):
        groups, tau = oracle.partition(seqs, K)
        sizes = [oracle.tree_cost([s for s, g in zip(seqs, groups) if g == j]) for j in range(K)]
        assert sum(sizes) <= total + (K - 1) * max(len(s) for s in seqs)
        assert max(sizes) == tau


def test_dummy_tries():
    assert oracle.dummy_tries([3, 1, 3, 0]) == [0, 2, 0, 3]
    assert oracle.dummy_tries([]) == []
