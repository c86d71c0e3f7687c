"""Pins of the oracle's prefix-order packing (sequences in lexicographic
order, the DFS order of one tree over the batch, filling tries of at most
max_tokens_per_mb tree tokens one after another), against:

* a hand-worked batch;
* an independent model that counts a trie's tokens as the distinct non-empty
  prefixes of its sequences, on random batches;
* the run structure: every trie is a contiguous run of the lexicographic
  order, and the first sequence of each trie would not have fit the one
  before (greedy maximality);
* the closed form of the total: each run costs its first sequence's length
  plus, for every later sequence, its length minus its common prefix with
  the sequence before it;
* the packed-layout properties the FFD path is held to (sequence recovery,
  pre-order, compression, mask rule, position ids);
* the validation error for an unknown order.
"""

import numpy as np
import pytest

import oracle
import workloads
from test_oracle_packing import _check_structure, _random_batch


def _prefix_set_model(seqs, M):
    order = sorted(range(len(seqs)), key=lambda r: (tuple(seqs[r]), r))
    tries = []  # (set of prefixes, rows)
    for r in order:
        s = tuple(seqs[r])
        pre = {s[: t + 1] for t in range(len(s))}
        if tries and len(tries[-1][0] | pre) <= M:
            tries[-1][0].update(pre)
            tries[-1][1].append(r)
        else:
            tries.append((set(pre), [r]))
    return tries


def _lcp(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


def test_hand_worked_batch():
    # rows 0..4; lexicographic order is rows 2, 0, 4, 1, 3
    seqs = [[1, 2, 3, 7, 8], [4, 5, 9], [1, 2, 3, 6], [4, 5, 9, 9], [1, 2, 3, 7, 9]]
    tries = oracle.prefix_order_build_tries(seqs, 8)
    # row 2 opens trie 0 (4 tokens); row 0 adds 7, 8 (6); row 4 adds 9 (7);
    # row 1 would add 3 (10 > 8) and opens trie 1 (3); row 3 adds one 9 (4)
    assert [t.sequence_ids for t in tries] == [[2, 0, 4], [1, 3]]
    assert [t.num_tokens for t in tries] == [7, 4]
    # with a budget of 11 everything fits one trie: 7 + 4 tokens, no sharing
    # across the two prompts
    one = oracle.prefix_order_build_tries(seqs, 11)
    assert [t.sequence_ids for t in one] == [[2, 0, 4, 1, 3]] and one[0].num_tokens == 11


def test_ffd_spreads_groups_prefix_order_does_not():
    # two prompts of 4 tokens with a long and a short response each, budget
    # 16: FFD (longest first) puts the two long responses of different
    # prompts in one trie and the two short ones in another, so both prompts
    # are stored twice (26 tree tokens); prefix order keeps prompt A's group
    # in one trie and stores prompt B twice only across the trie boundary
    # (22 tree tokens)
    A, B = [1] * 4, [2] * 4
    seqs = [A + [6] * 4, B + [8] * 4, A + [5], B + [7]]
    ffd = oracle.ffd_build_tries(seqs, 16)
    assert [t.sequence_ids for t in ffd] == [[0, 1], [2, 3]]
    assert [t.num_tokens for t in ffd] == [16, 10]
    pre = oracle.prefix_order_build_tries(seqs, 16)
    assert [t.sequence_ids for t in pre] == [[2, 0, 3], [1]]
    assert [t.num_tokens for t in pre] == [14, 8]


@pytest.mark.parametrize("seed", range(40))
def test_random_batches_against_prefix_set_model(seed):
    rng = np.random.default_rng(1000 + seed)
    seqs = [list(map(int, s)) for s in _random_batch(rng, int(rng.integers(1, 16)), 20, 3 if seed % 2 else 6)]
    budget = max(len(s) for s in seqs) + int(rng.integers(0, 30))
    tries = oracle.prefix_order_build_tries(seqs, budget)
    ref = _prefix_set_model(seqs, budget)
    assert [t.sequence_ids for t in tries] == [r for _, r in ref]
    assert [t.num_tokens for t in tries] == [len(st) for st, _ in ref]
    # runs of the lexicographic order, greedy, and the closed-form total
    order = oracle.dfs_order(seqs)
    assert [r for t in tries for r in t.sequence_ids] == order
    total = 0
    for k, t in enumerate(tries):
        assert t.num_tokens <= budget
        first = seqs[t.sequence_ids[0]]
        if k > 0:  # it did not fit the trie before
            assert tries[k - 1].num_tokens + len(first) - _lcp(first, seqs[tries[k - 1].sequence_ids[-1]]) > budget
        total += len(first)
        for a, b in zip(t.sequence_ids, t.sequence_ids[1:]):
            total += len(seqs[b]) - _lcp(seqs[b], seqs[a])
    assert total == sum(t.num_tokens for t in tries)


@pytest.mark.parametrize("seed", range(8))
def test_packed_layout_structure(seed):
    rng = np.random.default_rng(2000 + seed)
    seqs = _random_batch(rng, int(rng.integers(2, 14)), 60, 3)
    ids, mask = workloads.pad_rows(seqs)
    for budget in (128, 256):
        if max(len(s) for s in seqs) > budget:
            continue
        packed = oracle.pack(ids, mask, budget, order="prefix")
        ref = _prefix_set_model([list(map(int, s)) for s in seqs], budget)
        assert [p.seq_ids.tolist() for p in packed] == [r for _, r in ref]
        for p in packed:
            assert p.n_tokens <= budget and p.L % 128 == 0
            _check_structure(p, seqs)


def test_unknown_order_is_an_error():
    ids, mask = workloads.pad_rows([np.array([1, 2, 3], np.int32)])
    with pytest.raises(oracle.PackError):
        oracle.pack(ids, mask, 128, order="lpt")
