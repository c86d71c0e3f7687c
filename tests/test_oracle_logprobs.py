"""Pins of the oracle's tree log-probability / entropy gather against things
other than itself:

* library routines -- every sequence's predictions equal
  ``-torch.nn.functional.cross_entropy`` (and
  ``torch.distributions.Categorical(...).entropy()``) over the logits rows of
  its own packed positions, taken flat from the packer's sequence intervals,
  with labels from the input batch (no node walk, no cache);
* closed forms -- uniform logits give log-probability -log V and entropy
  log V everywhere; logits that are the logs of a normalised probability
  table give exactly log of the table entry, and the table's entropy
  (``scipy.stats.entropy``);
* layout -- l - 1 predictions per row, the padding value after them, rows in
  batch order across several tries; duplicated and prefix-sharing sequences
  get identical values where their predictions coincide.
"""

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import workloads


def _batch(seed, n_seq=7, max_len=30, vocab=4, M=1024):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_seq):
        if seqs and rng.random() < 0.7:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(1, len(base) + 1))
            tail = rng.integers(0, vocab, int(rng.integers(0 if cut > 1 else 1, max_len)))
            s = np.concatenate([base[:cut], tail]).astype(np.int32)
        else:
            s = rng.integers(0, vocab, int(rng.integers(1, max_len))).astype(np.int32)
        seqs.append(s)
    ids, mask = workloads.pad_rows(seqs)
    return seqs, ids, mask, oracle.pack(ids, mask, M)


def _rand_logits(tries, V, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(t.L, V, generator=g, dtype=torch.float64).numpy() * 3.0 for t in tries]


@pytest.mark.parametrize("seed", range(6))
def test_matches_cross_entropy_per_sequence(seed):
    V = 64  # > every token id of the batch
    if seed % 2:  # more, less-shared sequences in 128-token tries: several tries
        seqs, ids, mask, tries = _batch(seed, n_seq=14, vocab=50, M=128)
        assert len(tries) >= 2
    else:
        seqs, ids, mask, tries = _batch(seed)
    lg = _rand_logits(tries, V, seed)
    B, S = ids.shape
    logp, ent = oracle.gather_tree_logprobs_entropy(tries, lg, B, S, padding_value=-7.0)
    seen = set()
    for t, trie in enumerate(tries):
        for k, row in enumerate(trie.seq_ids):
            pos = trie.sequence_indices(k)
            seq = seqs[int(row)]
            assert (trie.token_ids[pos] == seq).all()
            x = torch.from_numpy(lg[t][pos[:-1]])
            y = torch.from_numpy(seq[1:].astype(np.int64))
            ref = -torch.nn.functional.cross_entropy(x, y, reduction="none").numpy()
            refe = torch.distributions.Categorical(logits=x).entropy().numpy()
            n = len(seq) - 1
            np.testing.assert_allclose(logp[row, :n], ref, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(ent[row, :n], refe, rtol=1e-12, atol=1e-12)
            assert (logp[row, n:] == -7.0).all() and (ent[row, n:] == -7.0).all()
            seen.add(int(row))
    assert seen == set(range(B))


def test_uniform_logits_closed_form():
    V = 37
    seqs, ids, mask, tries = _batch(11, n_seq=9)
    lg = [np.zeros((t.L, V)) for t in tries]
    logp, ent = oracle.gather_tree_logprobs_entropy(tries, lg, ids.shape[0], ids.shape[1], padding_value=0.0)
    for r, s in enumerate(seqs):
        n = len(s) - 1
        np.testing.assert_allclose(logp[r, :n], -np.log(V), rtol=0, atol=1e-13)
        np.testing.assert_allclose(ent[r, :n], np.log(V), rtol=0, atol=1e-13)
        assert (logp[r, n:] == 0).all()


def test_worked_example_probability_table():
    # [TT] packing figure: Seq0 [A,B,C,D], Seq1 [A,B,E,F], Seq2 [A,G,H] with
    # ids A..H = 1..8.  Logits row p = log q_p with q_p(v) proportional to
    # (v + 1) (p + 2): each prediction's log-probability is log q_p(label)
    ids, mask = workloads.worked_example()
    (trie,) = oracle.pack(ids, mask, 128)
    V = 9
    q = np.array([[(v + 1.0) * (p + 2.0) for v in range(V)] for p in range(trie.L)])
    q /= q.sum(1, keepdims=True)
    logp, ent = oracle.gather_tree_logprobs_entropy([trie], [np.log(q)], 3, ids.shape[1], padding_value=0.0)
    # packed positions (Appendix of the layout): A0 B1 C2 D3 E4 F5 G6 H7
    expect = {0: [(0, 2), (1, 3), (2, 4)],   # A->B, B->C, C->D
              1: [(0, 2), (1, 5), (4, 6)],   # A->B, B->E, E->F
              2: [(0, 7), (6, 8)]}           # A->G, G->H
    for r, pairs in expect.items():
        for j, (p, label) in enumerate(pairs):
            assert logp[r, j] == pytest.approx(np.log(q[p, label]), abs=1e-13)
            assert ent[r, j] == pytest.approx(scipy.stats.entropy(q[p]), abs=1e-13)
        assert (logp[r, len(pairs):] == 0).all()


def test_shared_and_duplicate_sequences_agree():
    seqs = [np.array([5, 1, 2, 3, 4], np.int32), np.array([5, 1, 2, 3, 4], np.int32),
            np.array([5, 1, 2, 9, 9, 9], np.int32), np.array([7], np.int32)]
    ids, mask = workloads.pad_rows(seqs)
    tries = oracle.pack(ids, mask, 128)
    lg = _rand_logits(tries, 10, 3)
    logp, ent = oracle.gather_tree_logprobs_entropy(tries, lg, 4, ids.shape[1], padding_value=0.0)
    assert (logp[0] == logp[1]).all() and (ent[0] == ent[1]).all()
    # the first three predictions (of 1, 2, 3 / 9) share predicting positions
    assert (logp[0, :2] == logp[2, :2]).all() and (ent[0, :3] == ent[2, :3]).all()
    assert logp[0, 2] != logp[2, 2]  # same position, different label
    assert (logp[3] == 0).all()  # one token: nothing to predict


def test_minus_inf_logits_are_excluded():
    # a -inf logit is probability 0: entropy and log-probabilities equal those
    # of the distribution over the remaining entries (scipy.stats.entropy of
    # the renormalised table)
    ids, mask = workloads.worked_example()
    (trie,) = oracle.pack(ids, mask, 128)
    V = 12
    rng = np.random.default_rng(4)
    lg = rng.normal(size=(trie.L, V))
    lg[:, 9:] = -np.inf  # ids are 1..8, so every label stays finite
    logp, ent = oracle.gather_tree_logprobs_entropy([trie], [lg], 3, ids.shape[1])
    for r, pairs in {0: [(0, 2), (1, 3), (2, 4)], 2: [(0, 7), (6, 8)]}.items():
        for j, (p, label) in enumerate(pairs):
            q = np.exp(lg[p, :9] - lg[p, :9].max())
            q /= q.sum()
            assert logp[r, j] == pytest.approx(np.log(q[label]), abs=1e-12)
            assert ent[r, j] == pytest.approx(scipy.stats.entropy(q), abs=1e-12)
