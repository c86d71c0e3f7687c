"""Pins of the oracle's depth-first (DTA) execution against things other
than itself: its outputs equal the dense-mask oracle's (a different route to
the same attention: per-node attention over a stack of ancestor keys instead
of a masked softmax over the whole trie) at several chunk lengths, including
chunks shorter than a node; the stack's peak holds exactly the longest
root-to-node path over internal nodes (closed forms on the worked example and
the deep-shared workload); leaves' keys are never pushed; the number of
forward and backward chunks is sum over nodes of ceil(tokens / chunk)."""

import math

import numpy as np
import pytest

import oracle
import workloads


def _inputs(p, hq=4, hkv=2, d=16, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(p.L, hq, d)) / math.sqrt(d) ** 0.5
    k = rng.normal(size=(p.L, hkv, d)) / math.sqrt(d) ** 0.5
    v = rng.normal(size=(p.L, hkv, d))
    do = rng.normal(size=(p.L, hq, d))
    return q, k, v, do


def _check_against_dense(p, chunk, seed):
    q, k, v, do = _inputs(p, seed=seed)
    scale = 0.37
    m = oracle.dense_ancestor_mask(p)
    o_ref, lse_ref = oracle.attention_forward(q, k, v, m, scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(q, k, v, o_ref, lse_ref, do, m, scale)
    o, lse, dq, dk, dv, st = oracle.dfs_attention(p, q, k, v, do, scale, chunk=chunk)
    n = p.n_tokens
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[:, :n], lse_ref[:, :n], rtol=1e-12, atol=1e-12)
    assert np.isneginf(lse[:, n:]).all()
    for x, r in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(x, r, rtol=1e-9, atol=1e-11)
    sizes = p.node_end.astype(np.int64) - p.node_start + 1
    assert st["fwd_chunks"] == st["bwd_chunks"] == int(sum(-(-s // chunk) for s in sizes))
    return st


@pytest.mark.parametrize("chunk", [2048, 64, 7, 1])
def test_small_workloads_equal_dense(chunk):
    cases = [workloads.worked_example() + (128,)] + [workloads.small_workload(k) for k in
                                                    ("nested", "deep-small", "multiturn-small")]
    for c, (ids, mask, M) in enumerate(cases):
        for t, p in enumerate(oracle.pack(ids, mask, M)):
            _check_against_dense(p, chunk, 10 * c + t)


@pytest.mark.parametrize("seed", range(12))
def test_random_tries_equal_dense(seed):
    rng = np.random.default_rng(500 + seed)
    seqs = []
    for _ in range(int(rng.integers(1, 12))):
        if seqs and rng.random() < 0.7:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(1, len(base) + 1))
            seqs.append(np.concatenate([base[:cut], rng.integers(0, 3, int(rng.integers(1, 30)))]).astype(np.int32))
        else:
            seqs.append(rng.integers(0, 3, int(rng.integers(1, 40))).astype(np.int32))
    ids, mask = workloads.pad_rows(seqs)
    for p in oracle.pack(ids, mask, 1024):
        _check_against_dense(p, int(rng.choice([3, 16, 2048])), seed)


def test_stack_holds_the_longest_internal_path():
    # worked example: internal nodes {A} and {B} (path A, B); leaves are not pushed
    ids, mask = workloads.worked_example()
    (p,) = oracle.pack(ids, mask, 128)
    st = _check_against_dense(p, 2048, 1)
    assert st["peak_stack_tokens"] == 2 and st["max_path_tokens"] == 4
    # deep-shared: the 16384-token prefix is the only internal node
    w = workloads.make_workload("4a")
    (p,) = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    q = np.zeros((p.L, 1, 2))
    _, _, _, _, _, st = oracle.dfs_attention(p, q, np.zeros((p.L, 1, 2)), np.zeros((p.L, 1, 2)), q, 1.0)
    assert st["peak_stack_tokens"] == 16384 and st["max_path_tokens"] == 16384 + 256
    assert st["fwd_chunks"] == 16384 // 2048 + 64
