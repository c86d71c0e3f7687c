"""Pins of the oracle packer against what the pages and combinatorics fix:
the worked example of the tree-training guide's packing figure, brute-force
FFD with an independent prefix-set model, sequence recovery, compression and
pre-order properties, closed-form counts for the two extreme workloads, and
the validation errors."""

import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_example_layout():
    g = _golden()
    ids, mask = workloads.worked_example()
    tries = oracle.pack(ids, mask, 128)
    assert len(tries) == g["n_tries"]
    p = tries[0]
    n = g["n_tokens"]
    assert p.n_tokens == n and p.L == g["L"]
    assert p.token_ids[:n].tolist() == g["token_ids_real"]
    assert p.node_id[:n].tolist() == g["node_id_real"]
    assert p.subtree_end[:n].tolist() == g["subtree_end_real"]
    assert (p.token_ids[n:] == 0).all() and (p.node_id[n:] == -1).all() and (p.subtree_end[n:] == -1).all()
    assert p.node_start.tolist() == g["node_start"]
    assert p.node_end.tolist() == g["node_end"]
    assert p.node_parent.tolist() == g["node_parent"]
    assert p.seq_ids.tolist() == g["seq_ids"]
    for k, ivs in enumerate(g["seq_intervals"]):
        a, b = p.seq_iv_ptr[k], p.seq_iv_ptr[k + 1]
        assert p.seq_iv[a:b].tolist() == ivs


def test_worked_example_mask_pos_tiles_accounting():
    g = _golden()
    ids, mask = workloads.worked_example()
    p = oracle.pack(ids, mask, 128)[0]
    m = oracle.dense_ancestor_mask(p)
    for i, cols in g["mask_rows_real"].items():
        assert np.nonzero(m[int(i)])[0].tolist() == cols
    assert not m[p.n_tokens:].any() and not m[:, p.n_tokens:].any()
    pos = oracle.position_ids(m)
    assert pos[:8].tolist() == g["position_ids_real"]
    assert (pos[8:] == 0).all()
    assert oracle.tile_classes(m).tolist() == g["tile_classes"]
    acc = oracle.accounting([p], [m], mask.sum(1))
    assert acc["n_pairs"] == g["n_pairs"]
    assert acc["unpacked_pairs"] == g["unpacked_pairs"]
    assert acc["tree_token_ratio"] == pytest.approx(g["tree_token_ratio_num"] / g["tree_token_ratio_den"])


def test_children_follow_insertion_order_not_token_order():
    # Relabel so that E's id is smaller than C's: a layout ordered by token id
    # would put the E-F branch first; insertion order keeps C-D first.
    A, B, C, D, E, F, G, H = 1, 2, 9, 4, 3, 6, 7, 8
    ids, mask = workloads.pad_rows([np.array(s, np.int32) for s in
                                    ([A, B, C, D], [A, B, E, F], [A, G, H])])
    p = oracle.pack(ids, mask, 128)[0]
    assert p.token_ids[:8].tolist() == [A, B, C, D, E, F, G, H]
    # and G (id 7) after B (id 2) although inserted later than B: same order
    ids2, mask2 = workloads.pad_rows([np.array(s, np.int32) for s in
                                      ([10, 20, 5], [10, 3, 4, 5])])
    p2 = oracle.pack(ids2, mask2, 128)[0]
    # the longer sequence is inserted first (FFD), so its branch comes first
    assert p2.token_ids[:6].tolist() == [10, 3, 4, 5, 20, 5]


def _prefix_set_ffd(seqs, M):
    """Independent model of FFD: a trie's token count is the number of
    distinct non-empty prefixes of the sequences in it."""
    order = sorted(range(len(seqs)), key=lambda r: (-len(seqs[r]), r))
    tries = []  # list of (set of prefixes, list of rows)
    for r in order:
        s = tuple(seqs[r])
        pre = {s[: t + 1] for t in range(len(s))}
        for st in tries:
            if len(st[0] | pre) <= M:
                st[0].update(pre)
                st[1].append(r)
                break
        else:
            tries.append((set(pre), [r]))
    return tries


def _random_batch(rng, n_seq, max_len, vocab):
    seqs = []
    for _ in range(n_seq):
        if seqs and rng.random() < 0.6:  # share a prefix with an earlier one
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            tail = rng.integers(0, vocab, int(rng.integers(0 if cut else 1, max_len - cut + 1)))
            s = np.concatenate([base[:cut], tail]).astype(np.int32)
            if len(s) == 0:
                s = np.array([1], np.int32)
        else:
            s = rng.integers(0, vocab, int(rng.integers(1, max_len + 1))).astype(np.int32)
        seqs.append(s)
    return seqs


@pytest.mark.parametrize("seed", range(40))
def test_ffd_brute_force_and_structure(seed):
    rng = np.random.default_rng(seed)
    seqs = _random_batch(rng, int(rng.integers(1, 14)), 20, 3 if seed % 2 else 6)
    M = 128 if seed % 3 else 256
    ids, mask = workloads.pad_rows(seqs)
    if seed % 5 == 0:  # non-contiguous mask rows: tokens are taken in column order
        perm_ids = np.zeros((len(seqs), ids.shape[1] * 2), np.int32)
        perm_mask = np.zeros_like(perm_ids, dtype=np.uint8)
        for r, s in enumerate(seqs):
            cols = np.sort(rng.choice(perm_ids.shape[1], len(s), replace=False))
            perm_ids[r, cols] = s
            perm_mask[r, cols] = 1
            perm_ids[r, perm_mask[r] == 0] = rng.integers(0, 50, int((perm_mask[r] == 0).sum()))
        ids, mask = perm_ids, perm_mask
    small_M = max(len(s) for s in seqs) + int(rng.integers(0, 25))
    for budget in (M, small_M):
        if budget % 128:
            tries = oracle.ffd_build_tries([list(map(int, s)) for s in seqs], budget)
            ref = _prefix_set_ffd([list(map(int, s)) for s in seqs], budget)
            assert [t.sequence_ids for t in tries] == [r for _, r in ref]
            assert [t.num_tokens for t in tries] == [len(st) for st, _ in ref]
            continue
        tries = oracle.pack(ids, mask, budget)
        ref = _prefix_set_ffd([list(map(int, s)) for s in seqs], budget)
        assert [p.seq_ids.tolist() for p in tries] == [r for _, r in ref]
        assert [p.n_tokens for p in tries] == [len(st) for st, _ in ref]
        for p in tries:
            assert p.n_tokens <= budget and p.L % 128 == 0 and p.L >= p.n_tokens
            _check_structure(p, seqs)


def _check_structure(p, seqs):
    n = p.n_tokens
    # every sequence is recovered from its intervals, in root-to-leaf order
    for k, sid in enumerate(p.seq_ids):
        idx = p.sequence_indices(k)
        assert p.token_ids[idx].tolist() == list(map(int, seqs[sid]))
        assert (np.diff(idx) > 0).all()
    # pre-order: each node's subtree is the contiguous node range after it
    se = p.subtree_end
    for v in range(p.n_nodes):
        s, e = p.node_start[v], p.node_end[v]
        assert (p.node_id[s:e + 1] == v).all()
        par = p.node_parent[v]
        if par >= 0:
            assert p.node_start[par] < s and se[s] <= se[p.node_start[par]]
    assert (np.diff(p.node_start) > 0).all() and p.node_start[0] == 0
    # no compressible pair remains: single child with identical sequence set
    for v, cn in enumerate(p.nodes):
        if len(cn.children) == 1:
            assert set(p.nodes[cn.children[0]].seqs) != set(cn.seqs)
    # the dense mask from the parent walk equals the subtree-interval rule
    m = oracle.dense_ancestor_mask(p)
    i = np.arange(p.L)[:, None]
    j = np.arange(p.L)[None, :]
    assert (m == ((j <= i) & (i <= se[None, :]))).all()
    # position id = offset of the token in every sequence through it
    pos = oracle.position_ids(m)
    for k in range(len(p.seq_ids)):
        idx = p.sequence_indices(k)
        assert (pos[idx] == np.arange(len(idx))).all()
    assert (pos[n:] == 0).all()


def test_tile_classes_brute_force_small():
    rng = np.random.default_rng(7)
    seqs = _random_batch(rng, 12, 120, 4)
    ids, mask = workloads.pad_rows(seqs)
    for p in oracle.pack(ids, mask, 1024):
        m = oracle.dense_ancestor_mask(p)
        tc = oracle.tile_classes(m)
        nb = p.L // 128
        for a in range(nb):
            for b in range(nb):
                blk = m[a * 128:(a + 1) * 128, b * 128:(b + 1) * 128]
                want = 2 if blk.sum() == blk.size else (1 if blk.sum() else 0)
                assert tc[a, b] == want


@pytest.mark.slow
def test_extreme_configs_closed_forms():
    # 4b: 16 disjoint causal sequences of 2048 = 16 blocks each
    w = workloads.make_workload("4b")
    (p,) = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    m = oracle.dense_ancestor_mask(p)
    tc = oracle.tile_classes(m)
    assert int((tc == 2).sum()) == 16 * (16 * 15 // 2) and int((tc == 1).sum()) == 16 * 16
    assert int(m.sum(dtype=np.int64)) == 16 * 2048 * 2049 // 2 == 33_570_816
    del m
    # 4a: 16384 prefix (128 blocks) + 64 leaves of 256 (2 blocks each)
    w = workloads.make_workload("4a")
    (p,) = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    m = oracle.dense_ancestor_mask(p)
    tc = oracle.tile_classes(m)
    prefix_full, prefix_partial = 128 * 127 // 2, 128
    leaf_full, leaf_partial = 2 * 128 + 1, 2
    assert int((tc == 2).sum()) == prefix_full + 64 * leaf_full
    assert int((tc == 1).sum()) == prefix_partial + 64 * leaf_partial
    n_pairs = 16384 * 16385 // 2 + 64 * (256 * 16384 + 256 * 257 // 2)
    assert int(m.sum(dtype=np.int64)) == n_pairs == 404_766_720
    acc = oracle.accounting([p], [m], w.mask.sum(1))
    assert acc["unpacked_pairs"] == 64 * 16640 * 16641 // 2
    assert acc["tree_token_ratio"] == pytest.approx(32768 / (64 * 16640))


def test_config1_is_one_trie():
    w = workloads.make_workload("1")
    tries = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    assert len(tries) == 1 and tries[0].L == 512
    _check_structure(tries[0], [w.ids[r][w.mask[r] != 0] for r in range(w.ids.shape[0])])


@pytest.mark.parametrize("pad_to_max", [False, True])
def test_padding_modes(pad_to_max):
    ids, mask = workloads.worked_example()
    (p,) = oracle.pack(ids, mask, 384, pad_to_maximum=pad_to_max, pad_id=7)
    assert p.L == (384 if pad_to_max else 128)
    assert (p.token_ids[8:] == 7).all()


def test_errors():
    ids, mask = workloads.worked_example()
    for bad, code in ((0, "max_tokens"), (-128, "max_tokens"), (None, "max_tokens"), (100, "align")):
        with pytest.raises(oracle.PackError) as e:
            oracle.pack(ids, mask, bad)
        assert e.value.code == code
    long_ids, long_mask = workloads.pad_rows([np.arange(1, 200, dtype=np.int32)])
    with pytest.raises(oracle.PackError) as e:
        oracle.pack(long_ids, long_mask, 128)
    assert e.value.code == "seq_too_long"
    mask2 = mask.copy()
    mask2[1] = 0
    with pytest.raises(oracle.PackError) as e:
        oracle.pack(ids, mask2, 128)
    assert e.value.code == "empty_seq"
