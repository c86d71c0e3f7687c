"""Host-side tests of libtreeattn: the library loads and exports every symbol
include/tree_attn.h declares, the C++ packer matches the oracle bit for bit
on every generator and on random batches, and argument errors carry the
codes the header documents.  No device compute is issued here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from prefix_tree_attention_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tree_attn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pta.library_path()):
        from prefix_tree_attention_amd import build
        build.build()
    return pta.lib()


def test_exports_every_declared_symbol(L):
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(tree_[a-z_0-9]+)\s*\(", text, re.M))
    assert {"tree_pack", "tree_meta", "tree_attn_fwd", "tree_attn_bwd", "tree_last_error"} <= names
    for n in sorted(names):
        assert hasattr(L, n), n
    assert set(_lib.SIGNATURES) == names
    assert L.tree_abi_version() == 7


def _compare(tries_lib, tries_or):
    assert len(tries_lib) == len(tries_or)
    for a, b in zip(tries_lib, tries_or):
        assert a.n_tokens == b.n_tokens and a.L == b.L
        for f in ("token_ids", "node_id", "subtree_end", "node_start", "node_end", "node_parent", "seq_ids",
                  "seq_iv_ptr", "seq_iv"):
            x, y = getattr(a, f), getattr(b, f)
            assert x.shape == y.shape and (x == y).all(), f


def _stats_vs_oracle(stats, tries_or, w_mask):
    lens = np.asarray(w_mask).astype(bool).sum(1)
    assert stats["n_tries"] == len(tries_or)
    assert stats["original_tokens"] == int(lens.sum())
    assert stats["tree_tokens"] == sum(p.n_tokens for p in tries_or)
    assert stats["unpacked_pairs"] == int((lens.astype(np.int64) * (lens + 1) // 2).sum())


def test_worked_example(L):
    ids, mask = workloads.worked_example()
    tl, st = pta.pack(ids, mask, 128)
    to = oracle.pack(ids, mask, 128)
    _compare(tl, to)
    assert st["n_pairs"] == 22 and st["unpacked_pairs"] == 26
    assert st["tree_token_ratio"] == pytest.approx(8 / 11)
    assert (st["tiles_full"], st["tiles_partial"], st["tiles_causal"]) == (0, 1, 1)


def _tiles_vs_oracle(st, masks):
    tcs = [oracle.tile_classes(m) for m in masks]
    assert st["tiles_full"] == sum(int((t == 2).sum()) for t in tcs)
    assert st["tiles_partial"] == sum(int((t == 1).sum()) for t in tcs)
    assert st["tiles_causal"] == sum(t.shape[0] * (t.shape[0] + 1) // 2 for t in tcs)


@pytest.mark.parametrize("config", ["1", "2", "3", "4a", "4b"])
def test_configs_bit_exact(L, config):
    w = workloads.make_workload(config)
    tl, st = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    _compare(tl, to)
    _stats_vs_oracle(st, to, w.mask)
    if config == "4a":  # closed forms: prefix 128 blocks, 64 leaves of 2 blocks
        assert st["n_pairs"] == 404_766_720
        assert st["tiles_full"] == 128 * 127 // 2 + 64 * (2 * 128 + 1)
        assert st["tiles_partial"] == 128 + 64 * 2 and st["tiles_causal"] == 256 * 257 // 2
    if config == "4b":  # 16 disjoint causal sequences of 16 blocks
        assert st["n_pairs"] == 33_570_816
        assert st["tiles_full"] == 16 * (16 * 15 // 2) and st["tiles_partial"] == 16 * 16
        assert 1 - (st["tiles_full"] + st["tiles_partial"]) / st["tiles_causal"] == pytest.approx(0.93385, abs=1e-5)
    if config in ("1", "2"):
        _tiles_vs_oracle(st, [oracle.dense_ancestor_mask(p) for p in to])


@pytest.mark.parametrize("L_,b", [(8192, 1), (8192, 8), (16384, 2), (16384, 4)])
def test_sweep_points_bit_exact(L, L_, b):
    w = workloads.sweep_workload(L_, b)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    _compare(tl, oracle.pack(w.ids, w.mask, w.max_tokens_per_mb))


@pytest.mark.parametrize("seed", range(60))
def test_random_batches_bit_exact(L, seed):
    rng = np.random.default_rng(1000 + seed)
    n_seq = int(rng.integers(1, 30))
    vocab = int(rng.choice([2, 3, 5, 50]))
    seqs = []
    for _ in range(n_seq):
        if seqs and rng.random() < 0.6:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            tail = rng.integers(0, vocab, int(rng.integers(0 if cut else 1, 90)))
            s = np.concatenate([base[:cut], tail]).astype(np.int32)
        else:
            s = rng.integers(0, vocab, int(rng.integers(1, 120))).astype(np.int32)
        seqs.append(s if len(s) else np.array([0], np.int32))
    ids, mask = workloads.pad_rows(seqs)
    M = int(rng.choice([128, 256, 512]))
    M = max(M, -(-max(len(s) for s in seqs) // 128) * 128)
    pad_max = bool(seed % 3 == 0)
    tl, st = pta.pack(ids, mask, M, pad_to_maximum=pad_max, pad_id=seed % 7)
    to = oracle.pack(ids, mask, M, pad_to_maximum=pad_max, pad_id=seed % 7)
    _compare(tl, to)
    masks = [oracle.dense_ancestor_mask(p) for p in to]
    acc = oracle.accounting(to, masks, mask.sum(1))
    assert st["n_pairs"] == acc["n_pairs"]
    _tiles_vs_oracle(st, masks)


@pytest.mark.parametrize("config", ["1", "2", "3", "4a", "4b"])
def test_prefix_order_configs_bit_exact(L, config):
    w = workloads.make_workload(config)
    tl, st = pta.pack(w.ids, w.mask, w.max_tokens_per_mb, order="prefix")
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb, order="prefix")
    _compare(tl, to)
    _stats_vs_oracle(st, to, w.mask)
    # the layout of every trie is the same as if its rows were packed alone
    for p in to:
        rows = p.seq_ids
        alone = oracle.pack(w.ids[rows], w.mask[rows], w.max_tokens_per_mb, order="prefix")
        assert len(alone) == 1 and alone[0].n_tokens == p.n_tokens


@pytest.mark.parametrize("L_,b", [(8192, 1), (8192, 8), (16384, 4)])
def test_prefix_order_sweep_points_bit_exact(L, L_, b):
    w = workloads.sweep_workload(L_, b)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb, order="prefix")
    _compare(tl, oracle.pack(w.ids, w.mask, w.max_tokens_per_mb, order="prefix"))


@pytest.mark.parametrize("seed", range(30))
def test_prefix_order_random_batches_bit_exact(L, seed):
    rng = np.random.default_rng(5000 + seed)
    seqs = []
    for _ in range(int(rng.integers(1, 30))):
        if seqs and rng.random() < 0.6:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            tail = rng.integers(0, 4, int(rng.integers(0 if cut else 1, 90)))
            s = np.concatenate([base[:cut], tail]).astype(np.int32)
        else:
            s = rng.integers(0, 4, int(rng.integers(1, 120))).astype(np.int32)
        seqs.append(s if len(s) else np.array([0], np.int32))
    ids, mask = workloads.pad_rows(seqs)
    M = max(int(rng.choice([128, 256])), -(-max(len(s) for s in seqs) // 128) * 128)
    tl, _ = pta.pack(ids, mask, M, pad_to_maximum=bool(seed % 2), pad_id=seed % 5, order="prefix")
    _compare(tl, oracle.pack(ids, mask, M, pad_to_maximum=bool(seed % 2), pad_id=seed % 5, order="prefix"))


def test_prefix_order_unknown_order(L):
    ids, mask = workloads.worked_example()
    h = ctypes.c_void_p()
    rc = L.tree_pack_ordered(np.ascontiguousarray(ids, np.int32).ctypes.data,
                             np.ascontiguousarray(mask, np.uint8).ctypes.data, ids.shape[0], ids.shape[1], 128, 128,
                             0, 0, 2, ctypes.byref(h))
    assert rc == -5 and not h.value and "unknown order" in L.tree_last_error().decode()
    with pytest.raises(pta.TreeAttnError):
        pta.pack(ids, mask, 128, order="lpt")


def test_error_codes_match_oracle(L):
    ids, mask = workloads.worked_example()
    cases = [(0, "max_tokens", -1), (-128, "max_tokens", -1), (100, "align", -2)]
    for M, ocode, lcode in cases:
        with pytest.raises(oracle.PackError) as eo:
            oracle.pack(ids, mask, M)
        assert eo.value.code == ocode
        with pytest.raises(pta.TreeAttnError) as el:
            pta.pack(ids, mask, M)
        assert el.value.code == lcode and pta.lib().tree_last_error()
    long_ids, long_mask = workloads.pad_rows([np.arange(1, 200, dtype=np.int32)])
    with pytest.raises(pta.TreeAttnError) as el:
        pta.pack(long_ids, long_mask, 128)
    assert el.value.code == -3
    m2 = mask.copy()
    m2[2] = 0
    with pytest.raises(pta.TreeAttnError) as el:
        pta.pack(ids, m2, 128)
    assert el.value.code == -4
    with pytest.raises(pta.TreeAttnError) as el:
        pta.pack(ids, mask, 128, block_size=64)
    assert el.value.code == -5


def test_device_entry_points_validate_before_launch(L):
    # bad arguments are rejected on the host, before any device work
    assert L.tree_meta_workspace_bytes(100) == 0 and L.tree_meta_workspace_bytes(0) == 0
    assert L.tree_meta_workspace_bytes(1024) > 0
    assert L.tree_meta(None, 1024, None, None, None, 0, None) == -5
    assert L.tree_meta(None, 1000, None, None, None, 0, None) == -5
    p = ctypes.c_void_p(256)
    ws = L.tree_meta_workspace_bytes(1024)
    assert L.tree_meta(p, 1024, p, p, p, ws - 1, None) == -6
    args = [p] * 7
    assert L.tree_attn_fwd(*args, 1024, 6, 4, 128, 0.1, 0, None) == -5   # Hq % Hkv
    assert L.tree_attn_fwd(*args, 1024, 8, 2, 96, 0.1, 0, None) == -5    # D
    assert L.tree_attn_fwd(*args, 1024, 8, 2, 128, 0.1, 7, None) == -5   # dtype
    assert L.tree_attn_fwd(*args, 1000, 8, 2, 128, 0.1, 0, None) == -5   # L % 128
    assert L.tree_attn_fwd(ctypes.c_void_p(257), *args[1:], 1024, 8, 2, 128, 0.1, 0, None) == -5  # alignment
    need = L.tree_attn_bwd_workspace_bytes(1024, 8, 128, 0)
    assert need >= 1024 * 8 * 4
    assert L.tree_attn_bwd(*([p] * 12), need - 1, 1024, 8, 2, 128, 0.1, 0, None) == -6
    assert b"workspace" in L.tree_last_error()
    # the static-scratch backward: its size limit and argument checks come
    # before any device call
    assert L.tree_attn_bwd_noalloc(*([p] * 11), 1 << 20, 16, 2, 128, 0.1, 0, None) == -5
    assert b"static scratch" in L.tree_last_error()
    limit = pta.BWD_STATIC_SCRATCH_BYTES // 8  # L * Hq rows that fit
    assert L.tree_attn_bwd_workspace_bytes(limit // 32, 32, 128, 0) == pta.BWD_STATIC_SCRATCH_BYTES
    assert L.tree_attn_bwd_noalloc(*([p] * 11), limit // 32 + 128, 32, 8, 128, 0.1, 0, None) == -5
    assert L.tree_attn_bwd_noalloc(*([p] * 11), 1024, 6, 4, 128, 0.1, 0, None) == -5   # Hq % Hkv
    assert L.tree_attn_bwd_noalloc(*([p] * 10), None, 1024, 8, 2, 128, 0.1, 0, None) == -5  # NULL


def _oracle_concat(to):
    parts, off = [], 0
    for t in to:
        se = np.asarray(t.subtree_end, dtype=np.int64).copy()
        se[se >= 0] += off
        parts.append(se)
        off += t.L
    return np.concatenate(parts).astype(np.int32)


@pytest.mark.parametrize("config", ["1", "2", "3", "4b"])
def test_concat_layout_bit_exact(L, config):
    """tree_pack_concat lays the oracle's tries end to end with shifted
    subtree ends, and the concatenation is a packed layout of its own: the
    oracle's position ids and tile classes on it equal each trie's own on
    the trie's block range, and every tile across tries is empty."""
    w = workloads.make_workload(config)
    se, lengths, stats = pta.pack_concat(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    assert lengths == [t.L for t in to]
    assert (se == _oracle_concat(to)).all()
    assert stats["n_tries"] == len(to)


def test_concat_is_a_packed_layout(L):
    # per-trie metadata reproduced inside the concatenation (small batch so
    # the dense oracle mask of the whole concatenation stays small)
    ids, mask, M = next(c for c in small_cases_cpu() if c[0] == "grpo-small")[1:]  # three tries
    to = oracle.pack(ids, mask, M)
    assert len(to) > 1
    se, lengths, _ = pta.pack_concat(ids, mask, M)
    n = len(se)
    # dense ancestor mask of the concatenation from its subtree intervals
    j = np.arange(n)
    vis = (j[None, :] <= j[:, None]) & (j[:, None] <= se[None, :])
    pos_cat = np.where(se >= 0, vis.sum(1) - 1, 0)
    off = 0
    for t in to:
        m = oracle.dense_ancestor_mask(t)
        assert (pos_cat[off:off + t.L] == oracle.position_ids(m)).all()
        assert not vis[off:off + t.L, :off].any() and not vis[off:off + t.L, off + t.L:].any()
        off += t.L


def small_cases_cpu():
    for kind in workloads.SMALL_KINDS:
        ids, mask, M = workloads.small_workload(kind)
        yield kind, ids, mask, M


def test_concat_errors(L):
    w = workloads.make_workload("1")
    ids = np.ascontiguousarray(w.ids, dtype=np.int32)
    mask = np.ascontiguousarray(w.mask, dtype=np.uint8)
    h = ctypes.c_void_p()
    assert L.tree_pack(ids.ctypes.data, mask.ctypes.data, ids.shape[0], ids.shape[1], w.max_tokens_per_mb,
                       128, 0, 0, ctypes.byref(h)) == 0
    try:
        total = ctypes.c_int64()
        assert L.tree_pack_concat(h, None, 0, None) == -5
        assert L.tree_pack_concat(None, None, 0, ctypes.byref(total)) == -5
        assert L.tree_pack_concat(h, None, 0, ctypes.byref(total)) == 0 and total.value > 0
        buf = np.zeros(total.value, np.int32)
        assert L.tree_pack_concat(h, buf.ctypes.data, total.value - 1, ctypes.byref(total)) == -5
        assert b"capacity" in L.tree_last_error()
        assert L.tree_pack_concat(h, buf.ctypes.data, total.value, ctypes.byref(total)) == 0
    finally:
        L.tree_pack_free(h)


def _oracle_rows(to, B, S):
    """Packed (concatenated) position of each row's k-th token, from the
    oracle's tries and sequence intervals; -1 after the row's length."""
    rp = np.full((B, S), -1, np.int64)
    tok = []
    off = 0
    for t in to:
        for k, row in enumerate(t.seq_ids):
            pos = t.sequence_indices(k) + off
            rp[int(row), :len(pos)] = pos
        tok.append(t.token_ids)
        off += t.L
    return rp, np.concatenate(tok)


@pytest.mark.parametrize("config", ["1", "2", "3", "4b"])
def test_row_positions_and_ids_bit_exact(L, config):
    w = workloads.make_workload(config)
    se, tok, rp, lengths, _ = pta.pack_batch(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    rp_o, tok_o = _oracle_rows(to, *w.ids.shape)
    assert (rp == rp_o).all() and (tok == tok_o).all() and (se == _oracle_concat(to)).all()
    # each row's positions hold its own tokens, in order
    for r in range(w.ids.shape[0]):
        n = int(w.mask[r].astype(bool).sum())
        assert (tok[rp[r, :n]] == w.ids[r][w.mask[r].astype(bool)]).all()


def test_logprob_entry_points_validate_before_launch(L):
    p = ctypes.c_void_p(256)
    assert L.tree_logits_stats(p, 100, 0, 0, p, p, None) == -5          # V
    assert L.tree_logits_stats(p, 100, 50, 7, p, p, None) == -5         # dtype
    assert L.tree_logits_stats(None, 100, 50, 0, p, p, None) == -5      # NULL
    assert L.tree_logits_stats(ctypes.c_void_p(257), 10, 50, 0, p, p, None) == -5  # misaligned bf16
    assert L.tree_logits_stats(None, 0, 50, 0, None, None, None) == 0   # empty
    assert L.tree_gather_logprobs(p, 100, 50, 0, p, p, p, p, -1, 4, 0.0, p, p, None) == -5
    assert L.tree_gather_logprobs(p, 100, 50, 0, p, p, p, None, 2, 4, 0.0, p, p, None) == -5
    assert L.tree_gather_logprobs(None, 0, 50, 0, None, None, None, None, 0, 4, 0.0, None, None, None) == 0
    g = L.tree_gather_logprobs_rows
    assert g(p, 90, 20, 100, 50, 0, p, p, p, p, 2, 4, 0.0, p, p, None) == -5     # window past L
    assert b"rows [90, 110) outside [0, 100)" in L.tree_last_error()
    assert g(p, -1, 20, 100, 50, 0, p, p, p, p, 2, 4, 0.0, p, p, None) == -5     # negative start
    assert g(p, 0, -1, 100, 50, 0, p, p, p, p, 2, 4, 0.0, p, p, None) == -5      # negative rows
    assert g(None, 0, 20, 100, 50, 0, p, p, p, p, 2, 4, 0.0, p, p, None) == -5   # rows but no logits
    assert g(p, 0, 20, 100, 50, 3, p, p, p, p, 2, 4, 0.0, p, p, None) == -5      # dtype
    assert g(None, 0, 0, 100, 50, 0, p, p, p, p, 0, 4, 0.0, p, p, None) == 0     # empty batch
    h = ctypes.c_void_p()
    ids, mask = workloads.worked_example()
    ids = np.ascontiguousarray(ids, np.int32)
    mask = np.ascontiguousarray(mask, np.uint8)
    assert L.tree_pack(ids.ctypes.data, mask.ctypes.data, ids.shape[0], ids.shape[1], 128, 128, 0, 0,
                       ctypes.byref(h)) == 0
    try:
        buf = np.zeros(ids.size, np.int32)
        assert L.tree_pack_row_positions(h, buf.ctypes.data, ids.size - 1) == -5
        assert L.tree_pack_concat_ids(h, buf.ctypes.data, 127) == -5
    finally:
        L.tree_pack_free(h)


@pytest.mark.parametrize("config", ["1", "2", "3", "4a", "4b"])
@pytest.mark.parametrize("K", [1, 2, 3, 8])
def test_partition_bit_exact(L, config, K):
    w = workloads.make_workload(config)
    g, tau, costs = pta.partition(w.ids, w.mask, K)
    go, tauo = oracle.partition_batch(w.ids, w.mask, K)
    assert (g == go).all() and tau == tauo
    seqs = oracle.extract_sequences(w.ids, w.mask)
    for j in range(K):
        assert costs[j] == oracle.tree_cost([s for s, x in zip(seqs, g) if x == j])


@pytest.mark.parametrize("seed", range(40))
def test_partition_random_bit_exact(L, seed):
    rng = np.random.default_rng(7000 + seed)
    n_seq = int(rng.integers(1, 40))
    vocab = int(rng.choice([2, 3, 7]))
    seqs = []
    for _ in range(n_seq):
        if seqs and rng.random() < 0.6:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            s = np.concatenate([base[:cut], rng.integers(0, vocab, int(rng.integers(0 if cut else 1, 30)))])
        else:
            s = rng.integers(0, vocab, int(rng.integers(1, 40)))
        seqs.append(s.astype(np.int32))
    ids, mask = workloads.pad_rows(seqs)
    K = int(rng.integers(1, 10))
    g, tau, costs = pta.partition(ids, mask, K)
    go, tauo = oracle.partition_batch(ids, mask, K)
    assert (g == go).all() and tau == tauo


def test_partition_errors(L):
    ids, mask = workloads.worked_example()
    with pytest.raises(pta.TreeAttnError) as e:
        pta.partition(ids, mask, 0)
    assert e.value.code == -5
    g, tau, costs = pta.partition(ids, mask, 5)  # more workers than rows
    assert tau == 4 and g.tolist() == [0, 1, 2] and costs.tolist() == [4, 4, 3, 0, 0]  # one row per worker


def _dfs_cases():
    ids, mask = workloads.worked_example()
    yield "worked-example", ids, mask, 128
    for kind in workloads.SMALL_KINDS:
        ids, mask, M = workloads.small_workload(kind)
        yield kind, ids, mask, M
    for c in ("1", "2", "4a", "4b"):
        w = workloads.make_workload(c)
        yield f"config{c}", w.ids, w.mask, w.max_tokens_per_mb


@pytest.mark.parametrize("chunk", [128, 2048])
def test_dfs_plan_stack_matches_oracle(L, chunk):
    """tree_dfs_plan's stack peak and longest path equal the depth-first
    oracle's (the schedule's quantities that do not depend on how leaves are
    batched); the frame holds the stack's node segments from 128-aligned
    rows plus the leaf rows."""
    for name, ids, mask, M in _dfs_cases():
        tl, _ = pta.pack(ids, mask, M)
        for t, (pl, po) in enumerate(zip(tl, oracle.pack(ids, mask, M))):
            plan = pta.dfs_plan(pl, chunk)
            z = np.zeros((po.L, 1, 2))
            st = oracle.dfs_attention(po, z, z, z, z, 1.0, chunk=chunk)[5] if po.L <= 8192 else None
            if st is not None:
                assert plan["peak_stack_tokens"] == st["peak_stack_tokens"], (name, t)
                assert plan["max_path_tokens"] == st["max_path_tokens"], (name, t)
            assert plan["rows"] % 256 == 0 and plan["rows"] >= plan["stack_rows"]
            assert plan["leaf_rows"] >= max(chunk, 1) and plan["leaf_rows"] % 128 == 0
    w = workloads.make_workload("4a")
    (pl,), _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    plan = pta.dfs_plan(pl, 2048)
    assert plan["peak_stack_tokens"] == 16384 and plan["max_path_tokens"] == 16640 and plan["max_depth"] == 1
    assert plan["rows"] == 16384 + 8192 and plan["leaf_groups"] == 2 and plan["chunks"] == 8 + 2


def test_dfs_entry_points_validate(L):
    ids, mask = workloads.worked_example()
    (pl,), _ = pta.pack(ids, mask, 128)
    with pytest.raises(pta.TreeAttnError, match="chunk"):
        pta.dfs_plan(pl, 100)
    bad = pta.PackedTrie(**{**pl.__dict__, "node_start": pl.node_start + 1})
    with pytest.raises(pta.TreeAttnError, match="pre-order"):
        pta.dfs_plan(bad, 2048)
    bad = pta.PackedTrie(**{**pl.__dict__, "node_parent": np.full_like(pl.node_parent, 7)})
    with pytest.raises(pta.TreeAttnError, match="parent"):
        pta.dfs_plan(bad, 2048)
    # worked example nodes {A} {B} {C,D} {E,F} {G,H}: parents -1 0 1 1 0.  {G,H}
    # under {C,D}, or {E,F} under {B} after {C,D} moved to the root's children,
    # names a parent that the pre-order walk has already left
    assert list(pl.node_parent) == [-1, 0, 1, 1, 0]
    for par in ([-1, 0, 1, 1, 2], [-1, 0, 0, 1, 0]):
        bad = pta.PackedTrie(**{**pl.__dict__, "node_parent": np.array(par, np.int32)})
        with pytest.raises(pta.TreeAttnError, match="pre-order path"):
            pta.dfs_plan(bad, 2048)
    p = ctypes.c_void_p(256)
    ns, ne, npar = (np.ascontiguousarray(x, np.int32) for x in (pl.node_start, pl.node_end, pl.node_parent))
    args = [ns.ctypes.data, ne.ctypes.data, npar.ctypes.data, ns.size, pl.n_tokens]
    # bad heads and a missing workspace are rejected before any device work
    assert L.tree_attn_dfs(*args, *([p] * 10), None, 1 << 30, 128, 6, 4, 128, 0.1, 2048, None) == -5
    assert L.tree_attn_dfs(*args, *([p] * 10), p, 0, 128, 8, 2, 128, 0.1, 2048, None) == -6
