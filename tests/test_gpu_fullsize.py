"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: every trie of a batch laid end to end (tree_pack_concat) and run as
one tree_meta / tree_attn_fwd / tree_attn_bwd launch at 32 query / 8
key-value heads, D = 128, bf16, with bench.py's own inputs (trie t drawn with
seed 1_000_000 + t) where the host can draw them quickly.

What each workload gets, against the oracle in float32 (the precision the
target names for it):

* deep-shared 4a (one 32768-token trie) and no-sharing 4b: every row and
  every key of key/value head 0's group (query heads 0..3; 4b also head 7's
  group) elementwise -- O, LSE, dQ, dK, dV -- including every shared-prefix
  key, whose dK / dV sum over ~32K descendant rows x 4 heads; and the
  backward alone (fed the oracle's O and LSE for those heads) to the tight
  per-vector bound;
* GRPO batch 2 (24 tries, L = 191,872): every trie, one key/value head group
  per trie (head t mod 8 for trie t) elementwise, so every group is covered;
* multi-turn batch 3 (6 tries, L = 191,616): every trie, sampled rows (O,
  LSE, dQ over all 32 heads) and sampled keys (dK, dV over all 8 heads);
* the 16 points of the length x branching sweep (launches up to L =
  338,176, where the metadata kernel's scan covers several blocks per
  thread): the first and the last trie of every launch on sampled rows and
  keys, and the largest launch's position ids and tile classes bit for bit
  on its first and last trie, with every tile between tries empty.  These
  launches draw their inputs on the device (seeded) and copy them back for
  the oracle.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, announce, assert_attn_close, assert_close, bf16_ref,
                        oracle_kv_group, run_attention, torch_cuda)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _launch(torch, w, device_inputs=False, seed=0):
    """Pack, lay out and run the whole batch as one launch; returns the
    oracle's tries, offsets and host copies of inputs and outputs."""
    se, lengths, stats = pta.pack_concat(w.ids, w.mask, w.max_tokens_per_mb)
    tries = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    assert [t.L for t in tries] == lengths
    L = len(se)
    if device_inputs:
        qd, kd, vd, dod = workloads.device_attention_inputs(L, w.hq, w.hkv, w.d, w.qkv_std, seed, "cuda")
    else:
        q, k, v, do = workloads.batch_attention_inputs(lengths, w.hq, w.hkv, w.d, "bf16", w.qkv_std)
        qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
        del q, k, v, do
    meta = pta.tree_meta(se)
    o, lse, dq, dk, dv = run_attention(torch, qd, kd, vd, dod, meta)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    announce(f"  launch L={L}, {len(tries)} tries, pairs {stats['n_pairs']}")
    res = {"q": qd, "k": kd, "v": vd, "do": dod, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "meta": meta}
    for name in ("dq", "dk", "dv", "o"):
        assert bool(torch.isfinite(res[name]).all()), f"{name} has non-finite entries"
    for t, po in enumerate(tries):  # pads: zero outputs, LSE -inf
        a, b = int(offs[t]) + po.n_tokens, int(offs[t + 1])
        if b > a:
            for name in ("o", "dq", "dk", "dv"):
                assert bool((res[name][a:b] == 0).all()), f"trie {t} pad rows of {name}"
            assert bool(torch.isneginf(lse[:, a:b]).all()), f"trie {t} pad LSE"
    return tries, offs, res


def _host(x, a, b, heads=None, dtype=np.float64):
    t = x[a:b] if heads is None else x[a:b, heads]
    return t.float().cpu().numpy().astype(dtype, copy=False)


def _group_check(torch, res, po, off, kv, g, tag, alone=True):
    """Every row and key of key/value head ``kv``'s group of query heads
    against the oracle run on those heads only (a query head's output and a
    key/value head's gradients depend on no other head)."""
    a, b = int(off), int(off) + po.L
    hs = list(range(kv * g, (kv + 1) * g))
    m = oracle.dense_ancestor_mask(po)
    K = _host(res["k"], a, b, [kv])
    V = _host(res["v"], a, b, [kv])
    Qs = [_host(res["q"], a, b, [h]) for h in hs]
    Gs = [_host(res["do"], a, b, [h]) for h in hs]
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = oracle_kv_group(m, Qs, K, V, Gs, SCALE, tag)
    assert_attn_close(_host(res["o"], a, b, hs), o_ref, BF16_ATOL, BF16_RTOL, f"{tag} O")
    n = po.n_tokens
    assert_close(_host(res["lse"].T, a, b, hs).T[:, :n], lse_ref[:, :n], BF16_ATOL, BF16_RTOL, f"{tag} LSE")
    assert_attn_close(_host(res["dq"], a, b, hs), dq_ref, BF16_ATOL, BF16_RTOL, f"{tag} dQ", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(_host(res["dk"], a, b, [kv]), dk_ref, BF16_ATOL, BF16_RTOL, f"{tag} dK", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(_host(res["dv"], a, b, [kv]), dv_ref, BF16_ATOL, BF16_RTOL, f"{tag} dV")
    # two exact identities over every key of the group, bounded by the
    # oracle's magnitudes: sum_j dK_j = 0 (each dS row sums to zero) and
    # sum_j dV_j = sum_i dO_i over real rows (each P row sums to one)
    n = po.n_tokens
    dk_sum = _host(res["dk"], a, b, [kv])[:n].sum(axis=0)
    dv_sum = _host(res["dv"], a, b, [kv])[:n].sum(axis=0)
    do_sum = sum(_host(res["do"], a, b, [h])[:n].sum(axis=0) for h in hs)
    assert np.abs(dk_sum).max() <= 1e-2 * np.abs(dk_ref[:n]).sum(axis=0).max(), f"{tag} sum dK"
    assert np.abs(dv_sum - do_sum).max() <= 1e-2 * np.abs(dv_ref[:n]).sum(axis=0).max(), f"{tag} sum dV"
    if not alone:
        return
    # the backward alone: heads hs get the oracle's O (bf16) and LSE, the
    # oracle's backward runs on exactly those values
    o_in = res["o"].clone()
    lse_in = res["lse"].clone()
    o_in[a:b, hs[0]:hs[-1] + 1] = torch.from_numpy(o_ref).to(torch.bfloat16).cuda()
    lse_in[hs[0]:hs[-1] + 1, a:b] = torch.from_numpy(lse_ref).float().cuda()
    dq2, dk2, dv2 = (torch.full_like(t, float("nan")) for t in (res["dq"], res["dk"], res["dv"]))
    pta.attn_bwd(res["q"], res["k"], res["v"], o_in, lse_in, res["do"], res["meta"], dq=dq2, dk=dk2, dv=dv2)
    torch.cuda.synchronize()
    ob = _host(o_in, a, b, hs)
    lb = lse_in[hs[0]:hs[-1] + 1, a:b].double().cpu().numpy()
    dq_ref = np.zeros_like(dq_ref)
    dk_ref = np.zeros_like(dk_ref)
    dv_ref = np.zeros_like(dv_ref)
    for x, h in enumerate(hs):
        Q = _host(res["q"], a, b, [h])
        G = _host(res["do"], a, b, [h])
        q1, k1, v1 = oracle.attention_backward(Q, K, V, ob[:, x:x + 1], lb[x:x + 1], G, m, SCALE, dtype=np.float32)
        dq_ref[:, x] = q1[:, 0]
        dk_ref += k1
        dv_ref += v1
    assert_attn_close(_host(dq2, a, b, hs), dq_ref, BF16_ATOL, BF16_RTOL, f"{tag} dQ (backward alone)")
    assert_attn_close(_host(dk2, a, b, [kv]), dk_ref, BF16_ATOL, BF16_RTOL, f"{tag} dK (backward alone)")
    assert_attn_close(_host(dv2, a, b, [kv]), dv_ref, BF16_ATOL, BF16_RTOL, f"{tag} dV (backward alone)")


def _sample_rows(po, rng, n_random):
    n = po.n_tokens
    rows = {0, n - 1, int(po.node_start[min(1, po.n_nodes - 1)]), int(po.node_end[min(1, po.n_nodes - 1)])}
    rows.update(int(x) for x in rng.integers(0, n, n_random))
    return sorted(rows)


def _sample_keys(po, rng, n_keys, max_desc):
    """Keys with at most ``max_desc`` descendants, the first of them a key
    with a branch below it where there is one (a shared key)."""
    keys = []
    shared = [int(po.node_end[v]) for v in range(po.n_nodes) if len(po.nodes[v].children) > 1]
    for j in shared[::-1] + [int(x) for x in rng.permutation(po.n_tokens)]:
        dsc = oracle.descendants_of(po, j)
        if len(dsc) <= max_desc and j not in [k for k, _ in keys]:
            keys.append((j, dsc))
        if len(keys) == n_keys:
            break
    return keys


def _sampled_check(res, po, off, tag, rng, n_random=4, n_keys=3, max_desc=48):
    a, b = int(off), int(off) + po.L
    Q, K, V, G = (_host(res[x], a, b, dtype=np.float32) for x in ("q", "k", "v", "do"))
    rows = _sample_rows(po, rng, n_random)
    anc = [oracle.ancestors_of(po, i) for i in rows]
    o_ref, lse_ref = oracle.attention_forward_rows(Q, K, V, rows, anc, SCALE, dtype=np.float32)
    dq_ref = oracle.attention_dq_rows(Q, K, V, G, rows, anc, SCALE, dtype=np.float32)
    gr = [a + r for r in rows]
    assert_attn_close(bf16_ref(res["o"][gr].cpu()), o_ref, BF16_ATOL, BF16_RTOL, f"{tag} O rows")
    assert_close(res["lse"][:, gr].cpu().numpy(), lse_ref, BF16_ATOL, BF16_RTOL, f"{tag} LSE rows")
    assert_attn_close(bf16_ref(res["dq"][gr].cpu()), dq_ref, BF16_ATOL, BF16_RTOL, f"{tag} dQ rows",
                      E2E_GRAD_VEC_FLOOR)
    picked = _sample_keys(po, rng, n_keys, max_desc)
    cols = [j for j, _ in picked]
    dk_ref, dv_ref = oracle.attention_dkdv_cols(Q, K, V, G, cols, [d for _, d in picked],
                                                lambda i: oracle.ancestors_of(po, i), SCALE, dtype=np.float32)
    gc = [a + j for j in cols]
    assert_attn_close(bf16_ref(res["dk"][gc].cpu()), dk_ref, BF16_ATOL, BF16_RTOL, f"{tag} dK keys",
                      E2E_GRAD_VEC_FLOOR)
    assert_attn_close(bf16_ref(res["dv"][gc].cpu()), dv_ref, BF16_ATOL, BF16_RTOL, f"{tag} dV keys")


def _meta_check(res, po, off, tag):
    a, b = int(off), int(off) + po.L
    m = oracle.dense_ancestor_mask(po)
    pos = res["meta"].pos[a:b].cpu().numpy()
    assert (pos == oracle.position_ids(m)).all(), f"{tag} position ids"
    b0, b1 = a // 128, b // 128
    tc = res["meta"].tile_class[b0:b1, b0:b1].cpu().numpy()
    assert (tc == oracle.tile_classes(m)).all(), f"{tag} tile classes"


@pytest.mark.timeout(900)
def test_deep_shared_4a_kv_group_elementwise():
    torch = torch_cuda()
    w = workloads.make_workload("4a")
    announce("full 4a (one launch, bench inputs)")
    tries, offs, res = _launch(torch, w)
    _meta_check(res, tries[0], 0, "4a")
    _group_check(torch, res, tries[0], 0, 0, w.hq // w.hkv, "4a kv0")
    _sampled_check(res, tries[0], 0, "4a all heads", np.random.default_rng(40))


@pytest.mark.timeout(600)
def test_no_sharing_4b_kv_groups_elementwise():
    torch = torch_cuda()
    w = workloads.make_workload("4b")
    announce("full 4b (one launch, bench inputs)")
    tries, offs, res = _launch(torch, w)
    _meta_check(res, tries[0], 0, "4b")
    for kv in (0, 7):
        _group_check(torch, res, tries[0], 0, kv, w.hq // w.hkv, f"4b kv{kv}")


@pytest.mark.timeout(900)
def test_grpo_2_every_trie_one_kv_group():
    torch = torch_cuda()
    w = workloads.make_workload("2")
    announce("full config 2 (one launch of every trie, bench inputs)")
    tries, offs, res = _launch(torch, w)
    g = w.hq // w.hkv
    for t, po in enumerate(tries):
        if t in (0, len(tries) - 1):
            _meta_check(res, po, offs[t], f"2[{t}]")
        _group_check(torch, res, po, offs[t], t % w.hkv, g, f"2[{t}] kv{t % w.hkv}", alone=(t == 0))
    nb = res["meta"].tile_class.shape[0]
    _cross_trie_tiles_empty(res, offs, nb)


def _cross_trie_tiles_empty(res, offs, nb):
    tc = res["meta"].tile_class.cpu().numpy()
    inside = np.zeros((nb, nb), bool)
    for a, b in zip(offs[:-1] // 128, offs[1:] // 128):
        inside[a:b, a:b] = True
    assert not tc[~inside].any(), "a tile across tries is not empty"


@pytest.mark.timeout(600)
def test_multiturn_3_every_trie_sampled():
    torch = torch_cuda()
    w = workloads.make_workload("3")
    announce("full config 3 (one launch of every trie, bench inputs)")
    tries, offs, res = _launch(torch, w)
    rng = np.random.default_rng(33)
    for t, po in enumerate(tries):
        _sampled_check(res, po, offs[t], f"3[{t}]", rng, n_random=6, n_keys=4, max_desc=64)
    _cross_trie_tiles_empty(res, offs, res["meta"].tile_class.shape[0])


SWEEP = [(L_, b) for L_ in (8192, 16384, 32768, 65536) for b in (1, 2, 4, 8)]


@pytest.mark.timeout(900)
def test_sweep_every_point_first_and_last_trie():
    torch = torch_cuda()
    rng = np.random.default_rng(55)
    for L_, b in SWEEP:
        w = workloads.sweep_workload(L_, b)
        announce(f"sweep L={L_} b={b} (one launch, device-drawn inputs)")
        tries, offs, res = _launch(torch, w, device_inputs=True, seed=L_ * 10 + b)
        for t in sorted({0, len(tries) - 1}):
            _sampled_check(res, tries[t], offs[t], f"L{L_}-b{b}[{t}]", rng, n_random=3, n_keys=2, max_desc=32)
        if (L_, b) == (65536, 8):  # the largest launch: metadata bit for bit
            assert offs[-1] == 338_176
            for t in (0, len(tries) - 1):
                _meta_check(res, tries[t], offs[t], f"L{L_}-b{b}[{t}]")
            _cross_trie_tiles_empty(res, offs, res["meta"].tile_class.shape[0])
        del res
        torch.cuda.empty_cache()
