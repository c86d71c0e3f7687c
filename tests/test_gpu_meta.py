"""tree_meta on the GPU vs the oracle: position ids and tile classes bit for
bit, and the tile lists / orders consistent with the oracle's classes."""

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import announce, dkdv_workgroups, key_groups_ref, meta_layout, small_cases, torch_cuda

pytestmark = pytest.mark.gpu


def _check_trie(torch, p_lib, p_or, tag):
    announce(f"meta {tag} L={p_lib.L}")
    meta = pta.tree_meta(p_lib.subtree_end)
    torch.cuda.synchronize()
    m = oracle.dense_ancestor_mask(p_or)
    pos_ref = oracle.position_ids(m)
    tc_ref = oracle.tile_classes(m)
    # per 64-key chunk: first and last query that sees any of its keys
    n64 = p_lib.L // 64
    seen_by = m.reshape(p_lib.L, n64, 64).any(2)  # [query, chunk]
    seen = [np.nonzero(seen_by[:, c])[0] for c in range(n64)]
    del seen_by
    del m
    pos = meta.pos.cpu().numpy()
    tc = meta.tile_class.cpu().numpy()
    assert (pos == pos_ref).all(), f"{tag}: position ids differ at {np.nonzero(pos != pos_ref)[0][:8]}"
    assert (tc == tc_ref).all(), f"{tag}: tile classes differ at {np.argwhere(tc != tc_ref)[:8]}"
    # tile lists: ascending nonempty tiles with their partial flag, both ways
    lay = meta_layout(p_lib.L)
    ws = meta.ws.view(torch.int32).cpu().numpy()
    nb = lay["nb"]
    rp = ws[lay["row_ptr"]:lay["row_ptr"] + nb + 1]
    cp = ws[lay["col_ptr"]:lay["col_ptr"] + nb + 1]
    for qb in range(nb):
        ent = ws[lay["row_ent"] + rp[qb]:lay["row_ent"] + rp[qb + 1]]
        kbs = np.nonzero(tc_ref[qb])[0]
        assert (ent >> 1).tolist() == kbs.tolist()
        assert ((ent & 1) == (tc_ref[qb, kbs] == 1)).all()
    for kb in range(nb):
        ent = ws[lay["col_ent"] + cp[kb]:lay["col_ent"] + cp[kb + 1]]
        qbs = np.nonzero(tc_ref[:, kb])[0]
        assert (ent >> 1).tolist() == qbs.tolist()
        assert ((ent & 1) == (tc_ref[qbs, kb] == 1)).all()
    cc = (tc_ref != 0).sum(0)
    qo = ws[lay["q_order"]:lay["q_order"] + nb]
    ko = ws[lay["k_order"]:lay["k_order"] + nb]
    assert qo.tolist() == list(range(nb - 1, -1, -1))
    assert ko.tolist() == sorted(range(nb), key=lambda x: (-cc[x], x))
    # dK/dV key groups: the chunk maxima and the grouping rule, bit for bit,
    # and (from the oracle's mask) every query that sees a group's keys lies
    # in the query steps the kernel walks for it, first chunk .. hi / 64
    hi_ref, starts, _ = key_groups_ref(p_lib.subtree_end)
    assert ws[lay["hi64"]:lay["hi64"] + n64].tolist() == hi_ref.tolist()
    ng = int(ws[lay["hdr"] + 3])
    assert ng == len(starts) and ng <= dkdv_workgroups(n64)
    ends = starts[1:] + [n64]
    ghi = {c: int(hi_ref[c:e].max()) for c, e in zip(starts, ends)}
    steps = {c: (ghi[c] // 64 - c + 1 if ghi[c] >= 0 else 0) for c in starts}
    want = [c | ((e - c - 1) << 14) for c, e in sorted(zip(starts, ends), key=lambda g: (-steps[g[0]], g[0]))]
    assert ws[lay["g_order"]:lay["g_order"] + ng].tolist() == want
    for c, e in zip(starts, ends):
        assert 1 <= e - c <= 4
        q = np.concatenate(seen[c:e])
        if q.size:
            assert q.min() >= 64 * c and q.max() <= 64 * (ghi[c] // 64) + 63, f"group at chunk {c}"
        else:
            assert ghi[c] == -1, f"group at chunk {c} has keys but no query sees them"
    assert ws[lay["hdr"] + 2] == p_or.n_tokens


@pytest.mark.parametrize("case", list(range(6)))
def test_meta_small(case):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    tl, _ = pta.pack(ids, mask, M)
    to = oracle.pack(ids, mask, M)
    for t, (a, b) in enumerate(zip(tl, to)):
        _check_trie(torch, a, b, f"{name}[{t}]")


@pytest.mark.parametrize("config", ["1", "2", "4a", "4b"])
def test_meta_configs(config):
    torch = torch_cuda()
    w = workloads.make_workload(config)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    for t in range(min(len(tl), 3)):
        _check_trie(torch, tl[t], to[t], f"config{config}[{t}]")


def test_meta_pad_to_maximum_and_largest_length():
    torch = torch_cuda()
    ids, mask = workloads.worked_example()
    tl, _ = pta.pack(ids, mask, 1024, pad_to_maximum=True)
    to = oracle.pack(ids, mask, 1024, pad_to_maximum=True)
    _check_trie(torch, tl[0], to[0], "example-padmax")
    w = workloads.sweep_workload(65536, 8)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    _check_trie(torch, tl[0], to[0], "sweep-L65536-b8[0]")
