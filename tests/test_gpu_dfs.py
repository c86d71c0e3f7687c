"""Depth-first (DTA) execution on the GPU (tree_attn_dfs) against the
oracle: the same attention and gradients as the packed-trie path, reached by
walking the trie with a stack of the path's keys.  Elementwise on every
scaled-down trie at two chunk lengths (128, so nodes and leaf groups run in
several chunks, and 2048) and two head shapes, with NaN-filled outputs; the
deep-shared workload at full size on key/value head 0's group (every
shared-prefix key, whose gradient is accumulated on the stack over 64 leaf
groups' launches); and sampled rows and keys of every trie of the
multi-turn batch.  Also: the oracle's depth-first model and the dense one
agree (pinned on the CPU), so both are the reference here."""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, announce, assert_attn_close, assert_close, bf16_ref,
                        oracle_kv_group, small_cases, torch_cuda)

pytestmark = pytest.mark.gpu


def _run(torch, pl, q, k, v, do, chunk):
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    nan = float("nan")
    outs = dict(o=torch.full_like(qd, nan), lse=torch.full((qd.shape[1], pl.L), nan, device="cuda"),
                dq=torch.full_like(qd, nan), dk=torch.full_like(kd, nan), dv=torch.full_like(vd, nan))
    plan = pta.dfs_plan(pl, chunk)
    o, lse, dq, dk, dv = pta.attn_dfs(pl, qd, kd, vd, dod, meta, chunk=chunk, **outs)
    torch.cuda.synchronize()
    return plan, o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("chunk", [128, 2048])
@pytest.mark.parametrize("shape", [(8, 2, 128), (4, 1, 64)])
@pytest.mark.parametrize("case", list(range(6)))
def test_dfs_small_elementwise(case, shape, chunk):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    hq, hkv, d = shape
    tl, _ = pta.pack(ids, mask, M)
    for t, (pl, po) in enumerate(zip(tl, oracle.pack(ids, mask, M))):
        q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, "bf16", 1.0 / math.sqrt(d), 800 + case + t)
        plan, o, lse, dq, dk, dv = _run(torch, pl, q, k, v, do, chunk)
        announce(f"dfs {name}[{t}] L={pl.L} chunk={chunk} hq={hq} d={d}: {plan}")
        scale = 1.0 / math.sqrt(d)
        Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
        m = oracle.dense_ancestor_mask(po)
        o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
        dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
        n = po.n_tokens
        tag = f"dfs {name}[{t}] chunk {chunk}"
        assert_attn_close(bf16_ref(o), o_ref, BF16_ATOL, BF16_RTOL, f"{tag} O")
        assert_close(lse.numpy()[:, :n], lse_ref[:, :n], BF16_ATOL, BF16_RTOL, f"{tag} LSE")
        assert np.isneginf(lse.numpy()[:, n:]).all()
        assert_attn_close(bf16_ref(dq), dq_ref, BF16_ATOL, BF16_RTOL, f"{tag} dQ", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dk), dk_ref, BF16_ATOL, BF16_RTOL, f"{tag} dK", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dv), dv_ref, BF16_ATOL, BF16_RTOL, f"{tag} dV")
        for x in (o, dq, dk, dv):
            assert (x[n:].float() == 0).all()


def test_dfs_matches_packed_path_and_repeats_bit_for_bit():
    """Same inputs through tree_attn_fwd/bwd and tree_attn_dfs: O and dQ of a
    leaf run in the same kernels on the same keys; every output agrees to the
    bf16 tolerance, and a second depth-first run repeats the first exactly."""
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("multiturn-small")
    (pl,), _ = pta.pack(ids, mask, M)
    q, k, v, do = workloads.attention_inputs(pl.L, 8, 2, 128, "bf16", 1.0 / math.sqrt(128), 901)
    r1 = _run(torch, pl, q, k, v, do, 256)[1:]
    r2 = _run(torch, pl, q, k, v, do, 256)[1:]
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    dq, dk, dv = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
    torch.cuda.synchronize()
    for name, a, b in zip(("O", "dQ", "dK", "dV"), (r1[0], r1[2], r1[3], r1[4]), (o, dq, dk, dv)):
        assert_attn_close(bf16_ref(a), bf16_ref(b.cpu()), BF16_ATOL, BF16_RTOL, f"dfs vs packed {name}")


@pytest.mark.timeout(900)
def test_dfs_deep_shared_4a_kv_group():
    torch = torch_cuda()
    w = workloads.make_workload("4a")
    (pl,), _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    (po,) = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    q, k, v, do = workloads.attention_inputs(pl.L, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 1_000_000)
    plan, o, lse, dq, dk, dv = _run(torch, pl, q, k, v, do, 2048)
    announce(f"dfs 4a: {plan}")
    assert plan["peak_stack_tokens"] == 16384
    m = oracle.dense_ancestor_mask(po)
    scale = 1.0 / math.sqrt(w.d)
    K = bf16_ref(k[:, 0:1])
    V = bf16_ref(v[:, 0:1])
    Qs = [bf16_ref(q[:, h:h + 1]) for h in range(4)]
    Gs = [bf16_ref(do[:, h:h + 1]) for h in range(4)]
    # the same inputs as the packed path's full-size 4a check (seed 1_000_000)
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = oracle_kv_group(m, Qs, K, V, Gs, scale, "dfs 4a kv0")
    assert_attn_close(bf16_ref(o[:, 0:4]), o_ref, BF16_ATOL, BF16_RTOL, "dfs 4a O")
    assert_close(lse.numpy()[0:4], lse_ref, BF16_ATOL, BF16_RTOL, "dfs 4a LSE")
    assert_attn_close(bf16_ref(dq[:, 0:4]), dq_ref, BF16_ATOL, BF16_RTOL, "dfs 4a dQ", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(bf16_ref(dk[:, 0:1]), dk_ref, BF16_ATOL, BF16_RTOL, "dfs 4a dK", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(bf16_ref(dv[:, 0:1]), dv_ref, BF16_ATOL, BF16_RTOL, "dfs 4a dV")


@pytest.mark.timeout(600)
def test_dfs_multiturn_3_every_trie_sampled():
    torch = torch_cuda()
    w = workloads.make_workload("3")
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    rng = np.random.default_rng(3)
    scale = 1.0 / math.sqrt(w.d)
    for t, (pl, po) in enumerate(zip(tl, to)):
        q, k, v, do = workloads.attention_inputs(pl.L, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 1_000_000 + t)
        plan, o, lse, dq, dk, dv = _run(torch, pl, q, k, v, do, 2048)
        announce(f"dfs config 3[{t}]: {plan}")
        Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
        n = po.n_tokens
        rows = sorted({0, n - 1, int(po.node_end[0])} | {int(x) for x in rng.integers(0, n, 5)})
        anc = [oracle.ancestors_of(po, i) for i in rows]
        o_ref, lse_ref = oracle.attention_forward_rows(Q, K, V, rows, anc, scale, dtype=np.float32)
        dq_ref = oracle.attention_dq_rows(Q, K, V, G, rows, anc, scale, dtype=np.float32)
        assert_attn_close(bf16_ref(o[rows]), o_ref, BF16_ATOL, BF16_RTOL, f"dfs 3[{t}] O rows")
        assert_close(lse[:, rows].numpy(), lse_ref, BF16_ATOL, BF16_RTOL, f"dfs 3[{t}] LSE rows")
        assert_attn_close(bf16_ref(dq[rows]), dq_ref, BF16_ATOL, BF16_RTOL, f"dfs 3[{t}] dQ rows",
                          E2E_GRAD_VEC_FLOOR)
        cols = []
        for j in rng.permutation(n):
            dsc = oracle.descendants_of(po, int(j))
            if len(dsc) <= 48:
                cols.append((int(j), dsc))
            if len(cols) == 3:
                break
        dk_ref, dv_ref = oracle.attention_dkdv_cols(Q, K, V, G, [j for j, _ in cols], [d_ for _, d_ in cols],
                                                    lambda i: oracle.ancestors_of(po, i), scale, dtype=np.float32)
        idx = [j for j, _ in cols]
        assert_attn_close(bf16_ref(dk[idx]), dk_ref, BF16_ATOL, BF16_RTOL, f"dfs 3[{t}] dK keys", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dv[idx]), dv_ref, BF16_ATOL, BF16_RTOL, f"dfs 3[{t}] dV keys")


def test_dfs_hip_graph_capture_and_replay():
    """The depth-first execution is many small launches (frame metadata,
    forward / backward over one node's query blocks, row copies) and no
    allocation, memset, copy or synchronisation, so one trie's whole walk
    captures into a HIP graph.  Each replay, with new values in the captured
    inputs and eager work in between, equals the eager run bit for bit."""
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("multiturn-small")
    (pl,), _ = pta.pack(ids, mask, M)
    q, k, v, do = workloads.attention_inputs(pl.L, 8, 2, 128, "bf16", 1.0 / math.sqrt(128), 4321)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    meta = pta.tree_meta(pl.subtree_end)
    plan = pta.dfs_plan(pl, 256)
    announce(f"dfs graph L={pl.L}: {plan}")
    ws = torch.empty(pta.dfs_workspace_bytes(plan, 8, 2, 128), dtype=torch.uint8, device="cuda")
    outs = dict(o=torch.empty_like(qd), lse=torch.empty((8, pl.L), device="cuda"), dq=torch.empty_like(qd),
                dk=torch.empty_like(kd), dv=torch.empty_like(vd))

    def walk():
        return pta.attn_dfs(pl, qd, kd, vd, dod, meta, chunk=256, workspace=ws, **outs)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        walk()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        walk()
    gen = torch.Generator().manual_seed(7)
    for rep in range(3):
        for dst in (qd, kd, vd, dod):
            dst.copy_((torch.randn(dst.shape, generator=gen) * 0.1).to(dst.dtype))
        torch.cuda.synchronize()
        ref = tuple(x.clone() for x in walk())  # eager, on the same inputs
        for x in outs.values():
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), (outs[n] for n in ("o", "lse", "dq", "dk", "dv")),
                              ref):
            assert torch.equal(x, y), f"replay {rep}: {name}"
