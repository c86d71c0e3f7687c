"""Backward tree attention on the GPU vs the oracle.

Elementwise dQ / dK / dV on scaled-down tries (bf16 MFMA path and fp32
check mode).  At full size: sampled dQ rows, sampled dK / dV keys whose
descendant sets are small enough for the one-column oracle, and two exact
identities over all keys -- sum_j dK_j = 0 (each softmax-gradient row sums
to zero) and sum_j dV_j = sum_i dO_i over real rows (each P row sums to
one), per key/value head with its query heads summed."""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, F32_ATOL, F32_RTOL, announce, assert_attn_close,
                        bf16_ref, grad_floor, run_attention, sample_rows, small_cases, torch_cuda)

pytestmark = pytest.mark.gpu


def _run(torch, p_lib, hq, hkv, d, dtype, std, seed):
    q, k, v, do = workloads.attention_inputs(p_lib.L, hq, hkv, d, dtype, std, seed)
    meta = pta.tree_meta(p_lib.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse, dq, dk, dv = run_attention(torch, qd, kd, vd, dod, meta)
    torch.cuda.synchronize()
    return q, k, v, do, o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def _full_check(torch, name, ids, mask, M, hq, hkv, d, dtype, seed):
    tl, _ = pta.pack(ids, mask, M)
    to = oracle.pack(ids, mask, M)
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    for t, (pl, po) in enumerate(zip(tl, to)):
        announce(f"bwd {name}[{t}] L={pl.L} {dtype} hq={hq} hkv={hkv} d={d}")
        q, k, v, do, o, lse, dq, dk, dv = _run(torch, pl, hq, hkv, d, dtype, std, seed + t)
        m = oracle.dense_ancestor_mask(po)
        Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
        o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, 1.0 / math.sqrt(d))
        dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, 1.0 / math.sqrt(d))
        for nm, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
            assert np.isfinite(x.float().numpy()).all(), nm
        assert_attn_close(bf16_ref(dq), dq_ref, atol, rtol, f"{name}[{t}] dQ", grad_floor(dtype))
        assert_attn_close(bf16_ref(dk), dk_ref, atol, rtol, f"{name}[{t}] dK", grad_floor(dtype))
        assert_attn_close(bf16_ref(dv), dv_ref, atol, rtol, f"{name}[{t}] dV")
        n = po.n_tokens
        assert (dq[n:].float() == 0).all() and (dk[n:].float() == 0).all() and (dv[n:].float() == 0).all()
        if dtype == "bf16":
            _isolated_check(torch, pl, po, q, k, v, do, o_ref, lse_ref, m, d, f"{name}[{t}]")


def _isolated_check(torch, pl, po, q, k, v, do, o_ref, lse_ref, m, d, tag):
    """The backward alone: the kernels are given the oracle's O (rounded to
    bf16) and LSE (float32) instead of the GPU forward's, and the oracle's
    backward runs on exactly those values, so the only differences left are
    the kernels' own roundings and the tight per-vector floor applies."""
    scale = 1.0 / math.sqrt(d)
    o_in = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse_in = torch.from_numpy(lse_ref).float()
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, bf16_ref(o_in), lse_in.double().numpy(), G, m, scale)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod, od, lsed = (t.cuda().contiguous() for t in (q, k, v, do, o_in, lse_in))
    ws = torch.full((pta.bwd_workspace_bytes(pl.L, q.shape[1], d),), 255, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    pta.attn_bwd(qd, kd, vd, od, lsed, dod, meta, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for nm, x, r in (("dQ", dq, dq_ref), ("dK", dk, dk_ref), ("dV", dv, dv_ref)):
        assert_attn_close(bf16_ref(x.cpu()), r, BF16_ATOL, BF16_RTOL, f"{tag} {nm} (backward alone)")


@pytest.mark.parametrize("case", list(range(6)))
@pytest.mark.parametrize("shape", [(8, 2, 128), (4, 1, 64), (2, 2, 128), (8, 1, 128)])
def test_bwd_bf16_small(case, shape):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    _full_check(torch, name, ids, mask, M, *shape, "bf16", 300 + case)


@pytest.mark.parametrize("case", list(range(6)))
@pytest.mark.parametrize("shape", [(1, 1, 64), (4, 2, 32), (2, 1, 128)])
def test_bwd_fp32_small(case, shape):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    _full_check(torch, name, ids, mask, M, *shape, "fp32", 400 + case)


def test_bwd_deep_shared_medium():
    # a scaled deep-shared trie: 1024-token prefix, 12 leaves of 100 tokens
    torch = torch_cuda()
    rng = np.random.default_rng(77)
    prefix = rng.integers(0, 1000, 1024).astype(np.int32)
    seqs = [np.concatenate([prefix, np.concatenate([[2000 + i], rng.integers(0, 1000, 99)]).astype(np.int32)])
            for i in range(12)]
    ids, mask = workloads.pad_rows(seqs)
    _full_check(torch, "deep-medium", ids, mask, 4096, 8, 2, 128, "bf16", 500)


def _pick_keys(po, rng, n_keys, max_desc):
    """Keys whose descendant sets have at most max_desc rows."""
    keys = []
    cand = rng.permutation(po.n_tokens)
    for j in cand:
        dsc = oracle.descendants_of(po, int(j))
        if len(dsc) <= max_desc:
            keys.append((int(j), dsc))
        if len(keys) == n_keys:
            break
    return keys


@pytest.mark.parametrize("config", ["4a", "4b", "2", "3", "L65536-b8"])
def test_bwd_full_size_sampled(config):
    # "L65536-b8": the sweep point whose first trie fills the largest budget
    # (L = 65536)
    torch = torch_cuda()
    w = workloads.sweep_workload(65536, 8) if config == "L65536-b8" else workloads.make_workload(config)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    pl, po = tl[0], to[0]
    announce(f"bwd full config{config}[0] L={pl.L}")
    q, k, v, do, o, lse, dq, dk, dv = _run(torch, pl, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 7000 + len(config))
    for nm, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.isfinite(x.float().numpy()).all(), nm
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(w.d)
    rows = sample_rows(po, 12, seed=11)
    anc = [oracle.ancestors_of(po, i) for i in rows]
    dq_ref = oracle.attention_dq_rows(Q, K, V, G, rows, anc, scale, dtype=np.float32)
    assert_attn_close(bf16_ref(dq[rows]), dq_ref, BF16_ATOL, BF16_RTOL, f"config{config} dQ rows", E2E_GRAD_VEC_FLOOR)
    rng = np.random.default_rng(3)
    picked = _pick_keys(po, rng, 6, 24)
    cols = [j for j, _ in picked]
    desc = [dsc for _, dsc in picked]
    dk_ref, dv_ref = oracle.attention_dkdv_cols(Q, K, V, G, cols, desc, lambda i: oracle.ancestors_of(po, i),
                                                scale, dtype=np.float32)
    assert_attn_close(bf16_ref(dk[cols]), dk_ref, BF16_ATOL, BF16_RTOL, f"config{config} dK cols", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(bf16_ref(dv[cols]), dv_ref, BF16_ATOL, BF16_RTOL, f"config{config} dV cols")
    # identities over every key, per key/value head: a consistency check of
    # the whole backward (its bound uses the GPU's own magnitudes; the
    # elementwise checks above and tests/test_gpu_fullsize.py, which bounds
    # the same identities by the oracle's magnitudes, are what bind)
    n = po.n_tokens
    grp = w.hq // w.hkv
    dk_sum = bf16_ref(dk[:n]).sum(axis=0)
    dv_sum = bf16_ref(dv[:n]).sum(axis=0)
    do_sum = G[:n].reshape(n, w.hkv, grp, w.d).sum(axis=(0, 2))
    scale_dk = np.abs(bf16_ref(dk[:n])).sum(axis=0).max()
    scale_dv = np.abs(bf16_ref(dv[:n])).sum(axis=0).max()
    print(f"  sum dK max {np.abs(dk_sum).max():.3e} (abs-sum {scale_dk:.3e}); "
          f"sum dV - sum dO max {np.abs(dv_sum - do_sum).max():.3e} (abs-sum {scale_dv:.3e})", flush=True)
    assert np.abs(dk_sum).max() <= 1e-2 * scale_dk
    assert np.abs(dv_sum - do_sum).max() <= 1e-2 * scale_dv
    assert (dq[n:].float() == 0).all() and (dk[n:].float() == 0).all() and (dv[n:].float() == 0).all()


def test_autograd_function_matches_entry_points():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("deep-small")
    (pl,), _ = pta.pack(ids, mask, M)
    q, k, v, do = workloads.attention_inputs(pl.L, 4, 2, 128, "bf16", 0.09, 9)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    o = pta.tree_attention(qd, kd, vd, meta)
    o.backward(do.cuda())
    o2, lse2 = pta.attn_fwd(qd.detach(), kd.detach(), vd.detach(), meta)
    dq, dk, dv = pta.attn_bwd(qd.detach(), kd.detach(), vd.detach(), o2, lse2, do.cuda(), meta)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_bwd_scale_argument(dtype, d):
    """A softmax scale other than 1/sqrt(D) reaches every place it enters:
    the -LSE / scale initial value of S, the exp2 argument and dK."""
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("nested")
    (pl,), _ = pta.pack(ids, mask, M)
    (po,) = oracle.pack(ids, mask, M)
    scale = 0.37
    announce(f"bwd scale {scale} {dtype} d={d}")
    q, k, v, do = workloads.attention_inputs(pl.L, 4, 2, d, dtype, 0.09 if dtype == "bf16" else 0.5, 17)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse, dq, dk, dv = run_attention(torch, qd, kd, vd, dod, meta, scale)
    torch.cuda.synchronize()
    m = oracle.dense_ancestor_mask(po)
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    assert_attn_close(bf16_ref(dq.cpu()), dq_ref, atol, rtol, "scaled dQ", grad_floor(dtype))
    assert_attn_close(bf16_ref(dk.cpu()), dk_ref, atol, rtol, "scaled dK", grad_floor(dtype))
    assert_attn_close(bf16_ref(dv.cpu()), dv_ref, atol, rtol, "scaled dV")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("phase", ["DELTA", "DQ_DELTA"])
@pytest.mark.parametrize("case", [1, 3, 5])
def test_delta_against_oracle(case, phase, dtype):
    """The backward's preprocessing term Delta_i = dO_i . O_i, read back from
    the workspace (bf16: -Delta in the first [Hq, L] floats and -LSE / scale
    in the next; fp32: Delta), against the oracle's Delta.  The kernel is
    given the oracle's own O (rounded to the tensor dtype) and LSE, so the
    expected values are the oracle's on exactly the inputs the kernel reads.
    Both the separate Delta pass and the dQ kernel that forms Delta itself
    (the whole backward's path) are checked.  Bound: a float32 dot product
    of D terms, |err| <= 1e-5 sum_d |dO_d O_d| + 1e-30."""
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    pl = pta.pack(ids, mask, M)[0][0]
    po = oracle.pack(ids, mask, M)[0]
    hq, hkv, d = (8, 2, 128) if dtype == "bf16" else (4, 2, 64)
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    announce(f"delta {name}[0] {phase} {dtype} L={pl.L}")
    q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, dtype, std, 600 + case)
    scale = 1.0 / math.sqrt(d)
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    m = oracle.dense_ancestor_mask(po)
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o_in = torch.from_numpy(o_ref).to(tdt)
    lse_in = torch.from_numpy(lse_ref).float()
    delta_ref = oracle.attention_delta(bf16_ref(o_in), G)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod, od, lsed = (t.cuda().contiguous() for t in (q, k, v, do, o_in, lse_in))
    code = pta.DTYPE_BF16 if dtype == "bf16" else pta.DTYPE_FP32
    ws = torch.full((pta.bwd_workspace_bytes(pl.L, hq, d, code),), 255, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    pta.attn_bwd_phase(getattr(pta, f"BWD_{phase}"), qd, kd, vd, od, lsed, dod, dq, dk, dv, meta, ws)
    torch.cuda.synchronize()
    n_rows = pl.L * hq
    w = ws[: 4 * 2 * n_rows].view(torch.float32).cpu().numpy().astype(np.float64)
    got = -w[:n_rows].reshape(hq, pl.L) if dtype == "bf16" else w[:n_rows].reshape(hq, pl.L)
    mag = (np.abs(bf16_ref(o_in)) * np.abs(G)).sum(axis=2).T
    err = np.abs(got - delta_ref)
    print(f"  Delta: max err / bound {float((err / (1e-5 * mag + 1e-30)).max()):.3e}", flush=True)
    assert (err <= 1e-5 * mag + 1e-30).all(), f"Delta off at {np.argwhere(err > 1e-5 * mag + 1e-30)[:5]}"
    n = po.n_tokens
    assert (got[:, n:] == 0).all()
    if dtype == "bf16":
        nls = w[n_rows:].reshape(hq, pl.L)
        ref_nls = -lse_ref / scale
        assert np.isposinf(nls[:, n:]).all()
        assert np.allclose(nls[:, :n], ref_nls[:, :n], rtol=2e-7, atol=0), "-LSE / scale"
