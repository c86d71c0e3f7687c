"""Rotary embedding fused into the attention kernels (tree_attn_fwd_rope /
tree_attn_bwd_rope) against the oracle: attention of the rotated queries and
keys -- oracle.rope by the oracle's position ids, rounded to bf16 as the
operands of a bf16 pipeline are -- and gradients with respect to the
unrotated q and k, which are the inverse rotation of the gradients with
respect to the rotated operands (oracle.rope with inverse=True).

Elementwise on every scaled-down trie at two head shapes, with NaN-filled
outputs; the rotated operands the forward leaves for the backward equal the
standalone rotation (tree_rope) bit for bit; at full size (deep-shared
32K, 32 / 8 heads) on sampled rows and keys, shared-prefix rows included.
The autograd wrapper's gradients equal the entry points'."""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, announce, assert_attn_close, assert_close, bf16_ref,
                        small_cases, torch_cuda)

pytestmark = pytest.mark.gpu

BASE = 1e6


def _round_bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _fused(torch, pl, q, k, v, do):
    meta = pta.tree_meta(pl.subtree_end)
    tab = pta.rope_table(pl.L, q.shape[2], BASE)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    nan = float("nan")
    o = torch.full_like(qd, nan)
    lse = torch.full((qd.shape[1], pl.L), nan, device="cuda")
    o, lse, q_rot, k_rot = pta.attn_fwd_rope(qd, kd, vd, meta, tab, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(t, nan) for t in (qd, kd, vd))
    pta.attn_bwd_rope(q_rot, k_rot, vd, o, lse, dod, meta, tab, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    # the rotated operands equal the standalone rotation bit for bit
    assert torch.equal(q_rot, pta.rope(qd, meta.pos, BASE)), "q_rot differs from tree_rope"
    assert torch.equal(k_rot, pta.rope(kd, meta.pos, BASE)), "k_rot differs from tree_rope"
    return meta, tuple(x.cpu() for x in (o, lse, dq, dk, dv))


@pytest.mark.parametrize("shape", [(8, 2, 128), (4, 1, 64)])
@pytest.mark.parametrize("case", list(range(6)))
def test_fused_rope_small_elementwise(case, shape):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    hq, hkv, d = shape
    tl, _ = pta.pack(ids, mask, M)
    for t, (pl, po) in enumerate(zip(tl, oracle.pack(ids, mask, M))):
        announce(f"fused rope {name}[{t}] L={pl.L} hq={hq} d={d}")
        q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, "bf16", 1.0 / math.sqrt(d), 1200 + case + t)
        meta, (o, lse, dq, dk, dv) = _fused(torch, pl, q, k, v, do)
        m = oracle.dense_ancestor_mask(po)
        pos = oracle.position_ids(m)
        assert (meta.pos.cpu().numpy() == pos).all()
        Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
        Qr, Kr = _round_bf16(oracle.rope(Q, pos, BASE)), _round_bf16(oracle.rope(K, pos, BASE))
        scale = 1.0 / math.sqrt(d)
        o_ref, lse_ref = oracle.attention_forward(Qr, Kr, V, m, scale)
        dqr, dkr, dv_ref = oracle.attention_backward(Qr, Kr, V, o_ref, lse_ref, G, m, scale)
        dq_ref = oracle.rope(dqr, pos, BASE, inverse=True)
        dk_ref = oracle.rope(dkr, pos, BASE, inverse=True)
        n = po.n_tokens
        tag = f"fused rope {name}[{t}]"
        assert_attn_close(bf16_ref(o), o_ref, BF16_ATOL, BF16_RTOL, f"{tag} O")
        assert_close(lse.numpy()[:, :n], lse_ref[:, :n], BF16_ATOL, BF16_RTOL, f"{tag} LSE")
        assert_attn_close(bf16_ref(dq), dq_ref, BF16_ATOL, BF16_RTOL, f"{tag} dQ", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dk), dk_ref, BF16_ATOL, BF16_RTOL, f"{tag} dK", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dv), dv_ref, BF16_ATOL, BF16_RTOL, f"{tag} dV")
        for x in (o, dq, dk, dv):
            assert (x[n:].float() == 0).all()


def test_fused_rope_autograd_matches_entry_points():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("deep-small")
    (pl,), _ = pta.pack(ids, mask, M)
    q, k, v, do = workloads.attention_inputs(pl.L, 8, 2, 128, "bf16", 1.0 / math.sqrt(128), 77)
    meta = pta.tree_meta(pl.subtree_end)
    tab = pta.rope_table(pl.L, 128, BASE)
    qd, kd, vd = (t.cuda().requires_grad_(True) for t in (q, k, v))
    out = pta.tree_attention_rope(qd, kd, vd, meta, tab)
    out.backward(do.cuda())
    o, lse, q_rot, k_rot = pta.attn_fwd_rope(qd.detach(), kd.detach(), vd.detach(), meta, tab)
    dq, dk, dv = pta.attn_bwd_rope(q_rot, k_rot, vd.detach(), o, lse, do.cuda(), meta, tab)
    torch.cuda.synchronize()
    assert torch.equal(out, o)
    assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)


@pytest.mark.timeout(600)
def test_fused_rope_deep_shared_4a_sampled():
    torch = torch_cuda()
    w = workloads.make_workload("4a")
    (pl,), _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    (po,) = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    announce("fused rope 4a (32 / 8 heads, D 128)")
    q, k, v, do = workloads.attention_inputs(pl.L, w.hq, w.hkv, w.d, "bf16", w.qkv_std, 1_000_000)
    meta, (o, lse, dq, dk, dv) = _fused(torch, pl, q, k, v, do)
    pos = meta.pos.cpu().numpy()
    Q, K, V, G = (bf16_ref(x).astype(np.float32) for x in (q, k, v, do))
    Qr = _round_bf16(oracle.rope(Q, pos, BASE)).astype(np.float32)
    Kr = _round_bf16(oracle.rope(K, pos, BASE)).astype(np.float32)
    scale = 1.0 / math.sqrt(w.d)
    rng = np.random.default_rng(12)
    rows = sorted({0, 16383, 16384, 16639, 32767} | {int(x) for x in rng.integers(0, 32768, 6)})
    anc = [oracle.ancestors_of(po, i) for i in rows]
    o_ref, lse_ref = oracle.attention_forward_rows(Qr, Kr, V, rows, anc, scale, dtype=np.float32)
    dqr = oracle.attention_dq_rows(Qr, Kr, V, G, rows, anc, scale, dtype=np.float32)
    dq_ref = oracle.rope(dqr, pos[rows], BASE, inverse=True)
    assert_attn_close(bf16_ref(o[rows]), o_ref, BF16_ATOL, BF16_RTOL, "fused rope 4a O rows")
    assert_close(lse[:, rows].numpy(), lse_ref, BF16_ATOL, BF16_RTOL, "fused rope 4a LSE rows")
    assert_attn_close(bf16_ref(dq[rows]), dq_ref, BF16_ATOL, BF16_RTOL, "fused rope 4a dQ rows", E2E_GRAD_VEC_FLOOR)
    cols = []
    for j in rng.permutation(32768):
        dsc = oracle.descendants_of(po, int(j))
        if len(dsc) <= 64:
            cols.append((int(j), dsc))
        if len(cols) == 4:
            break
    dkr, dv_ref = oracle.attention_dkdv_cols(Qr, Kr, V, G, [j for j, _ in cols], [x for _, x in cols],
                                             lambda i: oracle.ancestors_of(po, i), scale, dtype=np.float32)
    idx = [j for j, _ in cols]
    dk_ref = oracle.rope(dkr, pos[idx], BASE, inverse=True)
    assert_attn_close(bf16_ref(dk[idx]), dk_ref, BF16_ATOL, BF16_RTOL, "fused rope 4a dK keys", E2E_GRAD_VEC_FLOOR)
    assert_attn_close(bf16_ref(dv[idx]), dv_ref, BF16_ATOL, BF16_RTOL, "fused rope 4a dV keys")
