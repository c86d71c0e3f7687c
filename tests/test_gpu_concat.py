"""One launch over a whole batch: the tries of a pack laid end to end
(tree_pack_concat) and run through tree_meta / tree_attn_fwd / tree_attn_bwd
as a single packed layout, which is how bench.py times multi-trie batches.
Every trie's slice of the results must equal that trie run alone against
the oracle: elementwise on a scaled-down batch of several tries (in the
pages' first-fit-decreasing and in prefix order), and on sampled rows and
key columns of the full GRPO batch (24 tries, or 22 in prefix order)."""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, announce, assert_attn_close, assert_close, bf16_ref, run_attention,
                        sample_rows, torch_cuda)

pytestmark = pytest.mark.gpu


def _concat_run(torch, ids, mask, M, hq, hkv, d, std, seed, order="ffd"):
    se, lengths, _ = pta.pack_concat(ids, mask, M, order=order)
    parts = [workloads.attention_inputs(Lt, hq, hkv, d, "bf16", std, seed + t) for t, Lt in enumerate(lengths)]
    q, k, v, do = (torch.cat([p[j] for p in parts]) for j in range(4))
    meta = pta.tree_meta(se)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse, dq, dk, dv = run_attention(torch, qd, kd, vd, dod, meta)
    torch.cuda.synchronize()
    return (se, lengths, meta.tile_class.cpu().numpy(), meta.pos.cpu().numpy(),
            q, k, v, do, o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu())


@pytest.mark.parametrize("order", ["ffd", "prefix"])
def test_concat_small_elementwise(order):
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("grpo-small")
    to = oracle.pack(ids, mask, M, order=order)
    hq, hkv, d = 8, 2, 128
    announce(f"concat grpo-small ({order} order): {len(to)} tries, L={[t.L for t in to]}")
    se, lengths, tc, pos, q, k, v, do, o, lse, dq, dk, dv = _concat_run(torch, ids, mask, M, hq, hkv, d,
                                                                         1.0 / math.sqrt(d), 500, order)
    assert lengths == [t.L for t in to] and len(to) > 1
    scale = 1.0 / math.sqrt(d)
    off = 0
    for t, po in enumerate(to):
        sl = slice(off, off + po.L)
        b0, b1 = off // 128, (off + po.L) // 128
        m = oracle.dense_ancestor_mask(po)
        assert (pos[sl] == oracle.position_ids(m)).all(), f"trie {t} position ids"
        assert (tc[b0:b1, b0:b1] == oracle.tile_classes(m)).all(), f"trie {t} tile classes"
        assert not tc[b0:b1, :b0].any() and not tc[b0:b1, b1:].any(), f"trie {t} cross-trie tiles"
        Q, K, V, G = (bf16_ref(x[sl]) for x in (q, k, v, do))
        o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
        dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
        assert_attn_close(bf16_ref(o[sl]), o_ref, BF16_ATOL, BF16_RTOL, f"trie {t} O")
        assert_close(lse[:, sl].numpy(), lse_ref, BF16_ATOL, BF16_RTOL, f"trie {t} LSE")
        assert_attn_close(bf16_ref(dq[sl]), dq_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dQ", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dk[sl]), dk_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dK", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dv[sl]), dv_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dV")
        off += po.L


@pytest.mark.parametrize("order", ["ffd", "prefix"])
def test_concat_grpo_full_size_sampled(order):
    torch = torch_cuda()
    w = workloads.make_workload("2")
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb, order=order)
    announce(f"concat config2 ({order} order): {len(to)} tries, L={sum(t.L for t in to)}")
    se, lengths, tc, pos, q, k, v, do, o, lse, dq, dk, dv = _concat_run(torch, w.ids, w.mask, w.max_tokens_per_mb,
                                                                         w.hq, w.hkv, w.d, w.qkv_std, 9000, order)
    for nm, x in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.isfinite(x.float().numpy()).all(), nm
    scale = 1.0 / math.sqrt(w.d)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    rng = np.random.default_rng(5)
    for t in sorted({0, len(to) // 2, len(to) - 1}):
        po = to[t]
        sl = slice(int(offs[t]), int(offs[t + 1]))
        Q, K, V, G = (bf16_ref(x[sl]) for x in (q, k, v, do))
        rows = sample_rows(po, 8, seed=20 + t)
        anc = [oracle.ancestors_of(po, i) for i in rows]
        o_ref, lse_ref = oracle.attention_forward_rows(Q, K, V, rows, anc, scale, dtype=np.float32)
        g_rows = [int(offs[t]) + i for i in rows]
        assert_attn_close(bf16_ref(o[g_rows]), o_ref, BF16_ATOL, BF16_RTOL, f"trie {t} O rows")
        assert_close(lse[:, g_rows].numpy(), lse_ref, BF16_ATOL, BF16_RTOL, f"trie {t} LSE rows")
        dq_ref = oracle.attention_dq_rows(Q, K, V, G, rows, anc, scale, dtype=np.float32)
        assert_attn_close(bf16_ref(dq[g_rows]), dq_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dQ rows", E2E_GRAD_VEC_FLOOR)
        keys = []
        for j in rng.permutation(po.n_tokens):
            dsc = oracle.descendants_of(po, int(j))
            if len(dsc) <= 24:
                keys.append((int(j), dsc))
            if len(keys) == 4:
                break
        cols = [j for j, _ in keys]
        dk_ref, dv_ref = oracle.attention_dkdv_cols(Q, K, V, G, cols, [dsc for _, dsc in keys],
                                                    lambda i: oracle.ancestors_of(po, i), scale, dtype=np.float32)
        g_cols = [int(offs[t]) + j for j in cols]
        assert_attn_close(bf16_ref(dk[g_cols]), dk_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dK cols", E2E_GRAD_VEC_FLOOR)
        assert_attn_close(bf16_ref(dv[g_cols]), dv_ref, BF16_ATOL, BF16_RTOL, f"trie {t} dV cols")
        n = po.n_tokens
        pads = slice(int(offs[t]) + n, int(offs[t + 1]))
        assert (o[pads].float() == 0).all() and (dq[pads].float() == 0).all()
        assert (dk[pads].float() == 0).all() and (dv[pads].float() == 0).all()
