"""Degenerate packed layouts through tree_meta / tree_attn_fwd /
tree_attn_bwd, elementwise against the oracle (bf16 and fp32):

* a trie holding one real token (L = 128, 127 pads): O = V_0, dV_0 = dO_0,
  and dQ = dK = 0 up to rounding in the oracle (one visible key: P = 1, so
  dS = P (dP - Delta) = 0);
* three copies of one sequence (one chain, three sequence ids);
* a trie filled to the last slot (n = L = 256, no pads);
* a single 1000-token sequence (plain causal attention over 8 blocks, the
  last one ragged);
* scores that grow along each row, so the forward's running max, and with
  it the reference of O and the row sum, moves every step or two.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from checks import assert_within_bound, conditioned_grad_bounds
from gpu_common import (BF16_ATOL, BF16_RTOL, F32_ATOL, F32_RTOL, announce, assert_attn_close, assert_close, bf16_ref,
                        grad_floor, run_attention, torch_cuda)

pytestmark = pytest.mark.gpu


def _cases():
    return workloads.edge_layouts()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name", ["one-token", "three-copies", "full-trie", "causal-1000"])
def test_degenerate_layouts(name, dtype):
    torch = torch_cuda()
    seqs, M = _cases()[name]
    ids, mask = workloads.pad_rows(seqs)
    (pl,), _ = pta.pack(ids, mask, M)
    (po,) = oracle.pack(ids, mask, M)
    if name == "full-trie":
        assert po.n_tokens == po.L == 256
    if name == "three-copies":
        assert po.n_tokens == 300 and len(po.seq_ids) == 3
    hq, hkv, d = (4, 2, 64) if dtype == "fp32" else (8, 2, 128)
    announce(f"edge {name} {dtype} L={pl.L} n={po.n_tokens}")
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, dtype, std, 31)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse, dq, dk, dv = run_attention(torch, qd, kd, vd, dod, meta)
    torch.cuda.synchronize()
    m = oracle.dense_ancestor_mask(po)
    scale = 1.0 / math.sqrt(d)
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    assert_attn_close(bf16_ref(o.cpu()), o_ref, atol, rtol, f"{name} O")
    n = po.n_tokens
    assert_close(lse.cpu().numpy()[:, :n], lse_ref[:, :n], atol, rtol, f"{name} LSE")
    assert np.isneginf(lse.cpu().numpy()[:, n:]).all()
    if name == "one-token":
        # one visible key: P = 1, so dS = P (dP - Delta) = 0 and dQ = dK = 0
        # exactly; the kernels leave only the rounding of dP - Delta (O is V_0
        # rounded), far below any input's scale.  Nothing to normalise by.
        assert np.abs(dq_ref).max() < 1e-12 and np.abs(dk_ref).max() < 1e-12
        assert float(dq.abs().max()) < 1e-6 and float(dk.abs().max()) < 1e-6
    else:
        assert_attn_close(bf16_ref(dq.cpu()), dq_ref, atol, rtol, f"{name} dQ", grad_floor(dtype))
        assert_attn_close(bf16_ref(dk.cpu()), dk_ref, atol, rtol, f"{name} dK", grad_floor(dtype))
    assert_attn_close(bf16_ref(dv.cpu()), dv_ref, atol, rtol, f"{name} dV")
    if name == "one-token":
        g = hq // hkv
        assert np.allclose(o_ref[0], np.repeat(V[0], g, axis=0))  # O_0 = V_0 of each head's key/value head
        assert np.abs(dq_ref).max() < 1e-12 and np.abs(dk_ref).max() < 1e-12
        assert np.allclose(dv_ref[0], G[0].reshape(hkv, g, d).sum(1))  # dV_0 = sum of the group's dO_0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("name", ["causal-1000", "full-trie"])
def test_forward_reference_moves_within_a_row(name, dtype):
    """Scores that grow along the key axis, so the online softmax's running
    max rises by 4 (1000-token sequence) to 16 (256-token trie) log2 units
    per 64-key step, and the forward carries O and the row sum over to a new
    reference every first or second step (it moves only past 8 log2 units);
    with N(0, 1/D) inputs the max settles after the first step and that path
    would go unexercised.  q = a u + noise, k_j = c_j u + noise with a fixed
    unit vector u and c_j rising linearly to c_max, so S_ij ~ a c_j / sqrt(D)
    reaches about 45 at the end of the row.  bf16 checks the forward; the
    fp32 check mode checks the gradients as well."""
    torch = torch_cuda()
    seqs, M = _cases()[name]
    ids, mask = workloads.pad_rows(seqs)
    (pl,), _ = pta.pack(ids, mask, M)
    (po,) = oracle.pack(ids, mask, M)
    hq, hkv, d = (4, 2, 64) if dtype == "fp32" else (8, 2, 128)
    L = pl.L
    announce(f"reference moves {name} {dtype} L={L}")
    q, k, v, do = workloads.score_ramp_inputs(L, hq, hkv, d, dtype)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    torch.cuda.synchronize()
    m = oracle.dense_ancestor_mask(po)
    scale = 1.0 / math.sqrt(d)
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
    n = po.n_tokens
    # the scores really do span many rescale thresholds along each row
    assert lse_ref[:, n - 1].min() > 30.0 and lse_ref[:, 0].max() < 10.0
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    assert_attn_close(bf16_ref(o.cpu()), o_ref, atol, rtol, f"{name} O")
    assert_close(lse.cpu().numpy()[:, :n], lse_ref[:, :n], atol, rtol, f"{name} LSE")
    dq, dk, dv = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
    if dtype == "bf16":
        # The backward reads LSE and never rescales.  At these score
        # magnitudes every key shares a large component along u, so
        # dQ = scale sum_j dS_ij k_j is a small difference of large terms
        # (sum_j dS_ij = 0) and the bf16 rounding of dS shows through in
        # proportion to that conditioning, not to |dQ|.  The bound per entry
        # follows the kernel's roundings (checks.conditioned_grad_bounds).
        bq, bk, bv = conditioned_grad_bounds(Q, K, V, G, o_ref, lse_ref, m, scale)
        assert_within_bound(bf16_ref(dq.cpu()), dq_ref, bq, 3.0, f"{name} dQ")
        assert_within_bound(bf16_ref(dk.cpu()), dk_ref, bk, 3.0, f"{name} dK")
        assert_within_bound(bf16_ref(dv.cpu()), dv_ref, bv, 3.0, f"{name} dV")
        return
    assert_attn_close(bf16_ref(dq.cpu()), dq_ref, atol, rtol, f"{name} dQ")
    assert_attn_close(bf16_ref(dk.cpu()), dk_ref, atol, rtol, f"{name} dK")
    assert_attn_close(bf16_ref(dv.cpu()), dv_ref, atol, rtol, f"{name} dV")
