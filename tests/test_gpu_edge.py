"""Degenerate packed layouts through tree_meta / tree_attn_fwd /
tree_attn_bwd, elementwise against the oracle (bf16 and fp32):

* a trie holding one real token (L = 128, 127 pads): O = V_0, dV_0 = dO_0,
  and dQ = dK = 0 up to rounding in the oracle (one visible key: P = 1, so
  dS = P (dP - Delta) = 0);
* three copies of one sequence (one chain, three sequence ids);
* a trie filled to the last slot (n = L = 256, no pads);
* a single 1000-token sequence (plain causal attention over 8 blocks, the
  last one ragged).
"""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import BF16_ATOL, BF16_RTOL, F32_ATOL, F32_RTOL, announce, assert_close, bf16_ref, torch_cuda

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(77)
    one = [np.array([5], np.int32)]
    seq = rng.integers(1, 1000, 300).astype(np.int32)
    copies = [seq, seq.copy(), seq.copy()]
    a = rng.integers(1, 1000, 100).astype(np.int32)
    full = [np.concatenate([a, rng.integers(1, 1000, 100)]).astype(np.int32),
            np.concatenate([a[:44], rng.integers(1000, 2000, 56)]).astype(np.int32)]  # 200 + 56 = 256
    long = [rng.integers(1, 1000, 1000).astype(np.int32)]
    return {"one-token": (one, 128), "three-copies": (copies, 384), "full-trie": (full, 256), "causal-1000": (long, 1024)}


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
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    dq, dk, dv = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
    torch.cuda.synchronize()
    m = oracle.dense_ancestor_mask(po)
    scale = 1.0 / math.sqrt(d)
    Q, K, V, G = (bf16_ref(x) for x in (q, k, v, do))
    o_ref, lse_ref = oracle.attention_forward(Q, K, V, m, scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(Q, K, V, o_ref, lse_ref, G, m, scale)
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    assert_close(bf16_ref(o.cpu()), o_ref, atol, rtol, f"{name} O")
    n = po.n_tokens
    assert_close(lse.cpu().numpy()[:, :n], lse_ref[:, :n], atol, rtol, f"{name} LSE")
    assert np.isneginf(lse.cpu().numpy()[:, n:]).all()
    assert_close(bf16_ref(dq.cpu()), dq_ref, atol, rtol, f"{name} dQ")
    assert_close(bf16_ref(dk.cpu()), dk_ref, atol, rtol, f"{name} dK")
    assert_close(bf16_ref(dv.cpu()), dv_ref, atol, rtol, f"{name} dV")
    if name == "one-token":
        g = hq // hkv
        assert np.allclose(o_ref[0], np.repeat(V[0], g, axis=0))  # O_0 = V_0 of each head's key/value head
        assert np.abs(dq_ref).max() < 1e-12 and np.abs(dk_ref).max() < 1e-12
        assert np.allclose(dv_ref[0], G[0].reshape(hkv, g, d).sum(1))  # dV_0 = sum of the group's dO_0
