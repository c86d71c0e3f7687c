"""Pins of the oracle attention against things other than itself:

* the per-sequence invariant -- on every root-to-leaf sequence, tree
  attention equals textbook causal attention of that sequence unpacked,
  computed here by ``torch.nn.functional.scaled_dot_product_attention``
  (is_causal=True, fp64, GQA expanded by repeat_interleave);
* the gradient invariant -- with dO = sum_s scatter(idx_s, dO_s), the tree
  gradients equal sum_s scatter(idx_s, autograd gradients of causal SDPA);
  shared-prefix gradients are therefore the sum over branches, as the DTA
  paper's problem formulation states;
* central finite differences of the oracle forward against its backward;
* pad rows and the sampled one-row / one-column forms.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads


def _tree_case(seed, hq=4, hkv=2, d=16, n_seq=5, max_len=40, vocab=3):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_seq):
        if seqs and rng.random() < 0.7:
            base = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(1, len(base) + 1))
            tail = rng.integers(0, vocab, int(rng.integers(1, max_len)))
            seqs.append(np.concatenate([base[:cut], tail]).astype(np.int32))
        else:
            seqs.append(rng.integers(0, vocab, int(rng.integers(1, max_len))).astype(np.int32))
    ids, mask = workloads.pad_rows(seqs)
    (p,) = oracle.pack(ids, mask, 1024)
    L = p.L
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(L, hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(L, hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(L, hkv, d, generator=g, dtype=torch.float64)
    return p, seqs, q, k, v


def _sdpa_causal(q, k, v, scale):
    # [n, H, D] -> SDPA's [H, n, D]; GQA: kv head h // g, expanded here
    g = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(g, dim=1)
    vv = v.repeat_interleave(g, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), kk.transpose(0, 1), vv.transpose(0, 1), is_causal=True, scale=scale)
    return o.transpose(0, 1)


@pytest.mark.parametrize("seed", range(8))
def test_forward_equals_per_sequence_causal(seed):
    p, seqs, q, k, v = _tree_case(seed)
    scale = 1.0 / np.sqrt(q.shape[-1])
    m = oracle.dense_ancestor_mask(p)
    o, lse = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, scale)
    for kidx in range(len(p.seq_ids)):
        idx = torch.as_tensor(p.sequence_indices(kidx))
        ref = _sdpa_causal(q[idx], k[idx], v[idx], scale)
        np.testing.assert_allclose(o[idx.numpy()], ref.numpy(), rtol=1e-10, atol=1e-12)
        # LSE: logsumexp of the causal score matrix of the unpacked sequence
        gq = q.shape[1] // k.shape[1]
        for h in range(q.shape[1]):
            s = scale * q[idx, h] @ k[idx, h // gq].T
            s = s.masked_fill(~torch.ones(len(idx), len(idx), dtype=torch.bool).tril(), -float("inf"))
            np.testing.assert_allclose(lse[h, idx.numpy()], torch.logsumexp(s, dim=1).numpy(),
                                       rtol=1e-12, atol=1e-12)
    pads = np.arange(p.n_tokens, p.L)
    assert (o[pads] == 0).all() and np.isneginf(lse[:, pads]).all()


@pytest.mark.parametrize("seed", range(6))
def test_backward_equals_sum_of_per_sequence_gradients(seed):
    p, seqs, q, k, v = _tree_case(seed + 100)
    scale = 1.0 / np.sqrt(q.shape[-1])
    m = oracle.dense_ancestor_mask(p)
    g = torch.Generator().manual_seed(seed)
    dq_ref, dk_ref, dv_ref = (torch.zeros_like(t) for t in (q, k, v))
    do_tree = torch.zeros_like(q)
    for kidx in range(len(p.seq_ids)):
        idx = torch.as_tensor(p.sequence_indices(kidx))
        qs, ks, vs = (t[idx].clone().requires_grad_(True) for t in (q, k, v))
        o = _sdpa_causal(qs, ks, vs, scale)
        dos = torch.randn(o.shape, generator=g, dtype=torch.float64)
        o.backward(dos)
        do_tree.index_add_(0, idx, dos)
        dq_ref.index_add_(0, idx, qs.grad)
        dk_ref.index_add_(0, idx, ks.grad)
        dv_ref.index_add_(0, idx, vs.grad)
    # pad rows of dO must not matter
    do_tree[p.n_tokens:] = torch.randn(do_tree[p.n_tokens:].shape, generator=g, dtype=torch.float64)
    # The invariant needs dO of a shared row summed over the sequences through it
    # and O of that row equal for all of them, which holds by construction.
    o, lse = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, scale)
    dq, dk, dv = oracle.attention_backward(q.numpy(), k.numpy(), v.numpy(), o, lse,
                                           do_tree.numpy(), m, scale)
    np.testing.assert_allclose(dq, dq_ref.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dk, dk_ref.numpy(), rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(dv, dv_ref.numpy(), rtol=1e-9, atol=1e-10)
    pads = np.arange(p.n_tokens, p.L)
    assert (dq[pads] == 0).all() and (dk[pads] == 0).all() and (dv[pads] == 0).all()


def test_backward_finite_differences():
    p, seqs, q, k, v = _tree_case(3, hq=2, hkv=1, d=4, n_seq=3, max_len=6)
    scale = 0.7
    m = oracle.dense_ancestor_mask(p)
    n = p.n_tokens
    rng = np.random.default_rng(0)
    do = rng.standard_normal(q.shape)
    Q, K, V = q.numpy().copy(), k.numpy().copy(), v.numpy().copy()

    def loss(Q, K, V):
        o, _ = oracle.attention_forward(Q, K, V, m, scale)
        return float((o * do).sum())

    o, lse = oracle.attention_forward(Q, K, V, m, scale)
    dq, dk, dv = oracle.attention_backward(Q, K, V, o, lse, do, m, scale)
    eps = 1e-6
    for name, X, G in (("q", Q, dq), ("k", K, dk), ("v", V, dv)):
        for _ in range(12):
            idx = (int(rng.integers(n)), int(rng.integers(X.shape[1])), int(rng.integers(X.shape[2])))
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = {"q": (Xp, K, V), "k": (Q, Xp, V), "v": (Q, K, Xp)}[name]
            args_m = {"q": (Xm, K, V), "k": (Q, Xm, V), "v": (Q, K, Xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert fd == pytest.approx(G[idx], rel=1e-6, abs=1e-8), (name, idx)


def test_single_sequence_is_causal_and_disjoint_is_varlen():
    rng = np.random.default_rng(5)
    # one sequence: the tree degenerates to causal attention
    ids, mask = workloads.pad_rows([rng.integers(0, 100, 70).astype(np.int32)])
    (p,) = oracle.pack(ids, mask, 128)
    m = oracle.dense_ancestor_mask(p)
    q, k, v = (torch.randn(p.L, 2, 8, dtype=torch.float64) for _ in range(3))
    o, _ = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, 0.3)
    ref = _sdpa_causal(q[:70], k[:70], v[:70], 0.3)
    np.testing.assert_allclose(o[:70], ref.numpy(), rtol=1e-10, atol=1e-12)
    # disjoint sequences (distinct first tokens): block-diagonal causal
    seqs = [np.concatenate([[f], rng.integers(0, 100, 30)]).astype(np.int32) for f in (101, 102, 103)]
    ids, mask = workloads.pad_rows(seqs)
    (p,) = oracle.pack(ids, mask, 128)
    m = oracle.dense_ancestor_mask(p)
    assert p.n_nodes == 3
    o, _ = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, 0.3)
    for kidx in range(3):
        idx = p.sequence_indices(kidx)
        ref = _sdpa_causal(q[idx], k[idx], v[idx], 0.3)
        np.testing.assert_allclose(o[idx], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_sampled_forms_match_dense():
    p, seqs, q, k, v = _tree_case(11, hq=4, hkv=1, d=8)
    scale = 0.35
    m = oracle.dense_ancestor_mask(p)
    Q, K, V = q.numpy(), k.numpy(), v.numpy()
    do = np.random.default_rng(1).standard_normal(Q.shape)
    o, lse = oracle.attention_forward(Q, K, V, m, scale)
    dq, dk, dv = oracle.attention_backward(Q, K, V, o, lse, do, m, scale)
    rows = list(range(p.n_tokens)) + [p.n_tokens]  # include one pad
    anc = [oracle.ancestors_of(p, i) for i in rows]
    for i, a in zip(rows, anc):
        assert a.tolist() == np.nonzero(m[i])[0].tolist()
    o_r, lse_r = oracle.attention_forward_rows(Q, K, V, rows, anc, scale)
    np.testing.assert_allclose(o_r, o[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_r, lse[:, rows], rtol=1e-12, atol=1e-13)
    dq_r = oracle.attention_dq_rows(Q, K, V, do, rows, anc, scale)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-10, atol=1e-12)
    cols = list(range(0, p.n_tokens, 3))
    desc = [oracle.descendants_of(p, j) for j in cols]
    for j, dsc in zip(cols, desc):
        assert dsc.tolist() == np.nonzero(m[:, j])[0].tolist()
    dk_c, dv_c = oracle.attention_dkdv_cols(Q, K, V, do, cols, desc,
                                            lambda i: oracle.ancestors_of(p, i), scale)
    np.testing.assert_allclose(dk_c, dk[cols], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_c, dv[cols], rtol=1e-10, atol=1e-12)


def test_fp32_mode_close_to_fp64():
    p, seqs, q, k, v = _tree_case(21, hq=2, hkv=2, d=32)
    m = oracle.dense_ancestor_mask(p)
    o64, l64 = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, 0.2)
    o32, l32 = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m, 0.2, dtype=np.float32)
    assert o32.dtype == np.float32
    np.testing.assert_allclose(o32, o64, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("seed", range(4))
def test_delta_is_the_softmax_weighted_row_of_dp(seed):
    """Delta_i = dO_i . O_i equals sum_j P_ij dP_ij with P the softmax of the
    masked scores (torch.softmax over -inf-filled scores, not the oracle's
    forward) and dP_ij = dO_i . v_j; it is what makes every dS row sum to
    zero.  Also pins the [Hq, L] layout and the zero on pads."""
    p, seqs, q, k, v = _tree_case(seed + 200)
    scale = 1.0 / np.sqrt(q.shape[-1])
    m = torch.as_tensor(oracle.dense_ancestor_mask(p))
    g = torch.Generator().manual_seed(seed)
    do = torch.randn(q.shape, generator=g, dtype=torch.float64)
    o, _ = oracle.attention_forward(q.numpy(), k.numpy(), v.numpy(), m.numpy(), scale)
    delta = oracle.attention_delta(o, do.numpy())
    assert delta.shape == (q.shape[1], p.L)
    gq = q.shape[1] // k.shape[1]
    n = p.n_tokens
    for h in range(q.shape[1]):
        s = (scale * q[:n, h] @ k[:n, h // gq].T).masked_fill(~m[:n, :n], -float("inf"))
        pr = torch.softmax(s, dim=1)
        dp = do[:n, h] @ v[:n, h // gq].T
        np.testing.assert_allclose(delta[h, :n], (pr * dp).sum(1).numpy(), rtol=1e-10, atol=1e-12)
    assert (delta[:, n:] == 0).all()
