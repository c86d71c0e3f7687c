"""Pins of the oracle's rotary embedding by tree position ids against
things other than itself:

* a complex-number form -- each pair (x_j, x_{j+D/2}) is the complex number
  x_j + i x_{j+D/2}, multiplied by exp(i p f_j) with numpy's complex
  arithmetic;
* the relative-position property of rotary embeddings: the dot product of a
  query at position m and a key at position n depends only on m - n;
* the per-sequence invariant with tree position ids: tree attention over
  rotated Q / K (positions from the packed trie's ancestor counts) equals,
  on every sequence, causal attention of that sequence unpacked and rotated
  at positions 0 .. l - 1 (torch scaled_dot_product_attention);
* position 0 is the identity, the inverse undoes the rotation, norms are
  kept.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_complex_form():
    rng = np.random.default_rng(0)
    L, H, D, base = 37, 3, 16, 10000.0
    x = rng.normal(size=(L, H, D))
    pos = rng.integers(0, 5000, L)
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    f = base ** (-2.0 * np.arange(D // 2) / D)
    zr = z * np.exp(1j * pos[:, None, None] * f[None, None, :])
    np.testing.assert_allclose(oracle.rope(x, pos, base), np.concatenate([zr.real, zr.imag], -1), atol=1e-12)


def test_relative_position_property():
    rng = np.random.default_rng(1)
    D, base = 32, 1e6
    q, k = rng.normal(size=(1, 1, D)), rng.normal(size=(1, 1, D))
    for m, n, t in [(5, 2, 100), (7, 7, 3), (1000, 10, 12345)]:
        a = (oracle.rope(q, [m], base) * oracle.rope(k, [n], base)).sum()
        b = (oracle.rope(q, [m + t], base) * oracle.rope(k, [n + t], base)).sum()
        assert a == pytest.approx(b, abs=1e-9)


def test_identity_inverse_norm():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(20, 2, 8))
    pos = rng.integers(0, 100000, 20)
    np.testing.assert_allclose(oracle.rope(x, np.zeros(20), 1e4), x, atol=0)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, pos, 1e4), pos, 1e4, inverse=True), x, atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(x, pos, 1e4), axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_tree_positions_give_per_sequence_rope_attention(seed):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(5):
        if seqs and rng.random() < 0.7:
            base_s = seqs[int(rng.integers(len(seqs)))]
            cut = int(rng.integers(1, len(base_s) + 1))
            seqs.append(np.concatenate([base_s[:cut], rng.integers(0, 3, int(rng.integers(1, 30)))]).astype(np.int32))
        else:
            seqs.append(rng.integers(0, 3, int(rng.integers(1, 30))).astype(np.int32))
    ids, mask = workloads.pad_rows(seqs)
    (p,) = oracle.pack(ids, mask, 1024)
    m = oracle.dense_ancestor_mask(p)
    pos = oracle.position_ids(m)
    hq, hkv, d, base = 4, 2, 16, 1e4
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(p.L, hq, d, generator=g, dtype=torch.float64).numpy()
    k = torch.randn(p.L, hkv, d, generator=g, dtype=torch.float64).numpy()
    v = torch.randn(p.L, hkv, d, generator=g, dtype=torch.float64).numpy()
    scale = 1.0 / np.sqrt(d)
    o, _ = oracle.attention_forward(oracle.rope(q, pos, base), oracle.rope(k, pos, base), v, m, scale)
    for kidx in range(len(p.seq_ids)):
        idx = p.sequence_indices(kidx)
        n = len(idx)
        qs = torch.from_numpy(oracle.rope(q[idx], np.arange(n), base)).transpose(0, 1)
        ks = torch.from_numpy(oracle.rope(k[idx], np.arange(n), base)).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        vs = torch.from_numpy(v[idx]).repeat_interleave(hq // hkv, 1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=scale)
        np.testing.assert_allclose(o[idx], ref.transpose(0, 1).numpy(), atol=1e-10)


def test_matches_transformers_qwen3_rotary():
    """The convention -- half-split pairs (j, j + D/2), the frequency schedule
    base^(-2j/D), the sign of the rotation -- against the Qwen3 rotary
    embedding of the transformers library (the model family the pages train;
    built from a config, no weights), at rope_theta 1e6, head_dim 128 and
    positions up to 65535.  transformers forms its angles in float32, so the
    bound per entry is (|x_j| + |x_{j+D/2}|) (p 2^-22 + 1e-6): the angle of
    position p is off by at most a few p 2^-24 rad there, exact in the oracle."""
    qwen3 = pytest.importorskip("transformers.models.qwen3.modeling_qwen3")
    from transformers import Qwen3Config

    D, H, base = 128, 4, 1e6
    cfg = Qwen3Config(hidden_size=32 * D, num_attention_heads=32, num_key_value_heads=8, head_dim=D,
                      rope_theta=base, max_position_embeddings=65536)
    rot = qwen3.Qwen3RotaryEmbedding(config=cfg)
    rng = np.random.default_rng(21)
    pos = np.concatenate([np.arange(0, 64), rng.integers(64, 65536, 192), [65535]]).astype(np.int64)
    L = pos.size
    q = torch.from_numpy(rng.normal(size=(1, H, L, D)))
    k = torch.from_numpy(rng.normal(size=(1, 1, L, D)))
    cos, sin = rot(q, torch.from_numpy(pos)[None])
    qr, kr = qwen3.apply_rotary_pos_emb(q, k, cos, sin)
    for x, ref in ((q, qr), (k, kr)):
        xs = x[0].permute(1, 0, 2).numpy()  # [L, heads, D]
        ours = oracle.rope(xs, pos, base)
        got = ref[0].permute(1, 0, 2).numpy()
        pair = np.abs(xs[..., :D // 2]) + np.abs(xs[..., D // 2:])
        bound = np.concatenate([pair, pair], -1) * (pos[:, None, None] * 2.0 ** -22 + 1e-6)
        assert (np.abs(ours - got) <= bound).all(), float((np.abs(ours - got) / bound).max())
    # the bound is tight enough to tell the schedule apart: base 1e4 (the
    # Llama-2 default) or interleaved pairs would fail it
    assert not (np.abs(oracle.rope(xs, pos, 1e4) - got) <= bound).all()
    a = pos[:, None, None] * base ** (-2.0 * np.arange(D // 2) / D)
    yi = np.empty_like(xs)  # interleaved pairs (2j, 2j + 1)
    yi[..., 0::2] = xs[..., 0::2] * np.cos(a) - xs[..., 1::2] * np.sin(a)
    yi[..., 1::2] = xs[..., 1::2] * np.cos(a) + xs[..., 0::2] * np.sin(a)
    assert not (np.abs(yi - got) <= bound).all()
