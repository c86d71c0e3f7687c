"""The GPU parity checker must reject plausible wrong outputs (CPU only).

At exactly the inputs the GPU attention tests and the smoke use (the same
scaled-down tries, head shapes, input scales and seeds), the oracle's outputs
are corrupted in ways a broken kernel could produce -- all zero, halved, the
heads or tokens swapped, one token's vector zeroed -- and the oracle is
re-run with mistakes planted in it: the diagonal of the mask dropped (no
token sees itself), each token's root ancestor dropped, Delta taken as 0.
``checks.assert_attn_close`` must raise on every one of them for every
output it changes, while the correct outputs rounded to the kernel dtype
(what a perfect kernel would return) pass.  Without this a check can be
vacuous: at N(0, 1)/sqrt(128) inputs most entries of dQ and dK are ~3e-4,
far below the 2e-2 absolute bound."""

import math

import numpy as np
import pytest

import oracle
import workloads
from checks import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, F32_ATOL, F32_RTOL, assert_attn_close, assert_within_bound, attn_errors,
                    conditioned_grad_bounds)

BF16_SHAPES = [(8, 2, 128), (4, 1, 64), (2, 2, 128), (8, 1, 128)]
F32_SHAPES = [(1, 1, 64), (4, 2, 32), (2, 1, 128)]


def _small_cases():
    ids, mask = workloads.worked_example()
    yield "worked-example", ids, mask, 128
    for k in workloads.SMALL_KINDS:
        ids, mask, M = workloads.small_workload(k)
        yield k, ids, mask, M


def _round(x, dtype):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdt).double().numpy()


def _inputs(L, hq, hkv, d, dtype, std, seed):
    q, k, v, do = workloads.attention_inputs(L, hq, hkv, d, dtype, std, seed)
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    return f(q), f(k), f(v), f(do)


def _outputs(Q, K, V, G, m, scale, o_for_delta=None):
    o, lse = oracle.attention_forward(Q, K, V, m, scale)
    dq, dk, dv = oracle.attention_backward(Q, K, V, o if o_for_delta is None else o_for_delta, lse, G, m, scale)
    return {"O": o, "dQ": dq, "dK": dk, "dV": dv}


def _median_row(x, n):
    norms = np.linalg.norm(x[:n].reshape(n, -1), axis=1)
    return int(np.argsort(norms)[n // 2])


def _corruptions(ref, n):
    out = {"zero": np.zeros_like(ref), "half": 0.5 * ref}
    if ref.shape[1] > 1:
        out["heads-rolled"] = np.roll(ref, 1, axis=1)
    elif n > 1:
        r = ref.copy()
        r[:n] = np.roll(ref[:n], 1, axis=0)
        out["tokens-rolled"] = r
    r = ref.copy()
    r[_median_row(ref, n)] = 0.0
    out["one-vector-zeroed"] = r
    return out


def _planted(po, Q, K, V, G, scale):
    """Outputs of the oracle with a mistake planted in it."""
    m = oracle.dense_ancestor_mask(po)
    n = po.n_tokens
    no_self = m.copy()
    no_self[np.arange(n), np.arange(n)] = False
    no_root = m.copy()
    for i in range(n):
        a = np.nonzero(m[i])[0]
        if len(a) > 1:
            no_root[i, a[0]] = False
    out = {"mask-without-self": _outputs(Q, K, V, G, no_self, scale),
           "mask-without-root": _outputs(Q, K, V, G, no_root, scale)}
    zero_o = np.zeros((Q.shape[0], Q.shape[1], Q.shape[2]))
    d0 = _outputs(Q, K, V, G, m, scale, o_for_delta=zero_o)
    out["delta-zero"] = {"dQ": d0["dQ"], "dK": d0["dK"]}
    return out


def _must_fail(got, ref, atol, rtol, what, vec_floor=None):
    fails, _ = attn_errors(got, ref, atol, rtol, vec_floor)
    assert fails, f"checker accepted {what} (per-vector floor {vec_floor})"


def _self_test(po, hq, hkv, d, dtype, seed, planted=True):
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    scale = 1.0 / math.sqrt(d)
    Q, K, V, G = _inputs(po.L, hq, hkv, d, dtype, std, seed)
    m = oracle.dense_ancestor_mask(po)
    ref = _outputs(Q, K, V, G, m, scale)
    n = po.n_tokens
    # dQ / dK of a backward fed the forward's bf16 O are checked with the
    # wider per-vector floor; every corruption must fail that form too
    floors = {nm: [None] + ([E2E_GRAD_VEC_FLOOR] if dtype == "bf16" and nm in ("dQ", "dK") else [])
              for nm in ref}
    for name, r in ref.items():
        assert_attn_close(_round(r, dtype), r, atol, rtol, f"rounded oracle {name}")
        for what, bad in _corruptions(r, n).items():
            if name in ("dQ", "dK") and n == 1:
                continue  # one visible key: dQ = dK = 0 exactly, nothing to corrupt
            for f in floors[name]:
                _must_fail(bad, r, atol, rtol, f"{what} {name}", f)
    if dtype == "bf16":
        # what a perfect kernel fed its own bf16 O would return: Delta from
        # the rounded O, outputs rounded; must pass with the wider floor
        o_b = _round(ref["O"], dtype)
        lse = oracle.attention_forward(Q, K, V, m, scale)[1]
        e2e = oracle.attention_backward(Q, K, V, o_b, lse, G, m, scale)
        for name, x in zip(("dQ", "dK"), e2e[:2]):
            assert_attn_close(_round(x, dtype), ref[name], atol, rtol, f"bf16-O oracle {name}", E2E_GRAD_VEC_FLOOR)
    if planted:
        for what, outs in _planted(po, Q, K, V, G, scale).items():
            for name, bad in outs.items():
                if np.array_equal(bad, ref[name]):
                    continue  # the mistake changes nothing here (e.g. no token has an ancestor)
                for f in floors[name]:
                    _must_fail(bad, ref[name], atol, rtol, f"{what} {name}", f)


@pytest.mark.parametrize("shape", BF16_SHAPES)
def test_checker_rejects_wrong_bf16_outputs(shape):
    # the GPU backward tests' inputs: trie t of case c drawn with seed 300 + c + t
    for c, (name, ids, mask, M) in enumerate(_small_cases()):
        for t, po in enumerate(oracle.pack(ids, mask, M)):
            _self_test(po, *shape, "bf16", 300 + c + t, planted=(shape == BF16_SHAPES[0]))


@pytest.mark.parametrize("shape", F32_SHAPES)
def test_checker_rejects_wrong_fp32_outputs(shape):
    for c, (name, ids, mask, M) in enumerate(_small_cases()):
        for t, po in enumerate(oracle.pack(ids, mask, M)):
            _self_test(po, *shape, "fp32", 400 + c + t, planted=(shape == F32_SHAPES[0]))


def test_checker_rejects_wrong_smoke_outputs():
    # __graft_entry__.smoke(): deep-small, 8 query / 2 key-value heads, D = 128, seed 123
    ids, mask, M = workloads.small_workload("deep-small")
    (po,) = oracle.pack(ids, mask, M)
    _self_test(po, 8, 2, 128, "bf16", 123)


@pytest.mark.parametrize("kind", ["one-token", "three-copies", "full-trie", "causal-1000"])
def test_checker_on_degenerate_layouts(kind):
    # inputs of the GPU degenerate-layout tests: 8 query / 2 key-value heads, D = 128, seed 31
    seqs, M = workloads.edge_layouts()[kind]
    ids, mask = workloads.pad_rows(seqs)
    (po,) = oracle.pack(ids, mask, M)
    _self_test(po, 8, 2, 128, "bf16", 31)


@pytest.mark.parametrize("kind", ["causal-1000", "full-trie"])
def test_conditioned_bound_on_score_ramp(kind):
    # inputs of the GPU score-ramp test in bf16: 8 query / 2 key-value heads, D = 128
    seqs, M = workloads.edge_layouts()[kind]
    ids, mask = workloads.pad_rows(seqs)
    (po,) = oracle.pack(ids, mask, M)
    q, k, v, do = workloads.score_ramp_inputs(po.L, 8, 2, 128, "bf16")
    Q, K, V, G = (t.double().numpy() for t in (q, k, v, do))
    m = oracle.dense_ancestor_mask(po)
    scale = 1.0 / math.sqrt(128)
    o, lse = oracle.attention_forward(Q, K, V, m, scale)
    grads = oracle.attention_backward(Q, K, V, o, lse, G, m, scale)
    bounds = conditioned_grad_bounds(Q, K, V, G, o, lse, m, scale)
    for name, r, b in zip(("dQ", "dK", "dV"), grads, bounds):
        assert_within_bound(_round(r, "bf16"), r, b, 3.0, f"rounded oracle {name}")
        for what, bad in _corruptions(r, po.n_tokens).items():
            with pytest.raises(AssertionError):
                assert_within_bound(bad, r, b, 3.0, f"{what} {name}")
