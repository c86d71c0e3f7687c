"""Tree log-probabilities and entropies on the GPU (tree_logits_stats +
tree_gather_logprobs, through pack_batch's row positions and packed ids)
against the oracle's node-walk gather, on the same logits:

* elementwise on scaled-down batches (several tries, a vocabulary size that
  leaves rows unaligned to 16 bytes, bf16 and fp32 logits);
* the deep-shared 32K layout at the full vocabulary size (151936, 10 GB of
  bf16 logits) on sampled predictions, including every prefix-to-leaf
  transition, plus the sharing invariant: every leaf's predictions inside
  the shared prefix are the same packed rows, hence identical;
* -inf logits (probability 0, excluded from the entropy) and token ids
  outside the vocabulary (NaN from the kernel's own range check);
* the chunked form (tree_logits_stats per chunk of rows, then
  tree_gather_logprobs_rows over its window): bit-identical to the one-pass
  form at every chunk size, in any window order, and at full size with
  the guide's default chunk of 1024 rows.

Tolerance: the GPU accumulates each row's V terms in float32, about V/256
terms per lane then a 256-way tree, so the relative error of the sums is at
most about (V/256 + 8) 2^-24 (3.6e-5 at V = 151936) and the log-probability
and entropy errors stay well below 1e-4 + 1e-4 |value|.
"""

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import announce, assert_close, torch_cuda

pytestmark = pytest.mark.gpu

LP_ATOL, LP_RTOL = 1e-4, 1e-4


def _run_small(torch, ids, mask, M, V, dtype, seed, pad=-3.0, minus_inf_cols=0):
    se, tok, rp, lengths, _ = pta.pack_batch(ids, mask, M)
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(len(se), V, generator=g) * 2.0).to(dtype)
    if minus_inf_cols:
        x[:, V - minus_inf_cols:] = float("-inf")
    logp, ent = pta.tree_logprobs(x.cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(rp).cuda(), pad)
    torch.cuda.synchronize()
    to = oracle.pack(ids, mask, M)
    xs = x.double().numpy()
    parts, off = [], 0
    for t in to:
        parts.append(xs[off:off + t.L])
        off += t.L
    ref_lp, ref_en = oracle.gather_tree_logprobs_entropy(to, parts, *ids.shape, padding_value=pad)
    return logp.cpu().numpy(), ent.cpu().numpy(), ref_lp, ref_en


@pytest.mark.parametrize("kind,V,dt", [("grpo-small", 1000, "bf16"), ("grpo-small", 1003, "bf16"),
                                       ("nested", 517, "fp32"), ("deep-small", 4096, "bf16"),
                                       ("disjoint-small", 2051, "fp32")])
def test_small_elementwise(kind, V, dt):
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload(kind)
    ids = (np.asarray(ids) % (V - 1)).astype(np.int32)  # every label inside the vocabulary
    announce(f"logprobs {kind} V={V} {dt}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    lp, en, rlp, ren = _run_small(torch, ids, mask, M, V, dtype, seed=V)
    assert_close(lp, rlp, LP_ATOL, LP_RTOL, f"{kind} logp")
    assert_close(en, ren, LP_ATOL, LP_RTOL, f"{kind} entropy")


def test_minus_inf_logits():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("grpo-small")
    V = 640
    ids = (np.asarray(ids) % 600).astype(np.int32)  # labels below the -inf columns
    announce("logprobs -inf columns")
    lp, en, rlp, ren = _run_small(torch, ids, mask, M, V, torch.bfloat16, seed=5, minus_inf_cols=40)
    assert np.isfinite(lp[rlp != -3.0]).all() and np.isfinite(en).all()
    assert_close(lp, rlp, LP_ATOL, LP_RTOL, "logp with -inf logits")
    assert_close(en, ren, LP_ATOL, LP_RTOL, "entropy with -inf logits")


def test_token_ids_outside_vocabulary_give_nan():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("grpo-small")
    V = 300
    ids = (np.asarray(ids) % 400).astype(np.int32)  # some ids >= V
    se, tok, rp, _, _ = pta.pack_batch(ids, mask, M)
    announce("logprobs ids outside the vocabulary")
    g = torch.Generator().manual_seed(9)
    x = torch.randn(len(se), V, generator=g).to(torch.bfloat16)
    logp, _ = pta.tree_logprobs(x.cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(rp).cuda(), 0.0)
    lp = logp.cpu().numpy()
    nxt = np.where(rp[:, 1:] >= 0, rp[:, 1:], 0)
    label = tok[nxt]
    real = (rp[:, :-1] >= 0) & (rp[:, 1:] >= 0)
    bad = real & (label >= V)
    assert bad.any() and (real & ~bad).any()
    assert np.isnan(lp[:, :-1][bad]).all()
    assert np.isfinite(lp[:, :-1][real & ~bad]).all()


@pytest.mark.parametrize("kind,V,dt", [("grpo-small", 1003, "bf16"), ("nested", 517, "fp32")])
def test_chunked_equals_one_pass(kind, V, dt):
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload(kind)
    ids = (np.asarray(ids) % (V - 1)).astype(np.int32)
    se, tok, rp, _, _ = pta.pack_batch(ids, mask, M)
    L = len(se)
    announce(f"logprobs chunked {kind} L={L} V={V} {dt}")
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator().manual_seed(V + 1)
    x = (torch.randn(L, V, generator=g) * 2.0).to(dtype).cuda()
    tk, rpd = torch.from_numpy(tok).cuda(), torch.from_numpy(rp).cuda()
    lp1, en1 = pta.tree_logprobs(x, tk, rpd, -3.0)
    calls = []

    def logits_of(a, b):
        calls.append((a, b))
        return x[a:b].contiguous()

    for chunk in (1, 7, 128, 1000, L, L + 5):
        calls.clear()
        lp2, en2 = pta.tree_logprobs_chunked(logits_of, L, tk, rpd, chunk, -3.0)
        torch.cuda.synchronize()
        assert calls == [(a, min(L, a + chunk)) for a in range(0, L, chunk)]
        assert torch.equal(lp1, lp2) and torch.equal(en1, en2), f"chunk {chunk}"
    # windows in reverse order through the C entry point, onto NaN-filled outputs
    lse, ent = pta.logits_stats(x)
    B, S = rp.shape
    lp3 = torch.full((B, S), float("nan"), device="cuda")
    en3 = torch.full((B, S), float("nan"), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lib = pta.lib()
    chunk = 300
    for a in reversed(range(0, L, chunk)):
        b = min(L, a + chunk)
        xa = x[a:b].contiguous()
        rc = lib.tree_gather_logprobs_rows(xa.data_ptr(), a, b - a, L, V, 0 if dt == "bf16" else 1,
                                           lse.data_ptr(), ent.data_ptr(), tk.data_ptr(), rpd.data_ptr(), B, S,
                                           -3.0, lp3.data_ptr(), en3.data_ptr(), stream)
        assert rc == 0, lib.tree_last_error()
    torch.cuda.synchronize()
    assert torch.equal(lp1, lp3) and torch.equal(en1, en3)
    # an empty window writes exactly the pad entries
    lp4 = torch.full((B, S), float("nan"), device="cuda")
    en4 = torch.full((B, S), float("nan"), device="cuda")
    rc = lib.tree_gather_logprobs_rows(None, 0, 0, L, V, 0 if dt == "bf16" else 1, lse.data_ptr(), ent.data_ptr(),
                                       tk.data_ptr(), rpd.data_ptr(), B, S, -3.0, lp4.data_ptr(), en4.data_ptr(),
                                       stream)
    assert rc == 0, lib.tree_last_error()
    torch.cuda.synchronize()
    pads = (lp1 == -3.0)
    assert torch.equal(lp4[pads], lp1[pads]) and torch.isnan(lp4[~pads]).all()


def test_deep_shared_full_vocabulary_sampled():
    torch = torch_cuda()
    w = workloads.make_workload("4a")
    V = 151936
    se, tok, rp, lengths, _ = pta.pack_batch(w.ids, w.mask, w.max_tokens_per_mb)
    L = len(se)
    announce(f"logprobs 4a L={L} V={V} (bf16 logits, {L * V * 2 / 1e9:.1f} GB)")
    g = torch.Generator(device="cuda").manual_seed(77)
    x = torch.empty((L, V), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, L, 2048):  # bounded temporaries
        x[r0:r0 + 2048] = (torch.randn((min(2048, L - r0), V), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    logp, ent = pta.tree_logprobs(x, torch.from_numpy(tok).cuda(), torch.from_numpy(rp).cuda(), -9.0)
    torch.cuda.synchronize()
    lp, en = logp.cpu().numpy(), ent.cpu().numpy()
    n = w.mask.astype(bool).sum(1)
    prefix = 16384
    # sharing: every leaf reads the same packed rows inside the prefix
    assert (lp[:, :prefix - 1] == lp[0:1, :prefix - 1]).all() and (en[:, :prefix - 1] == en[0:1, :prefix - 1]).all()
    for r in range(w.ids.shape[0]):
        assert (lp[r, n[r] - 1:] == -9.0).all() and np.isfinite(lp[r, :n[r] - 1]).all()
    rng = np.random.default_rng(3)
    picks = [(r, prefix - 1) for r in range(0, w.ids.shape[0], 8)]  # prefix -> leaf transitions
    picks += [(int(rng.integers(w.ids.shape[0])), int(rng.integers(n[0] - 1))) for _ in range(16)]
    picks += [(r, int(n[r]) - 2) for r in (0, w.ids.shape[0] - 1)]  # last predictions
    got_lp, got_en, ref_lp, ref_en = [], [], [], []
    for r, j in picks:
        pos, label = int(rp[r, j]), int(tok[rp[r, j + 1]])
        assert label == w.ids[r][w.mask[r].astype(bool)][j + 1]
        a, b = oracle.prediction_logprob_entropy(x[pos].double().cpu().numpy(), label)
        got_lp.append(lp[r, j])
        got_en.append(en[r, j])
        ref_lp.append(a)
        ref_en.append(b)
    assert_close(np.array(got_lp), np.array(ref_lp), LP_ATOL, LP_RTOL, "4a sampled logp")
    assert_close(np.array(got_en), np.array(ref_en), LP_ATOL, LP_RTOL, "4a sampled entropy")
    # the chunked form with the guide's default chunk: bit-identical everywhere
    lp2, en2 = pta.tree_logprobs_chunked(lambda a, b: x[a:b], L, torch.from_numpy(tok).cuda(),
                                         torch.from_numpy(rp).cuda(), 1024, -9.0)
    assert torch.equal(logp, lp2) and torch.equal(ent, en2)
    del x
    torch.cuda.empty_cache()
