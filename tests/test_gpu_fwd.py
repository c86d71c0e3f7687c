"""Forward tree attention on the GPU vs the oracle.

Elementwise on scaled-down tries (every element of O and LSE, several
tiles, ragged node boundaries, pads), in the bf16 MFMA path and the fp32
check mode; on sampled rows at the full sizes of the GRPO, multi-turn and
extreme workloads, with the launch configuration the bench times."""

import math

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import (BF16_ATOL, BF16_RTOL, F32_ATOL, F32_RTOL, announce, assert_attn_close, assert_close, bf16_ref,
                        run_attention, sample_rows, small_cases, torch_cuda)

pytestmark = pytest.mark.gpu


def _run_fwd(torch, p_lib, hq, hkv, d, dtype, std, seed, scale=None):
    q, k, v, _ = workloads.attention_inputs(p_lib.L, hq, hkv, d, dtype, std, seed, backward=False)
    meta = pta.tree_meta(p_lib.subtree_end)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = run_attention(torch, qd, kd, vd, None, meta, scale)
    torch.cuda.synchronize()
    return q, k, v, o.cpu(), lse.cpu()


def _full_check(torch, name, ids, mask, M, hq, hkv, d, dtype, seed):
    tl, _ = pta.pack(ids, mask, M)
    to = oracle.pack(ids, mask, M)
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    for t, (pl, po) in enumerate(zip(tl, to)):
        announce(f"fwd {name}[{t}] L={pl.L} {dtype} hq={hq} hkv={hkv} d={d}")
        q, k, v, o, lse = _run_fwd(torch, pl, hq, hkv, d, dtype, std, seed + t)
        m = oracle.dense_ancestor_mask(po)
        o_ref, lse_ref = oracle.attention_forward(bf16_ref(q), bf16_ref(k), bf16_ref(v), m, 1.0 / math.sqrt(d))
        atol, rtol = (F32_ATOL, F32_RTOL) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
        assert np.isfinite(o.float().numpy()).all()
        assert_attn_close(bf16_ref(o), o_ref, atol, rtol, f"{name}[{t}] O")
        assert_close(lse.numpy(), lse_ref, atol, rtol, f"{name}[{t}] LSE")
        n = po.n_tokens
        assert (o[n:].float() == 0).all() and np.isneginf(lse[:, n:].numpy()).all()


@pytest.mark.parametrize("case", list(range(6)))
@pytest.mark.parametrize("shape", [(8, 2, 128), (4, 1, 64), (2, 2, 128), (8, 1, 128)])
def test_fwd_bf16_small(case, shape):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    _full_check(torch, name, ids, mask, M, *shape, "bf16", 100 + case)


@pytest.mark.parametrize("case", list(range(6)))
@pytest.mark.parametrize("shape", [(1, 1, 64), (4, 2, 32), (2, 1, 128)])
def test_fwd_fp32_small(case, shape):
    torch = torch_cuda()
    name, ids, mask, M = list(small_cases())[case]
    _full_check(torch, name, ids, mask, M, *shape, "fp32", 200 + case)


def test_fwd_config1_fp32():
    torch = torch_cuda()
    w = workloads.make_workload("1")
    _full_check(torch, "config1", w.ids, w.mask, w.max_tokens_per_mb, w.hq, w.hkv, w.d, "fp32", 1001)


def test_fwd_config1_shapes_in_bf16():
    torch = torch_cuda()
    w = workloads.make_workload("1")
    _full_check(torch, "config1-bf16", w.ids, w.mask, w.max_tokens_per_mb, 8, 2, 128, "bf16", 1011)


def test_fwd_scale_argument():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("nested")
    (pl,), _ = pta.pack(ids, mask, M)
    (po,) = oracle.pack(ids, mask, M)
    q, k, v, o, lse = _run_fwd(torch, pl, 4, 2, 128, "bf16", 0.09, 5, scale=0.37)
    m = oracle.dense_ancestor_mask(po)
    o_ref, lse_ref = oracle.attention_forward(bf16_ref(q), bf16_ref(k), bf16_ref(v), m, 0.37)
    assert_attn_close(bf16_ref(o), o_ref, BF16_ATOL, BF16_RTOL, "scaled O")
    assert_close(lse.numpy(), lse_ref, BF16_ATOL, BF16_RTOL, "scaled LSE")


@pytest.mark.parametrize("config", ["4a", "4b", "2", "3", "L65536-b8"])
def test_fwd_full_size_sampled(config):
    # "L65536-b8": the sweep point whose first trie fills the largest budget
    # (L = 65536)
    torch = torch_cuda()
    w = workloads.sweep_workload(65536, 8) if config == "L65536-b8" else workloads.make_workload(config)
    tl, _ = pta.pack(w.ids, w.mask, w.max_tokens_per_mb)
    to = oracle.pack(w.ids, w.mask, w.max_tokens_per_mb)
    pl, po = tl[0], to[0]
    announce(f"fwd full config{config}[0] L={pl.L}")
    q, k, v, o, lse = _run_fwd(torch, pl, w.hq, w.hkv, w.d, "bf16", w.qkv_std, (1000 + 4) * 1000)
    assert np.isfinite(o.float().numpy()).all()
    rows = sample_rows(po, 24, seed=7)
    anc = [oracle.ancestors_of(po, i) for i in rows]
    o_ref, lse_ref = oracle.attention_forward_rows(bf16_ref(q), bf16_ref(k), bf16_ref(v), rows, anc,
                                                   1.0 / math.sqrt(w.d), dtype=np.float32)
    assert_attn_close(bf16_ref(o[rows]), o_ref, BF16_ATOL, BF16_RTOL, f"config{config} O rows")
    assert_close(lse[:, rows].numpy(), lse_ref, BF16_ATOL, BF16_RTOL, f"config{config} LSE rows")
    n = po.n_tokens
    assert (o[n:].float() == 0).all() and np.isneginf(lse[:, n:].numpy()).all()
