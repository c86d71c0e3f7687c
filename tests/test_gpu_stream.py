"""Determinism and stream semantics of the attention entry points.

* No kernel on the path accumulates with atomics or depends on scheduling
  order, so two runs on the same inputs give bit-identical O, LSE, dQ, dK
  and dV.
* The entry points enqueue on the caller's stream: the same calls made on a
  side stream (torch.cuda.Stream, default priority) give bit-identical
  results, ordered after the producer of their inputs by the stream itself.
"""

import math

import pytest

import workloads
import prefix_tree_attention_amd as pta
from gpu_common import announce, torch_cuda

pytestmark = pytest.mark.gpu


def _inputs(torch):
    ids, mask, M = workloads.small_workload("multiturn-small")
    (pl,), _ = pta.pack(ids, mask, M)
    q, k, v, do = workloads.attention_inputs(pl.L, 8, 2, 128, "bf16", 1.0 / math.sqrt(128), 4242)
    return pl, q, k, v, do


def _run(torch, pl, q, k, v, do):
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    dq, dk, dv = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
    return o, lse, dq, dk, dv


def test_repeated_runs_are_bit_identical():
    torch = torch_cuda()
    pl, q, k, v, do = _inputs(torch)
    announce(f"determinism L={pl.L}")
    a = _run(torch, pl, q, k, v, do)
    b = _run(torch, pl, q, k, v, do)
    torch.cuda.synchronize()
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), a, b):
        assert torch.equal(x, y), name


def test_side_stream_matches_default_stream():
    torch = torch_cuda()
    pl, q, k, v, do = _inputs(torch)
    announce(f"side stream L={pl.L}")
    ref = _run(torch, pl, q, k, v, do)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = _run(torch, pl, q, k, v, do)
    s.synchronize()
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), ref, got):
        assert torch.equal(x, y), name
