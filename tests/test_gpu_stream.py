"""Determinism and stream semantics of the attention entry points.

* No kernel on the path accumulates with atomics or depends on scheduling
  order, so two runs on the same inputs give bit-identical O, LSE, dQ, dK
  and dV.
* The entry points enqueue on the caller's stream: the same calls made on a
  side stream (torch.cuda.Stream, default priority) give bit-identical
  results, ordered after the producer of their inputs by the stream itself.
* The path captures into a HIP graph, and replays with fresh inputs match
  eager runs bit for bit.
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


def test_hip_graph_capture_and_replay():
    """The whole path (metadata, forward, backward) holds only kernel
    launches on the caller's stream -- no allocation, memset, copy or
    synchronisation inside the library -- so it can be captured into a HIP
    graph.  Each replay, with new values copied into the captured inputs and
    eager work in between, must equal the eager results bit for bit."""
    torch = torch_cuda()
    pl, q, k, v, do = _inputs(torch)
    announce(f"graph capture L={pl.L}")
    se_d = torch.from_numpy(pl.subtree_end).cuda()
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))

    def path():
        meta = pta.tree_meta(se_d)
        o, lse = pta.attn_fwd(qd, kd, vd, meta)
        dq, dk, dv = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
        return o, lse, dq, dk, dv

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = path()
    gen = torch.Generator().manual_seed(99)
    for rep in range(3):
        for dst in (qd, kd, vd, dod):  # new inputs, copied into the captured buffers
            dst.copy_((torch.randn(dst.shape, generator=gen) * 0.1).to(dst.dtype))
        torch.cuda.synchronize()
        ref = path()  # eager, on the same inputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), out, ref):
            assert torch.equal(x, y), f"replay {rep}: {name}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_phases_one_by_one_match_the_whole_backward(dtype):
    """tree_attn_bwd_phase: DELTA, DKDV, DQ run one by one (dQ reading the
    workspace the Delta kernel wrote) and DQ_DELTA, DKDV (the dQ kernel
    forming Delta itself, as the whole backward does) leave the same
    workspace and the same gradients as tree_attn_bwd.  Delta's two
    summation orders differ in the last bits, so the workspaces agree to
    fp32 rounding and the gradients to the bf16 bound (fp32: 1e-5)."""
    import numpy as np
    from gpu_common import BF16_ATOL, BF16_RTOL
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("multiturn-small")
    (pl,), _ = pta.pack(ids, mask, M)
    hq, hkv, d = (4, 2, 64) if dtype == "fp32" else (8, 2, 128)
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, dtype, std, 4343)
    announce(f"phases {dtype} L={pl.L}")
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    ref = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
    code = pta.DTYPE_FP32 if dtype == "fp32" else pta.DTYPE_BF16
    nbytes = pta.bwd_workspace_bytes(pl.L, hq, d, code)
    runs = {}
    for name, phases in (("split", (pta.BWD_DELTA, pta.BWD_DKDV, pta.BWD_DQ)),
                         ("fused", (pta.BWD_DQ_DELTA, pta.BWD_DKDV))):
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        for ph in phases:
            pta.attn_bwd_phase(ph, qd, kd, vd, o, lse, dod, dq, dk, dv, meta, ws)
        torch.cuda.synchronize()
        runs[name] = (ws, (dq, dk, dv))
    n = 2 * pl.L * hq if dtype == "bf16" else pl.L * hq  # bf16 keeps -Delta and -LSE / scale, fp32 Delta
    wa = runs["split"][0][: 4 * n].view(torch.float32).cpu().numpy()
    wb = runs["fused"][0][: 4 * n].view(torch.float32).cpu().numpy()
    fin = np.isfinite(wa)
    assert np.array_equal(fin, np.isfinite(wb)) and np.array_equal(wa[~fin], wb[~fin])
    assert np.allclose(wb[fin], wa[fin], rtol=1e-5, atol=1e-6)
    atol, rtol = (1e-5, 1e-5) if dtype == "fp32" else (BF16_ATOL, BF16_RTOL)
    for run in ("split", "fused"):
        for name, x, y in zip(("dQ", "dK", "dV"), runs[run][1], ref):
            assert torch.allclose(x.float(), y.float(), atol=atol, rtol=rtol), f"{run} {name}"
