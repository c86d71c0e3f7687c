"""tree_attn_bwd_noalloc, the backward whose workspace is the library's
static per-device scratch, against tree_attn_bwd (caller workspace) through
the C ABI: bit-identical gradients on two calls in a row, the second on a
smaller trie (so the scratch still holds the first call's larger contents),
in bf16 and the fp32 check mode."""

import math

import pytest

import workloads
import prefix_tree_attention_amd as pta
from gpu_common import announce, torch_cuda

pytestmark = pytest.mark.gpu


def _case(torch, ids, mask, M, hq, hkv, d, dtype, seed):
    pl = pta.pack(ids, mask, M)[0][0]
    std = 1.0 if dtype == "fp32" else 1.0 / math.sqrt(d)
    q, k, v, do = workloads.attention_inputs(pl.L, hq, hkv, d, dtype, std, seed)
    meta = pta.tree_meta(pl.subtree_end)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = pta.attn_fwd(qd, kd, vd, meta)
    return pl, meta, qd, kd, vd, dod, o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_backward_matches_workspace_backward(dtype):
    torch = torch_cuda()
    hq, hkv, d = (32, 8, 128) if dtype == "bf16" else (4, 2, 64)
    w = workloads.make_workload("4b")
    big = (w.ids, w.mask, w.max_tokens_per_mb)
    small = workloads.small_workload("deep-small")
    for step, (ids, mask, M) in enumerate((big, small)):
        pl, meta, qd, kd, vd, dod, o, lse = _case(torch, ids, mask, M, hq, hkv, d, dtype, 70 + step)
        announce(f"noalloc {dtype} call {step + 1}: L={pl.L} hq={hq} "
                 f"workspace {pta.bwd_workspace_bytes(pl.L, hq, d)} bytes")
        ref = pta.attn_bwd(qd, kd, vd, o, lse, dod, meta)
        got = tuple(torch.full_like(t, float("nan")) for t in ref)
        pta.attn_bwd_noalloc(qd, kd, vd, o, lse, dod, meta, dq=got[0], dk=got[1], dv=got[2])
        torch.cuda.synchronize()
        for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(x, y), f"call {step + 1}: {name} differs from tree_attn_bwd"
