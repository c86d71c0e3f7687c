"""Rotary embedding by tree position ids on the GPU (tree_rope) against the
oracle, with positions from tree_meta on the device and from the oracle's
dense ancestor mask on the host:

* elementwise on scaled-down packed batches, bf16 and fp32, D = 64 and 128,
  forward and inverse, in place and out of place;
* the autograd wrapper: the gradient is the inverse rotation;
* the deep-shared 32K layout, every element of a [32768, 32, 128] bf16 Q.

Tolerance: angles, sines and cosines are formed in float64 and the rotation
in float32, so a float32 result is within a few float32 ulps of |x|
(2e-6 relative, 1e-6 absolute at N(0, 1) inputs); a bf16 result adds the
bf16 rounding of the output, at most 2^-9 relative (4e-3 relative bound).
"""

import numpy as np
import pytest

import oracle
import workloads
import prefix_tree_attention_amd as pta
from gpu_common import announce, assert_close, torch_cuda

pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-5, 4e-3), "fp32": (1e-6, 2e-6)}


def _positions(torch, ids, mask, M):
    se, tok, rp, lengths, _ = pta.pack_batch(ids, mask, M)
    meta = pta.tree_meta(se)
    to = oracle.pack(ids, mask, M)
    pos_o = np.concatenate([oracle.position_ids(oracle.dense_ancestor_mask(t)) for t in to])
    pos = meta.pos
    assert (pos.cpu().numpy() == pos_o).all()
    return pos, pos_o


@pytest.mark.parametrize("kind,H,D,dt", [("grpo-small", 8, 128, "bf16"), ("deep-small", 4, 64, "fp32"),
                                         ("multiturn-small", 2, 128, "fp32"), ("nested", 3, 64, "bf16")])
def test_small_elementwise(kind, H, D, dt):
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload(kind)
    pos, pos_o = _positions(torch, ids, mask, M)
    L = pos.numel()
    announce(f"rope {kind} L={L} H={H} D={D} {dt}")
    g = torch.Generator().manual_seed(L + D)
    x = torch.randn(L, H, D, generator=g).to(torch.bfloat16 if dt == "bf16" else torch.float32)
    xd = x.cuda()
    atol, rtol = TOL[dt]
    for base in (1e4, 1e6):
        y = pta.rope(xd, pos, base)
        ref = oracle.rope(x.double().numpy(), pos_o, base)
        assert_close(y.float().cpu().numpy(), ref, atol, rtol, f"rope {kind} base {base:g}")
        yi = pta.rope(xd, pos, base, inverse=True)
        refi = oracle.rope(x.double().numpy(), pos_o, base, inverse=True)
        assert_close(yi.float().cpu().numpy(), refi, atol, rtol, f"inverse rope {kind}")
    z = xd.clone()
    pta.rope(z, pos, 1e6, out=z)  # in place
    assert torch.equal(z, pta.rope(xd, pos, 1e6))


def test_autograd_is_inverse_rotation():
    torch = torch_cuda()
    ids, mask, M = workloads.small_workload("grpo-small")
    pos, pos_o = _positions(torch, ids, mask, M)
    L = pos.numel()
    announce(f"rope autograd L={L}")
    g = torch.Generator().manual_seed(3)
    x = torch.randn(L, 4, 64, generator=g).cuda().requires_grad_(True)
    w = torch.randn(L, 4, 64, generator=g)
    (pta.tree_rope(x, pos, 1e6) * w.cuda()).sum().backward()
    ref = oracle.rope(w.double().numpy(), pos_o, 1e6, inverse=True)
    assert_close(x.grad.cpu().numpy(), ref, *TOL["fp32"], "rope gradient")


def test_deep_shared_full_size():
    torch = torch_cuda()
    w = workloads.make_workload("4a")
    se, _, _, _, _ = pta.pack_batch(w.ids, w.mask, w.max_tokens_per_mb)
    meta = pta.tree_meta(se)
    pos_o = np.concatenate([np.arange(16384), np.tile(16384 + np.arange(256), 64)])
    pos_o[se < 0] = 0
    assert (meta.pos.cpu().numpy() == pos_o).all()  # closed form: prefix then every leaf at 16384..16639
    L = len(se)
    announce(f"rope 4a L={L} H=32 D=128 bf16")
    g = torch.Generator().manual_seed(11)
    x = torch.randn(L, 32, 128, generator=g).to(torch.bfloat16)
    y = pta.rope(x.cuda(), meta.pos, 1e6)
    ref = oracle.rope(x.float().numpy(), pos_o, 1e6)
    assert_close(y.float().cpu().numpy(), ref, *TOL["bf16"], "rope 4a")
