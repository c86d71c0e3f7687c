"""Shared helpers of the GPU parity tests (not collected by pytest)."""

from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import workloads
import prefix_tree_attention_amd as pta

from checks import (BF16_ATOL, BF16_RTOL, E2E_GRAD_VEC_FLOOR, F32_ATOL, F32_RTOL, assert_attn_close,  # noqa: F401
                    assert_close, attn_tol)


def grad_floor(dtype: str):
    """Per-vector floor for dQ / dK of a backward fed the GPU forward's O."""
    return E2E_GRAD_VEC_FLOOR if dtype == "bf16" else None


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    if not os.path.exists(pta.library_path()):
        raise RuntimeError("libtreeattn.so is not built")
    return torch


def run_attention(torch, qd, kd, vd, dod, meta, scale=None):
    """tree_attn_fwd, and tree_attn_bwd when ``dod`` is given, into outputs
    pre-filled with NaN and a backward workspace filled with 0xFF bytes (NaN
    floats), so an output region a kernel fails to write, or a workspace
    word it reads before writing, cannot pass as the allocator's zeros.
    Returns (o, lse) or (o, lse, dq, dk, dv) on the device."""
    L, hq, _ = qd.shape
    nan = float("nan")
    o = torch.full_like(qd, nan)
    lse = torch.full((hq, L), nan, dtype=torch.float32, device=qd.device)
    o, lse = pta.attn_fwd(qd, kd, vd, meta, scale, o=o, lse=lse)
    if dod is None:
        return o, lse
    code = pta.DTYPE_BF16 if qd.dtype == torch.bfloat16 else pta.DTYPE_FP32
    ws = torch.full((pta.bwd_workspace_bytes(L, hq, qd.shape[2], code),), 255, dtype=torch.uint8, device=qd.device)
    dq, dk, dv = (torch.full_like(t, nan) for t in (qd, kd, vd))
    pta.attn_bwd(qd, kd, vd, o, lse, dod, meta, scale, workspace=ws, dq=dq, dk=dk, dv=dv)
    return o, lse, dq, dk, dv


_KV_GROUP_REFS = {}


def oracle_kv_group(m, Qs, K, V, Gs, scale, tag):
    """The oracle's fp32 forward and backward for the query heads of one
    key/value head on a dense mask ``m``: (O [L, g, D], LSE [g, L], dQ
    [L, g, D], dK [L, 1, D], dV [L, 1, D]).  Cached for the test session by
    the inputs' bytes, so tests that check the same inputs (the packed and
    the depth-first runs of one workload) pay for it once."""
    import hashlib

    h = hashlib.sha1()
    for x in (m, *Qs, K, V, *Gs):
        h.update(np.ascontiguousarray(x).tobytes())
    key = (h.hexdigest(), float(scale))
    if key in _KV_GROUP_REFS:
        announce(f"  {tag}: oracle reused")
        return _KV_GROUP_REFS[key]
    L, g, D = m.shape[0], len(Qs), K.shape[2]
    o_ref, lse_ref, dq_ref = np.zeros((L, g, D)), np.zeros((g, L)), np.zeros((L, g, D))
    dk_ref, dv_ref = np.zeros((L, 1, D)), np.zeros((L, 1, D))
    for x, (Q, G) in enumerate(zip(Qs, Gs)):
        o1, l1 = oracle.attention_forward(Q, K, V, m, scale, dtype=np.float32)
        q1, k1, v1 = oracle.attention_backward(Q, K, V, o1, l1, G, m, scale, dtype=np.float32)
        o_ref[:, x], lse_ref[x], dq_ref[:, x] = o1[:, 0], l1[0], q1[:, 0]
        dk_ref += k1
        dv_ref += v1
        announce(f"  {tag}: oracle head {x} done")
    _KV_GROUP_REFS.clear()  # one workload's references at a time (hundreds of MB)
    _KV_GROUP_REFS[key] = (o_ref, lse_ref, dq_ref, dk_ref, dv_ref)
    return _KV_GROUP_REFS[key]


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def meta_layout(L: int) -> dict:
    """Word offsets of the tree_meta workspace (the layout documented in the
    library's internal device header), for reading the tile lists back."""
    nb = L // 128
    T = nb * (nb + 1) // 2
    pad = lambda w: (w + 63) // 64 * 64  # noqa: E731
    o, out = 0, {}
    for name, size in (("hdr", 64), ("blk_min", pad(nb)), ("blk_max", pad(nb)), ("hist", pad(L + 1)),
                       ("row_cnt", pad(nb)), ("row_ptr", pad(nb + 1)), ("row_ent", pad(T)),
                       ("col_cnt", pad(nb)), ("col_ptr", pad(nb + 1)), ("col_ent", pad(T)),
                       ("q_order", pad(nb)), ("k_order", pad(nb)), ("blk_cnt", pad(nb)), ("blk_hsum", pad(nb)),
                       ("hi64", pad(2 * nb)), ("g_order", pad(2 * nb))):
        out[name] = o
        o += size
    out["nb"] = nb
    return out


def key_groups_ref(se):
    """The dK/dV key groups the metadata forms (the rule stated in the
    library's internal device header), in plain Python: (per-64-key-chunk
    maximum subtree end, first chunk of each group in chunk order, whether
    the four-chunk fallback applied)."""
    se = np.asarray(se, np.int64)
    n64 = len(se) // 64
    hi = np.full(n64, -1, np.int64)
    for c in range(n64):
        s = se[64 * c:64 * c + 64]
        s = s[s >= 0]
        if s.size:
            hi[c] = s.max()
    starts, rs = [], 0
    for c in range(n64):
        if c == 0 or hi[c - 1] != hi[c]:
            rs = c
        if (c - rs) % 4 == 0:
            starts.append(c)
    real = np.nonzero(hi >= 0)[0]
    c_end = int(real[-1]) + 1 if real.size else 0
    fallback = sum(c < c_end for c in starts) > (c_end + 3) // 4 + (c_end + 15) // 16
    if fallback:
        starts = list(range(0, n64, 4))
    return hi, starts, fallback


def dkdv_workgroups(c_end: int) -> int:
    """The dK/dV launch's workgroups per key/value head for groups before
    chunk c_end (the library's bound plus its slack of 2)."""
    return (c_end + 3) // 4 + (c_end + 15) // 16 + 2


def small_cases():
    """(name, ids, mask, M) of the scaled-down workloads and the worked example."""
    ids, mask = workloads.worked_example()
    yield "worked-example", ids, mask, 128
    for k in workloads.SMALL_KINDS:
        ids, mask, M = workloads.small_workload(k)
        yield k, ids, mask, M


def bf16_ref(t):
    """bf16 (or fp32) torch tensor -> float64 numpy of the same values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def sample_rows(p_oracle, n_random: int, seed: int):
    """Rows for sampled checks: node starts/ends, tile edges, random rows and
    a few pads."""
    rng = np.random.default_rng(seed)
    n, L = p_oracle.n_tokens, p_oracle.L
    rows = set()
    for s, e in zip(p_oracle.node_start[:16], p_oracle.node_end[:16]):
        rows.update({int(s), int(e)})
    rows.update({0, n - 1, min(127, n - 1), min(128, n - 1)})
    rows.update(int(x) for x in rng.integers(0, n, n_random))
    if L > n:
        rows.update({n, L - 1})
    return sorted(rows)
