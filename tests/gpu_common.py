"""Shared helpers of the GPU parity tests (not collected by pytest)."""

from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import workloads
import prefix_tree_attention_amd as pta

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2   # |gpu - oracle| <= atol + rtol * |oracle|
F32_ATOL, F32_RTOL = 1e-4, 1e-4


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    if not os.path.exists(pta.library_path()):
        raise RuntimeError("libtreeattn.so is not built")
    return torch


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def assert_close(gpu, ref, atol, rtol, what, mask=None):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    bound = atol + rtol * np.where(np.isinf(ref), 0.0, np.abs(ref))
    bad = ~(err <= bound)
    if mask is not None:
        bad &= mask
    fin = np.isfinite(ref) & np.isfinite(gpu)
    rel_l2 = float(np.linalg.norm((gpu - ref)[fin]) / max(np.linalg.norm(ref[fin]), 1e-30))
    print(f"  {what}: max|err|={float(err.max()) if err.size else 0:.3e} rel_l2={rel_l2:.3e}", flush=True)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={gpu[tuple(i)]:.6g} ref={ref[tuple(i)]:.6g}" for i in idx))


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
                       ("p_order", pad((nb + 1) // 2))):
        out[name] = o
        o += size
    out["nb"] = nb
    return out


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
