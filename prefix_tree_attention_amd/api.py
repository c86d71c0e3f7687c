"""Python face of libtreeattn: argument marshalling only.

Every step of the path -- packing, metadata, forward, backward -- runs in the
library (C++ on the host for the packer, HIP kernels on the GPU for the
rest).  PyTorch provides device memory and the current stream."""

from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import numpy as np

from ._lib import (BLOCK, DTYPE_BF16, DTYPE_FP32, DfsPlan, PackStats, TrieView, TreeAttnError, check, lib)


# ---------------------------------------------------------------------------
# packer (host)
# ---------------------------------------------------------------------------
@dataclass
class PackedTrie:
    """One packed trie, copied out of the library's pack."""
    n_tokens: int
    L: int
    token_ids: np.ndarray
    node_id: np.ndarray
    subtree_end: np.ndarray
    node_start: np.ndarray
    node_end: np.ndarray
    node_parent: np.ndarray
    seq_ids: np.ndarray
    seq_iv_ptr: np.ndarray
    seq_iv: np.ndarray  # [k, 2]

    @property
    def n_nodes(self) -> int:
        return int(self.node_start.shape[0])

    def sequence_indices(self, k: int) -> np.ndarray:
        a, b = int(self.seq_iv_ptr[k]), int(self.seq_iv_ptr[k + 1])
        return np.concatenate([np.arange(s, e + 1) for s, e in self.seq_iv[a:b]])


def _arr(ptr, n) -> np.ndarray:
    if n == 0:
        return np.zeros(0, np.int32)
    return np.ctypeslib.as_array(ptr, shape=(int(n),)).copy()


_ORDERS = {"ffd": 0, "prefix": 1}  # TREE_PACK_FFD, TREE_PACK_PREFIX


def _pack_handle(ids, mask, max_tokens_per_mb, block_size, pad_to_maximum, pad_id, order):
    """Validate the batch and call ``tree_pack_ordered``; returns the
    library-owned pack handle and the contiguous int32 ids."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    if ids.ndim != 2 or ids.shape != mask.shape:
        raise TreeAttnError(-5, "ids and mask must both be [B, S]")
    if order not in _ORDERS:
        raise TreeAttnError(-5, f"order must be one of {sorted(_ORDERS)} (got {order!r})")
    h = ctypes.c_void_p()
    check(lib().tree_pack_ordered(ids.ctypes.data, mask.ctypes.data, ids.shape[0], ids.shape[1],
                                  int(max_tokens_per_mb), int(block_size), int(bool(pad_to_maximum)), int(pad_id),
                                  _ORDERS[order], ctypes.byref(h)))
    return h, ids


def pack(ids, mask, max_tokens_per_mb: int, block_size: int = BLOCK, pad_to_maximum: bool = False,
         pad_id: int = 0, order: str = "ffd"):
    """Pack a padded [B, S] batch into tries (``tree_pack_ordered``; order
    ``"ffd"`` is the pages' first-fit decreasing, ``"prefix"`` the
    lexicographic next-fit packing).  Returns ``(tries, stats)`` with
    ``stats`` a dict of the pack's accounting."""
    L = lib()
    h, ids = _pack_handle(ids, mask, max_tokens_per_mb, block_size, pad_to_maximum, pad_id, order)
    try:
        tries = []
        for t in range(L.tree_pack_num_tries(h)):
            v = TrieView()
            check(L.tree_pack_trie(h, t, ctypes.byref(v)))
            n_iv = int(_arr(v.seq_iv_ptr, v.n_seqs + 1)[-1])
            tries.append(PackedTrie(
                n_tokens=int(v.n_tokens), L=int(v.L),
                token_ids=_arr(v.token_ids, v.L), node_id=_arr(v.node_id, v.L),
                subtree_end=_arr(v.subtree_end, v.L), node_start=_arr(v.node_start, v.n_nodes),
                node_end=_arr(v.node_end, v.n_nodes), node_parent=_arr(v.node_parent, v.n_nodes),
                seq_ids=_arr(v.seq_ids, v.n_seqs), seq_iv_ptr=_arr(v.seq_iv_ptr, v.n_seqs + 1),
                seq_iv=_arr(v.seq_iv, 2 * n_iv).reshape(-1, 2)))
        s = PackStats()
        check(L.tree_pack_stats(h, ctypes.byref(s)))
        stats = {k: getattr(s, k) for k, _ in PackStats._fields_}
    finally:
        L.tree_pack_free(h)
    return tries, stats


def pack_concat(ids, mask, max_tokens_per_mb: int, block_size: int = BLOCK, pad_to_maximum: bool = False,
                pad_id: int = 0, order: str = "ffd"):
    """Pack a batch and lay its tries end to end (``tree_pack_ordered``
    then ``tree_pack_concat``), for one launch over the whole batch.
    Returns ``(subtree_end, lengths, stats)``: the concatenated int32 subtree
    ends, each trie's padded length in order, and the pack's accounting."""
    L = lib()
    h, ids = _pack_handle(ids, mask, max_tokens_per_mb, block_size, pad_to_maximum, pad_id, order)
    try:
        total = ctypes.c_int64()
        check(L.tree_pack_concat(h, None, 0, ctypes.byref(total)))
        se = np.empty(int(total.value), dtype=np.int32)
        check(L.tree_pack_concat(h, se.ctypes.data, se.size, ctypes.byref(total)))
        lengths = []
        for t in range(L.tree_pack_num_tries(h)):
            v = TrieView()
            check(L.tree_pack_trie(h, t, ctypes.byref(v)))
            lengths.append(int(v.L))
        s = PackStats()
        check(L.tree_pack_stats(h, ctypes.byref(s)))
        stats = {k: getattr(s, k) for k, _ in PackStats._fields_}
    finally:
        L.tree_pack_free(h)
    return se, lengths, stats


def pack_batch(ids, mask, max_tokens_per_mb: int, block_size: int = BLOCK, pad_to_maximum: bool = False,
               pad_id: int = 0, order: str = "ffd"):
    """Pack a batch into the concatenated layout and return everything the
    attention and log-probability calls need: ``(subtree_end, token_ids,
    row_positions, lengths, stats)``.  ``token_ids`` is the packed ids
    (``tree_pack_concat_ids``), ``row_positions`` the int32 [B, S] packed
    position of each row's k-th real token, -1 after it
    (``tree_pack_row_positions``).  ``order`` as in ``pack``."""
    L = lib()
    h, ids = _pack_handle(ids, mask, max_tokens_per_mb, block_size, pad_to_maximum, pad_id, order)
    try:
        total = ctypes.c_int64()
        check(L.tree_pack_concat(h, None, 0, ctypes.byref(total)))
        se = np.empty(int(total.value), dtype=np.int32)
        check(L.tree_pack_concat(h, se.ctypes.data, se.size, ctypes.byref(total)))
        tok = np.empty(int(total.value), dtype=np.int32)
        check(L.tree_pack_concat_ids(h, tok.ctypes.data, tok.size))
        rp = np.empty(ids.shape, dtype=np.int32)
        check(L.tree_pack_row_positions(h, rp.ctypes.data, rp.size))
        lengths = []
        for t in range(L.tree_pack_num_tries(h)):
            v = TrieView()
            check(L.tree_pack_trie(h, t, ctypes.byref(v)))
            lengths.append(int(v.L))
        st = PackStats()
        check(L.tree_pack_stats(h, ctypes.byref(st)))
        stats = {k: getattr(st, k) for k, _ in PackStats._fields_}
    finally:
        L.tree_pack_free(h)
    return se, tok, rp, lengths, stats


def partition(ids, mask, K: int):
    """``tree_partition``: split the batch's rows over K workers in DFS
    order, minimising the largest per-worker prefix-tree size.  Returns
    ``(group [B] int32, max_cost, costs [K] int64)``."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    if ids.ndim != 2 or ids.shape != mask.shape:
        raise TreeAttnError(-5, "ids and mask must both be [B, S]")
    group = np.empty(ids.shape[0], dtype=np.int32)
    costs = np.empty(max(int(K), 1), dtype=np.int64)
    tau = ctypes.c_int64()
    check(lib().tree_partition(ids.ctypes.data, mask.ctypes.data, ids.shape[0], ids.shape[1], int(K),
                               group.ctypes.data, ctypes.byref(tau), costs.ctypes.data))
    return group, int(tau.value), costs


# ---------------------------------------------------------------------------
# device side
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def meta_workspace_bytes(L: int) -> int:
    return int(lib().tree_meta_workspace_bytes(int(L)))


def bwd_workspace_bytes(L: int, hq: int, d: int, dtype: int = DTYPE_BF16) -> int:
    return int(lib().tree_attn_bwd_workspace_bytes(int(L), int(hq), int(d), int(dtype)))


@dataclass
class TreeMeta:
    """Device metadata of one trie (the library's analogue of the guide's
    TreeAttentionMeta.from_trie): subtree ends, position ids, tile classes
    and the attention kernels' tile lists."""
    L: int
    se: "object"          # int32 [L] device
    pos: "object"         # int32 [L] device
    tile_class: "object"  # uint8 [nb, nb] device
    ws: "object"          # uint8 workspace device


def tree_meta(subtree_end, device=None) -> TreeMeta:
    """Run ``tree_meta`` on a trie's subtree ends (numpy array or device
    tensor)."""
    torch = _torch()
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    se = torch.as_tensor(np.asarray(subtree_end, np.int32) if not torch.is_tensor(subtree_end) else subtree_end)
    se = se.to(device=device, dtype=torch.int32).contiguous()
    L = int(se.numel())
    nb = L // BLOCK
    pos = torch.empty(L, dtype=torch.int32, device=device)
    tc = torch.empty((nb, nb), dtype=torch.uint8, device=device)
    nbytes = meta_workspace_bytes(L)
    if nbytes == 0:
        raise TreeAttnError(-5, f"bad packed length {L}")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check(lib().tree_meta(_ptr(se), L, _ptr(pos), _ptr(tc), _ptr(ws), nbytes, _stream(device)))
    return TreeMeta(L, se, pos, tc, ws)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TreeAttnError(-5, f"unsupported dtype {t.dtype}")


def _check_qkv(q, k, v, meta):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise TreeAttnError(-5, f"{name} must be a contiguous device tensor")
        if t.dim() != 3 or t.shape[0] != meta.L:
            raise TreeAttnError(-5, f"{name} must be [L={meta.L}, H, D], got {tuple(t.shape)}")
    if k.shape != v.shape or q.shape[2] != k.shape[2] or q.dtype != k.dtype or q.dtype != v.dtype:
        raise TreeAttnError(-5, "q/k/v shapes or dtypes disagree")


def _check_out(name, t, like_shape, like_dtype, device):
    if t.shape != like_shape or t.dtype != like_dtype or not t.is_contiguous() or t.device != device:
        raise TreeAttnError(-5, f"{name} must be a contiguous {like_dtype} tensor of shape {tuple(like_shape)} "
                                f"on {device}")
    return t


def attn_fwd(q, k, v, meta: TreeMeta, scale: float | None = None, o=None, lse=None):
    """``tree_attn_fwd``: returns (o [L,Hq,D], lse [Hq,L] fp32).  ``o`` and
    ``lse`` may be given (caller-owned outputs, fully overwritten)."""
    torch = _torch()
    _check_qkv(q, k, v, meta)
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else _check_out("o", o, q.shape, q.dtype, q.device)
    lse = (torch.empty((hq, L), dtype=torch.float32, device=q.device) if lse is None
           else _check_out("lse", lse, (hq, L), torch.float32, q.device))
    check(lib().tree_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(meta.se), _ptr(meta.ws), L, hq,
                              hkv, d, scale, _dtype_code(q), _stream(q.device)))
    return o, lse


def attn_bwd(q, k, v, o, lse, do, meta: TreeMeta, scale: float | None = None, workspace=None, dq=None, dk=None,
             dv=None):
    """``tree_attn_bwd``: returns (dq, dk, dv).  The outputs may be given
    (caller-owned, fully overwritten), and so may the workspace."""
    torch = _torch()
    _check_qkv(q, k, v, meta)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise TreeAttnError(-5, f"{name} must match q")
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    nbytes = bwd_workspace_bytes(L, hq, d, code)
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else _check_out("dq", dq, q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_out("dk", dk, k.shape, k.dtype, k.device)
    dv = torch.empty_like(v) if dv is None else _check_out("dv", dv, v.shape, v.dtype, v.device)
    if ws.numel() < nbytes:
        raise TreeAttnError(-6, f"workspace holds {ws.numel()} bytes, {nbytes} needed")
    check(lib().tree_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse.contiguous()), _ptr(do), _ptr(dq),
                              _ptr(dk), _ptr(dv), _ptr(meta.se), _ptr(meta.ws), _ptr(ws), ws.numel(), L, hq, hkv,
                              d, scale, code, _stream(q.device)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, meta: TreeMeta, scale: float | None = None, dq=None, dk=None, dv=None):
    """``tree_attn_bwd_noalloc``: the backward with the library's static
    per-device scratch as its workspace (no device allocation inside the
    library; outputs are allocated here unless given).  Returns (dq, dk, dv)."""
    torch = _torch()
    _check_qkv(q, k, v, meta)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise TreeAttnError(-5, f"{name} must match q")
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else _check_out("dq", dq, q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_out("dk", dk, k.shape, k.dtype, k.device)
    dv = torch.empty_like(v) if dv is None else _check_out("dv", dv, v.shape, v.dtype, v.device)
    check(lib().tree_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse.contiguous()), _ptr(do), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(meta.se), _ptr(meta.ws), L, hq, hkv, d, scale,
                                      _dtype_code(q), _stream(q.device)))
    return dq, dk, dv


def attn_bwd_phase(phase: int, q, k, v, o, lse, do, dq, dk, dv, meta: TreeMeta, workspace, scale=None):
    """``tree_attn_bwd_phase`` into caller-provided outputs and workspace
    (BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_DQ_DELTA or BWD_ALL); used to time the backward's
    kernels separately."""
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    check(lib().tree_attn_bwd_phase(int(phase), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(meta.se), _ptr(meta.ws), _ptr(workspace),
                                    workspace.numel(), L, hq, hkv, d, scale, _dtype_code(q), _stream(q.device)))


def _autograd_fn():
    torch = _torch()

    class TreeAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, meta, scale):
            o, lse = attn_fwd(q, k, v, meta, scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.meta, ctx.scale = meta, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.meta, ctx.scale)
            return dq, dk, dv, None, None

    return TreeAttentionFn


_FN = None


def tree_attention(q, k, v, meta: TreeMeta, scale: float | None = None):
    """Differentiable tree attention over one packed trie (batch 1):
    q [L,Hq,D], k/v [L,Hkv,D] -> o [L,Hq,D]."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    return _FN.apply(q, k, v, meta, scale)


# ---------------------------------------------------------------------------
# depth-first (DTA) execution
# ---------------------------------------------------------------------------
def _node_table(trie: PackedTrie):
    ns = np.ascontiguousarray(trie.node_start, dtype=np.int32)
    ne = np.ascontiguousarray(trie.node_end, dtype=np.int32)
    npar = np.ascontiguousarray(trie.node_parent, dtype=np.int32)
    return ns, ne, npar


def dfs_plan(trie: PackedTrie, chunk: int = 2048) -> dict:
    """``tree_dfs_plan``: sizes of the depth-first execution of one trie."""
    ns, ne, npar = _node_table(trie)
    plan = DfsPlan()
    check(lib().tree_dfs_plan(ns.ctypes.data, ne.ctypes.data, npar.ctypes.data, ns.size, int(trie.n_tokens),
                              int(chunk), ctypes.byref(plan)))
    return {k: getattr(plan, k) for k, _ in DfsPlan._fields_}


def dfs_workspace_bytes(plan: dict, hq: int, hkv: int, d: int) -> int:
    """``tree_attn_dfs_workspace_bytes`` of a plan from ``dfs_plan``."""
    return int(lib().tree_attn_dfs_workspace_bytes(ctypes.byref(DfsPlan(**plan)), int(hq), int(hkv), int(d)))


def attn_dfs(trie: PackedTrie, q, k, v, do, meta: TreeMeta, scale: float | None = None, chunk: int = 2048,
             o=None, lse=None, dq=None, dk=None, dv=None, workspace=None):
    """``tree_attn_dfs``: forward and backward of one trie by depth-first
    execution (bf16).  Returns (o, lse, dq, dk, dv) in the packed layout."""
    torch = _torch()
    _check_qkv(q, k, v, meta)
    if do.shape != q.shape or do.dtype != q.dtype or not do.is_contiguous():
        raise TreeAttnError(-5, "do must match q")
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ns, ne, npar = _node_table(trie)
    plan = DfsPlan()
    check(lib().tree_dfs_plan(ns.ctypes.data, ne.ctypes.data, npar.ctypes.data, ns.size, int(trie.n_tokens),
                              int(chunk), ctypes.byref(plan)))
    nbytes = int(lib().tree_attn_dfs_workspace_bytes(ctypes.byref(plan), hq, hkv, d))
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if o is None else _check_out("o", o, q.shape, q.dtype, q.device)
    lse = (torch.empty((hq, L), dtype=torch.float32, device=q.device) if lse is None
           else _check_out("lse", lse, (hq, L), torch.float32, q.device))
    dq = torch.empty_like(q) if dq is None else _check_out("dq", dq, q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_out("dk", dk, k.shape, k.dtype, k.device)
    dv = torch.empty_like(v) if dv is None else _check_out("dv", dv, v.shape, v.dtype, v.device)
    check(lib().tree_attn_dfs(ns.ctypes.data, ne.ctypes.data, npar.ctypes.data, ns.size, int(trie.n_tokens),
                              _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(meta.se), _ptr(ws), ws.numel(), L, hq, hkv, d, scale, int(chunk),
                              _stream(q.device)))
    return o, lse, dq, dk, dv


# ---------------------------------------------------------------------------
# log-probabilities of packed logits
# ---------------------------------------------------------------------------
def _check_logits(logits):
    if not logits.is_cuda or not logits.is_contiguous() or logits.dim() != 2:
        raise TreeAttnError(-5, "logits must be a contiguous device tensor [L, V]")


def logits_stats(logits):
    """``tree_logits_stats``: per packed row, (lse [L], entropy [L]) fp32."""
    torch = _torch()
    _check_logits(logits)
    L, V = logits.shape
    lse = torch.empty(L, dtype=torch.float32, device=logits.device)
    ent = torch.empty(L, dtype=torch.float32, device=logits.device)
    check(lib().tree_logits_stats(_ptr(logits), L, V, _dtype_code(logits), _ptr(lse), _ptr(ent),
                                  _stream(logits.device)))
    return lse, ent


def gather_logprobs(logits, lse, ent, token_ids, row_positions, pad_value: float = 0.0):
    """``tree_gather_logprobs``: (logp [B, S], entropy [B, S]) fp32; row r's
    j-th entry is the prediction of its token j + 1, pad_value after the
    row's last prediction.  ``token_ids`` [L] and ``row_positions`` [B, S]
    are int32 device tensors (see ``pack_batch``)."""
    torch = _torch()
    _check_logits(logits)
    L, V = logits.shape
    for name, t, dt in (("lse", lse, torch.float32), ("entropy", ent, torch.float32),
                        ("token_ids", token_ids, torch.int32), ("row_positions", row_positions, torch.int32)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
            raise TreeAttnError(-5, f"{name} must be a contiguous {dt} device tensor")
    if lse.numel() != L or ent.numel() != L or token_ids.numel() != L or row_positions.dim() != 2:
        raise TreeAttnError(-5, "lse / entropy / token_ids must have L entries, row_positions [B, S]")
    B, S = row_positions.shape
    logp = torch.empty((B, S), dtype=torch.float32, device=logits.device)
    oent = torch.empty((B, S), dtype=torch.float32, device=logits.device)
    check(lib().tree_gather_logprobs(_ptr(logits), L, V, _dtype_code(logits), _ptr(lse), _ptr(ent),
                                     _ptr(token_ids), _ptr(row_positions), B, S, float(pad_value), _ptr(logp),
                                     _ptr(oent), _stream(logits.device)))
    return logp, oent


def tree_logprobs(logits, token_ids, row_positions, pad_value: float = 0.0):
    """Per-sequence log-probabilities and entropies of a packed batch:
    ``logits_stats`` then ``gather_logprobs``."""
    lse, ent = logits_stats(logits)
    return gather_logprobs(logits, lse, ent, token_ids, row_positions, pad_value)


def tree_logprobs_chunked(logits_of, L: int, token_ids, row_positions, chunk: int = 1024,
                          pad_value: float = 0.0):
    """``tree_logprobs`` with the logits produced ``chunk`` packed rows at a
    time, so that at most [chunk, V] of them exist at once (the guide's
    chunk_size).  ``logits_of(r0, r1)`` returns the contiguous device
    logits of rows [r0, r1), e.g. ``lambda a, b: hidden[a:b] @ w_head.t()``;
    each chunk runs ``tree_logits_stats`` into its slice of the row
    statistics and ``tree_gather_logprobs_rows`` over its window.  Same
    results as ``tree_logprobs`` on the whole logits, bit for bit."""
    torch = _torch()
    if chunk <= 0:
        raise TreeAttnError(-5, "chunk must be positive")
    for name, t in (("token_ids", token_ids), ("row_positions", row_positions)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise TreeAttnError(-5, f"{name} must be a contiguous int32 device tensor")
    if token_ids.numel() != L or row_positions.dim() != 2:
        raise TreeAttnError(-5, "token_ids must have L entries, row_positions [B, S]")
    dev = token_ids.device
    B, S = row_positions.shape
    lse = torch.empty(L, dtype=torch.float32, device=dev)
    ent = torch.empty(L, dtype=torch.float32, device=dev)
    logp = torch.empty((B, S), dtype=torch.float32, device=dev)
    oent = torch.empty((B, S), dtype=torch.float32, device=dev)
    stream = _stream(dev)
    V = dt = None
    for r0 in range(0, max(L, 1), chunk):
        r1 = min(L, r0 + chunk)
        lg = logits_of(r0, r1) if r1 > r0 else None
        if lg is not None:
            _check_logits(lg)
            if lg.shape[0] != r1 - r0 or lg.device != dev or (V is not None and (lg.shape[1] != V
                                                                                   or lg.dtype != dt)):
                raise TreeAttnError(-5, f"logits_of({r0}, {r1}) must give [{r1 - r0}, V] on the same device, "
                                        "with one V and dtype for every chunk")
            V, dt = lg.shape[1], lg.dtype
            check(lib().tree_logits_stats(_ptr(lg), r1 - r0, V, _dtype_code(lg),
                                          ctypes.c_void_p(lse.data_ptr() + 4 * r0),
                                          ctypes.c_void_p(ent.data_ptr() + 4 * r0), stream))
        check(lib().tree_gather_logprobs_rows(_ptr(lg) if lg is not None else None, r0, r1 - r0, L, V or 1,
                                              _dtype_code(lg) if lg is not None else 0, _ptr(lse), _ptr(ent),
                                              _ptr(token_ids), _ptr(row_positions), B, S, float(pad_value),
                                              _ptr(logp), _ptr(oent), stream))
    return logp, oent


# ---------------------------------------------------------------------------
# rotary embedding by tree position ids
# ---------------------------------------------------------------------------
def rope(x, pos, base: float = 1e6, inverse: bool = False, out=None):
    """``tree_rope``: rotate head vectors x [L, H, D] by the tree position
    ids ``pos`` [L] (int32 device, e.g. ``tree_meta(...).pos``); in place
    when ``out is x``.  ``inverse`` rotates back (the gradient map)."""
    torch = _torch()
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 3:
        raise TreeAttnError(-5, "x must be a contiguous device tensor [L, H, D]")
    if not pos.is_cuda or pos.dtype != torch.int32 or pos.numel() != x.shape[0] or not pos.is_contiguous():
        raise TreeAttnError(-5, "pos must be a contiguous int32 device tensor [L]")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise TreeAttnError(-5, "out must match x")
    L, H, D = x.shape
    check(lib().tree_rope(_ptr(x), _ptr(y), _ptr(pos), L, H, D, float(base), int(bool(inverse)), _dtype_code(x),
                          _stream(x.device)))
    return y


def _rope_fn():
    torch = _torch()

    class _Rope(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, pos, base):
            ctx.save_for_backward(pos)
            ctx.base = base
            return rope(x.contiguous(), pos, base)

        @staticmethod
        def backward(ctx, gy):
            (pos,) = ctx.saved_tensors
            return rope(gy.contiguous(), pos, ctx.base, inverse=True), None, None

    return _Rope


def rope_table(L: int, d: int, base: float = 1e6, device=None):
    """``tree_rope_table``: (cos, sin) of every position < L, float32
    [L, d/2, 2] on the device, for the fused-rotation attention calls."""
    torch = _torch()
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    nbytes = int(lib().tree_rope_table_bytes(int(L), int(d)))
    if nbytes == 0:
        raise TreeAttnError(-5, f"bad table shape L={L} D={d}")
    tab = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    check(lib().tree_rope_table(float(base), int(L), int(d), _ptr(tab), nbytes, _stream(device)))
    return tab


def attn_fwd_rope(q, k, v, meta: TreeMeta, tab, scale: float | None = None, o=None, lse=None):
    """``tree_attn_fwd_rope``: attention of the rotated q, k (rotation fused
    into the kernels).  Returns (o, lse, q_rot, k_rot)."""
    torch = _torch()
    _check_qkv(q, k, v, meta)
    if q.dtype != torch.bfloat16:
        raise TreeAttnError(-5, "the fused rotation runs in bf16")
    L, hq, d = q.shape
    hkv = k.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if o is None else _check_out("o", o, q.shape, q.dtype, q.device)
    lse = (torch.empty((hq, L), dtype=torch.float32, device=q.device) if lse is None
           else _check_out("lse", lse, (hq, L), torch.float32, q.device))
    q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
    check(lib().tree_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(q_rot), _ptr(k_rot),
                                   _ptr(meta.pos), _ptr(tab), tab.numel() * 4, _ptr(meta.se), _ptr(meta.ws), L, hq,
                                   hkv, d, scale, _stream(q.device)))
    return o, lse, q_rot, k_rot


def attn_bwd_rope(q_rot, k_rot, v, o, lse, do, meta: TreeMeta, tab, scale: float | None = None, dq=None, dk=None,
                  dv=None, workspace=None):
    """``tree_attn_bwd_rope``: gradients w.r.t. the unrotated q and k (and
    v), from the forward's q_rot, k_rot, o and lse."""
    torch = _torch()
    _check_qkv(q_rot, k_rot, v, meta)
    L, hq, d = q_rot.shape
    hkv = k_rot.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = bwd_workspace_bytes(L, hq, d)
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=q_rot.device)
    dq = torch.empty_like(q_rot) if dq is None else _check_out("dq", dq, q_rot.shape, q_rot.dtype, q_rot.device)
    dk = torch.empty_like(k_rot) if dk is None else _check_out("dk", dk, k_rot.shape, k_rot.dtype, k_rot.device)
    dv = torch.empty_like(v) if dv is None else _check_out("dv", dv, v.shape, v.dtype, v.device)
    check(lib().tree_attn_bwd_rope(_ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(o), _ptr(lse.contiguous()),
                                   _ptr(do.contiguous()), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(meta.pos), _ptr(tab),
                                   tab.numel() * 4, _ptr(meta.se), _ptr(meta.ws), _ptr(ws), ws.numel(), L, hq, hkv,
                                   d, scale, _stream(q_rot.device)))
    return dq, dk, dv


def _attn_rope_fn():
    torch = _torch()

    class TreeAttentionRopeFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, meta, tab, scale):
            o, lse, q_rot, k_rot = attn_fwd_rope(q, k, v, meta, tab, scale)
            ctx.save_for_backward(q_rot, k_rot, v, o, lse, tab)
            ctx.meta, ctx.scale = meta, scale
            return o

        @staticmethod
        def backward(ctx, do):
            q_rot, k_rot, v, o, lse, tab = ctx.saved_tensors
            dq, dk, dv = attn_bwd_rope(q_rot, k_rot, v, o, lse, do.contiguous(), ctx.meta, tab, ctx.scale)
            return dq, dk, dv, None, None, None

    return TreeAttentionRopeFn


_ROPE_FN = None


def tree_attention_rope(q, k, v, meta: TreeMeta, tab, scale: float | None = None):
    """Differentiable tree attention with the rotary embedding by tree
    position ids fused into the kernels: attention(rot(q), rot(k), v)."""
    global _ROPE_FN
    if _ROPE_FN is None:
        _ROPE_FN = _attn_rope_fn()
    return _ROPE_FN.apply(q, k, v, meta, tab, scale)


def tree_rope(x, pos, base: float = 1e6):
    """Differentiable rotary embedding by tree position ids (the backward is
    the inverse rotation of the incoming gradient)."""
    return _rope_fn().apply(x, pos, base)
