"""ctypes loader and signatures of libtreeattn.so (include/tree_attn.h).

The library is built in-tree by ``prefix_tree_attention_amd.build``; there is
no fallback of any kind: if the library is missing or fails to load, every
entry point raises."""

from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

c_i32, c_i64, c_sz, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)

TREE_OK = 0
ERROR_NAMES = {
    -1: "TREE_E_MAX_TOKENS",
    -2: "TREE_E_ALIGN",
    -3: "TREE_E_SEQ_TOO_LONG",
    -4: "TREE_E_EMPTY_SEQ",
    -5: "TREE_E_ARG",
    -6: "TREE_E_WORKSPACE",
    -7: "TREE_E_HIP",
    -8: "TREE_E_NOMEM",
}
DTYPE_BF16, DTYPE_FP32 = 0, 1
BLOCK = 128


class TreeAttnError(RuntimeError):
    """A libtreeattn call returned a negative status."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))


class TrieView(ctypes.Structure):
    _fields_ = [
        ("n_tokens", c_i64), ("L", c_i64), ("n_nodes", c_i64), ("n_seqs", c_i64),
        ("token_ids", P_i32), ("node_id", P_i32), ("subtree_end", P_i32),
        ("node_start", P_i32), ("node_end", P_i32), ("node_parent", P_i32),
        ("seq_ids", P_i32), ("seq_iv_ptr", P_i32), ("seq_iv", P_i32),
    ]


class PackStats(ctypes.Structure):
    _fields_ = [
        ("n_tries", c_i64), ("original_tokens", c_i64), ("tree_tokens", c_i64),
        ("tree_token_ratio", ctypes.c_double), ("n_pairs", c_i64), ("unpacked_pairs", c_i64),
        ("tiles_full", c_i64), ("tiles_partial", c_i64), ("tiles_causal", c_i64),
    ]


class DfsPlan(ctypes.Structure):
    _fields_ = [
        ("rows", c_i64), ("stack_rows", c_i64), ("leaf_rows", c_i64), ("peak_stack_tokens", c_i64),
        ("max_path_tokens", c_i64), ("chunks", c_i64), ("leaf_groups", c_i64), ("max_depth", c_i64),
    ]


# name -> (restype, argtypes), in header order
SIGNATURES = {
    "tree_abi_version": (ctypes.c_int, []),
    "tree_last_error": (ctypes.c_char_p, []),
    "tree_pack": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "tree_pack_ordered": (ctypes.c_int,
                          [c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "tree_pack_num_tries": (c_i64, [c_vp]),
    "tree_pack_trie": (ctypes.c_int, [c_vp, c_i64, ctypes.POINTER(TrieView)]),
    "tree_pack_stats": (ctypes.c_int, [c_vp, ctypes.POINTER(PackStats)]),
    "tree_pack_concat": (ctypes.c_int, [c_vp, c_vp, c_i64, ctypes.POINTER(c_i64)]),
    "tree_pack_concat_ids": (ctypes.c_int, [c_vp, c_vp, c_i64]),
    "tree_pack_row_positions": (ctypes.c_int, [c_vp, c_vp, c_i64]),
    "tree_partition": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, ctypes.POINTER(c_i64), c_vp]),
    "tree_pack_free": (None, [c_vp]),
    "tree_meta_workspace_bytes": (c_sz, [c_i64]),
    "tree_meta": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "tree_attn_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32,
                                     c_f32, c_i32, c_vp]),
    "tree_attn_bwd_workspace_bytes": (c_sz, [c_i64, c_i32, c_i32, c_i32]),
    "tree_attn_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_sz, c_i64, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "tree_attn_bwd_phase": (ctypes.c_int, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_vp, c_sz, c_i64, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "tree_attn_bwd_noalloc": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                             c_i64, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "tree_dfs_plan": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_i32, ctypes.POINTER(DfsPlan)]),
    "tree_attn_dfs_workspace_bytes": (c_sz, [ctypes.POINTER(DfsPlan), c_i32, c_i32, c_i32]),
    "tree_attn_dfs": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_vp, c_vp, c_sz, c_i64, c_i32, c_i32, c_i32, c_f32, c_i32, c_vp]),
    "tree_logits_stats": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "tree_gather_logprobs": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_f32,
                                            c_vp, c_vp, c_vp]),
    "tree_gather_logprobs_rows": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp,
                                                 c_i64, c_i64, c_f32, c_vp, c_vp, c_vp]),
    "tree_rope_table_bytes": (c_sz, [c_i64, c_i32]),
    "tree_rope_table": (ctypes.c_int, [ctypes.c_double, c_i64, c_i32, c_vp, c_sz, c_vp]),
    "tree_attn_fwd_rope": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp,
                                          c_i64, c_i32, c_i32, c_i32, c_f32, c_vp]),
    "tree_attn_bwd_rope": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                          c_vp, c_vp, c_vp, c_sz, c_i64, c_i32, c_i32, c_i32, c_f32, c_vp]),
    "tree_rope": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, ctypes.c_double, c_i32, c_i32, c_vp]),
}
BWD_ALL, BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_DQ_DELTA = 0, 1, 2, 3, 4
BWD_STATIC_SCRATCH_BYTES = 64 << 20  # TREE_BWD_STATIC_SCRATCH_BYTES

_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libtreeattn.so (once) and declare its signatures."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run `python -m prefix_tree_attention_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def check(rc: int) -> None:
    if rc != TREE_OK:
        msg = lib().tree_last_error()
        raise TreeAttnError(rc, msg.decode() if msg else "")
