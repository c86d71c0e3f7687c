"""Trie-packed tree attention for AMD MI355X (gfx950).

Rollout sequences that share prefixes are packed into compressed prefix
tries (host C++ packer), per-token metadata and 128x128 tile classes are
derived on the GPU, and forward / backward attention run in hand-written
HIP kernels with bf16 MFMA.  Everything sits behind the C ABI of
``include/tree_attn.h`` (libtreeattn.so); this package only marshals
arguments into it.
"""

from ._lib import (TreeAttnError, lib, library_path, DTYPE_BF16, DTYPE_FP32, BLOCK,  # noqa: F401
                   BWD_ALL, BWD_DELTA, BWD_DKDV, BWD_DQ, BWD_DQ_DELTA, BWD_STATIC_SCRATCH_BYTES)
from .api import (  # noqa: F401
    PackedTrie,
    TreeMeta,
    pack,
    pack_concat,
    pack_batch,
    partition,
    tree_meta,
    meta_workspace_bytes,
    bwd_workspace_bytes,
    attn_fwd,
    attn_bwd,
    attn_bwd_phase,
    attn_bwd_noalloc,
    dfs_plan,
    dfs_workspace_bytes,
    attn_dfs,
    tree_attention,
    logits_stats,
    gather_logprobs,
    tree_logprobs,
    tree_logprobs_chunked,
    rope,
    tree_rope,
    rope_table,
    attn_fwd_rope,
    attn_bwd_rope,
    tree_attention_rope,
)
