"""CPU oracle for trie-packed tree attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or helper with the HIP library under ``prefix_tree_attention_amd/`` and
never imports it.

It is deliberately plain and slow: a token-level dictionary trie, a dense
boolean ancestor mask built by walking the trie, and naive masked-softmax
attention with closed-form gradients.  Every function cites the passage of
the source pages it follows.  The pages are:

  [TT]  "AReaL Tree Training 完全指南：基于共享前缀打包的 RL 训练加速原理与实战配置"
        (2kiu.com) -- the tree-training guide: packing, position ids,
        block-mask attention, validation errors, the tree_token_ratio metric.
  [DTA] "AREAL-DTA: Dynamic Tree Attention for Efficient Reinforcement
        Learning of Large Language Models" (papercache.org paper notes) --
        problem formulation (loss summed over root-to-leaf sequences, shared
        prefixes computed once and their gradients accumulated).

Every oracle function is pinned by a test in ``tests/`` that does not re-type
its formula (worked example from [TT]'s packing figure, per-sequence causal
attention through a library routine, autograd and finite differences, brute
force on tiny inputs, closed-form counts).  No function here is "parity
unpinned".
"""

from .packing import (  # noqa: F401
    PackError,
    OracleTrie,
    PackedTrie,
    extract_sequences,
    ffd_build_tries,
    prefix_order_build_tries,
    compress_trie,
    flatten_trie,
    pack,
    dense_ancestor_mask,
    ancestors_of,
    descendants_of,
    position_ids,
    tile_classes,
    accounting,
    BLOCK_SIZE,
)
from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_delta,
    attention_forward_rows,
    attention_dq_rows,
    attention_dkdv_cols,
)
from .logprobs import gather_tree_logprobs_entropy, prediction_logprob_entropy  # noqa: F401
from .partition import dfs_order, tree_cost, partition, partition_batch, dummy_tries  # noqa: F401
from .rope import rope  # noqa: F401
from .dfs import dfs_attention  # noqa: F401
