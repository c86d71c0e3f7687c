"""Oracle packer: extraction, first-fit-decreasing (or prefix-order) trie
building, chain compression, pre-order flattening, padding, the dense ancestor mask, position
ids, 128x128 tile classes and the packed-run accounting.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python and NumPy;
no code is shared with the HIP library.

Readings of points the pages leave open (each one is also listed in the
design notes of the repository):
  * FFD sort key is the real sequence length, descending; equal lengths keep
    their original row order (stable sort).
  * First fit scans the tries in creation order; a sequence goes into the
    first trie whose token count plus the tokens the insertion adds stays
    within ``max_tokens_per_mb``.  Counts are uncompressed trie tokens.
  * Children are laid out in insertion order (the pages' node type keeps
    children in a dict, which iterates in insertion order).
  * Compression merges a node into its only child when both carry the same
    set of sequences; a sequence ending inside a chain therefore splits it.
  * Padding goes to the next multiple of the block size (default) or to
    ``max_tokens_per_mb`` with ``pad_to_maximum``; pad tokens carry
    ``pad_id``, node -1 and subtree end -1, attend to nothing and are
    attended by nothing; their position id is 0.
  * An empty sequence (all-zero mask row) is an error.
  * A trie's sequence list (``all_sequence_ids``) is in insertion order.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 128  # [TT] "两种注意力实现 / FlexAttention + BlockMask": 128-token blocks


class PackError(ValueError):
    """Argument / input error of the packer.

    ``code`` is one of ``"max_tokens"``, ``"align"``, ``"seq_too_long"``,
    ``"empty_seq"``, ``"arg"``.  [TT] "参数背后的源码校验逻辑" lists the
    validation the packing entry point performs: a missing or non-positive
    token budget, a budget that is not a multiple of the block size, and a
    sequence longer than the budget all raise.
    """

    def __init__(self, code: str, msg: str):
        super().__init__(msg)
        self.code = code


# ---------------------------------------------------------------------------
# step 1: extraction
# ---------------------------------------------------------------------------
def extract_sequences(ids: np.ndarray, mask: np.ndarray) -> list[list[int]]:
    """[TT] 树构建流程 step 1: a row's real tokens are its ids where the
    attention mask is non-zero, kept in column order."""
    if ids.ndim != 2 or ids.shape != mask.shape:
        raise PackError("arg", "ids and mask must both be [B, S]")
    return [ids[r][mask[r] != 0].astype(np.int64).tolist() for r in range(ids.shape[0])]


# ---------------------------------------------------------------------------
# step 2: greedy first-fit-decreasing into token-level tries
# ---------------------------------------------------------------------------
class _Tok:
    __slots__ = ("token", "children", "seqs")

    def __init__(self, token):
        self.token = token
        self.children: dict[int, _Tok] = {}  # insertion-ordered
        self.seqs: list[int] = []


class OracleTrie:
    """Uncompressed trie: one node per distinct prefix of the inserted
    sequences, so ``num_tokens`` is the number of tokens the trie stores."""

    def __init__(self):
        self.root = _Tok(None)
        self.num_tokens = 0
        self.sequence_ids: list[int] = []

    def additional_tokens(self, seq: list[int]) -> int:
        """Tokens an insertion of ``seq`` would add: its length minus the
        longest prefix already present ([TT] 树构建流程 step 2, the count of
        extra nodes an insertion needs)."""
        node, shared = self.root, 0
        for t in seq:
            nxt = node.children.get(t)
            if nxt is None:
                break
            node, shared = nxt, shared + 1
        return len(seq) - shared

    def insert(self, seq: list[int], sid: int) -> None:
        node = self.root
        for t in seq:
            nxt = node.children.get(t)
            if nxt is None:
                nxt = _Tok(t)
                node.children[t] = nxt
                self.num_tokens += 1
            nxt.seqs.append(sid)
            node = nxt
        self.sequence_ids.append(sid)


def ffd_build_tries(seqs: list[list[int]], max_tokens: int) -> list[OracleTrie]:
    """[TT] 树构建流程 step 2: first-fit decreasing.  Sequences are taken
    longest first; each goes into the first existing trie whose occupied count
    plus the count the insertion adds fits the budget, otherwise a new trie is
    opened."""
    order = sorted(range(len(seqs)), key=lambda r: len(seqs[r]), reverse=True)  # stable
    tries: list[OracleTrie] = []
    for r in order:
        s = seqs[r]
        for t in tries:
            if t.num_tokens + t.additional_tokens(s) <= max_tokens:
                t.insert(s, r)
                break
        else:
            t = OracleTrie()
            t.insert(s, r)
            tries.append(t)
    return tries


def prefix_order_build_tries(seqs: list[list[int]], max_tokens: int) -> list[OracleTrie]:
    """Prefix-order packing, an option beside the pages' first-fit
    decreasing.  [DTA] section 4 (负载均衡并行化) puts the sequences in
    lexicographic order, the DFS order of one tree over all of them, so that
    a contiguous run of them loses the least sharing.  Here the same order
    fills tries of at most ``max_tokens`` tree tokens: each sequence goes into
    the most recently opened trie if the tokens it adds keep that trie within
    the budget, otherwise it opens a new one.  Reading: ties in the order
    keep the row order, as in the partition."""
    order = sorted(range(len(seqs)), key=lambda r: (list(seqs[r]), r))
    tries: list[OracleTrie] = []
    for r in order:
        s = seqs[r]
        if tries and tries[-1].num_tokens + tries[-1].additional_tokens(s) <= max_tokens:
            tries[-1].insert(s, r)
        else:
            t = OracleTrie()
            t.insert(s, r)
            tries.append(t)
    return tries


# ---------------------------------------------------------------------------
# step 3: compression (and pre-order numbering)
# ---------------------------------------------------------------------------
@dataclass
class CNode:
    tokens: list[int]
    seqs: list[int]
    parent: int
    children: list[int] = field(default_factory=list)


def compress_trie(trie: OracleTrie) -> list[CNode]:
    """[TT] 树构建流程 step 3 and the node type of "核心数据结构": a run of
    single-child nodes whose sequence sets are identical becomes one node.
    Nodes are returned in pre-order (children in insertion order), the order
    of the root's ``nodes`` list."""
    out: list[CNode] = []
    # explicit stack of (token node, parent index); children pushed reversed
    stack = [(c, -1) for c in reversed(list(trie.root.children.values()))]
    while stack:
        tok, parent = stack.pop()
        idx = len(out)
        cn = CNode([tok.token], list(tok.seqs), parent)
        out.append(cn)
        if parent >= 0:
            out[parent].children.append(idx)
        cur = tok
        while len(cur.children) == 1:
            (only,) = cur.children.values()
            if set(only.seqs) != set(cur.seqs):
                break
            cn.tokens.append(only.token)
            cur = only
        for c in reversed(list(cur.children.values())):
            stack.append((c, idx))
    return out


# ---------------------------------------------------------------------------
# step 4: flattening, padding, per-token metadata
# ---------------------------------------------------------------------------
@dataclass
class PackedTrie:
    n_tokens: int
    L: int
    token_ids: np.ndarray     # int32 [L]
    node_id: np.ndarray       # int32 [L], -1 for pads
    subtree_end: np.ndarray   # int32 [L], inclusive, -1 for pads
    node_start: np.ndarray    # int32 [n_nodes]
    node_end: np.ndarray      # int32 [n_nodes] (inclusive)
    node_parent: np.ndarray   # int32 [n_nodes], -1 for children of the root
    seq_ids: np.ndarray       # int32 [n_seqs], insertion order
    seq_iv_ptr: np.ndarray    # int32 [n_seqs + 1]
    seq_iv: np.ndarray        # int32 [k, 2]  (start, end) per visited node
    nodes: list[CNode]

    @property
    def n_nodes(self) -> int:
        return len(self.nodes)

    def sequence_indices(self, k: int) -> np.ndarray:
        """Packed positions of the k-th sequence of this trie, root to leaf
        (the pages' get_sequence_tree_indices, expanded to indices)."""
        a, b = self.seq_iv_ptr[k], self.seq_iv_ptr[k + 1]
        return np.concatenate([np.arange(s, e + 1) for s, e in self.seq_iv[a:b]])


def flatten_trie(trie: OracleTrie, nodes: list[CNode], L: int, pad_id: int) -> PackedTrie:
    """[TT] "核心数据结构" / "打包数据的生成": tokens are laid out node after
    node in pre-order; each node covers the inclusive range [start, end].
    The subtree end of a token is the last index of its node's subtree."""
    nn = len(nodes)
    start = np.zeros(nn, np.int64)
    off = 0
    for v, cn in enumerate(nodes):
        start[v] = off
        off += len(cn.tokens)
    n = off
    assert n == trie.num_tokens
    end = start + np.array([len(cn.tokens) for cn in nodes], np.int64) - 1
    parent = np.array([cn.parent for cn in nodes], np.int64)
    sub_end = end.copy()
    for v in range(nn - 1, -1, -1):  # children follow their parent in pre-order
        if parent[v] >= 0:
            sub_end[parent[v]] = max(sub_end[parent[v]], sub_end[v])

    token_ids = np.full(L, pad_id, np.int64)
    node_id = np.full(L, -1, np.int64)
    se = np.full(L, -1, np.int64)
    for v, cn in enumerate(nodes):
        token_ids[start[v]:end[v] + 1] = cn.tokens
        node_id[start[v]:end[v] + 1] = v
        se[start[v]:end[v] + 1] = sub_end[v]

    ptr = [0]
    ivs: list[tuple[int, int]] = []
    for sid in trie.sequence_ids:
        for v, cn in enumerate(nodes):  # pre-order: ancestors before descendants
            if sid in cn.seqs:
                ivs.append((int(start[v]), int(end[v])))
        ptr.append(len(ivs))

    i32 = lambda a: np.asarray(a, dtype=np.int32)  # noqa: E731
    return PackedTrie(
        n_tokens=n, L=L, token_ids=i32(token_ids), node_id=i32(node_id),
        subtree_end=i32(se), node_start=i32(start), node_end=i32(end),
        node_parent=i32(parent), seq_ids=i32(trie.sequence_ids), seq_iv_ptr=i32(ptr),
        seq_iv=i32(ivs).reshape(-1, 2), nodes=nodes,
    )


def pack(ids, mask, max_tokens_per_mb, block_size: int = BLOCK_SIZE,
         pad_to_maximum: bool = False, pad_id: int = 0, order: str = "ffd") -> list[PackedTrie]:
    """Whole packing path of [TT] "参数背后的源码校验逻辑" and "树构建流程":
    validate, extract, build tries (the pages' first-fit decreasing, or with
    ``order="prefix"`` the prefix-order packing above), compress, flatten and
    pad."""
    if order not in ("ffd", "prefix"):
        raise PackError("arg", f"unknown packing order {order!r}")
    if max_tokens_per_mb is None or int(max_tokens_per_mb) <= 0:
        raise PackError("max_tokens", "max_tokens_per_mb must be a positive integer")
    M = int(max_tokens_per_mb)
    if block_size <= 0:
        raise PackError("arg", "block_size must be positive")
    if M % block_size != 0:
        raise PackError("align", f"max_tokens_per_mb={M} is not a multiple of {block_size}")
    ids = np.asarray(ids)
    mask = np.asarray(mask)
    seqs = extract_sequences(ids, mask)
    for r, s in enumerate(seqs):
        if len(s) == 0:
            raise PackError("empty_seq", f"row {r} has no real token")
        if len(s) > M:
            raise PackError("seq_too_long", f"row {r} has {len(s)} tokens > max_tokens_per_mb={M}")
    out = []
    build = ffd_build_tries if order == "ffd" else prefix_order_build_tries
    for trie in build(seqs, M):
        nodes = compress_trie(trie)
        n = trie.num_tokens
        L = M if pad_to_maximum else -(-n // block_size) * block_size
        out.append(flatten_trie(trie, nodes, L, pad_id))
    return out


# ---------------------------------------------------------------------------
# mask, position ids, tile classes, accounting
# ---------------------------------------------------------------------------
def dense_ancestor_mask(p: PackedTrie) -> np.ndarray:
    """[TT] packing figure: a token attends only to itself and its ancestors.
    Built by walking each node's parent chain in the compressed trie (never
    from the subtree ends).  Pads attend to nothing.  bool [L, L]."""
    m = np.zeros((p.L, p.L), dtype=bool)
    for v in range(p.n_nodes):
        s, e = int(p.node_start[v]), int(p.node_end[v])
        m[s:e + 1, s:e + 1] = np.tril(np.ones((e - s + 1, e - s + 1), dtype=bool))
        u = int(p.node_parent[v])
        while u >= 0:
            m[s:e + 1, int(p.node_start[u]):int(p.node_end[u]) + 1] = True
            u = int(p.node_parent[u])
    return m


def ancestors_of(p: PackedTrie, i: int) -> np.ndarray:
    """Keys visible to packed position i (itself plus its ancestors), by the
    same parent walk as :func:`dense_ancestor_mask`; empty for a pad."""
    v = int(p.node_id[i])
    if v < 0:
        return np.zeros(0, np.int64)
    parts = [np.arange(int(p.node_start[v]), i + 1)]
    u = int(p.node_parent[v])
    while u >= 0:
        parts.append(np.arange(int(p.node_start[u]), int(p.node_end[u]) + 1))
        u = int(p.node_parent[u])
    return np.sort(np.concatenate(parts))


def descendants_of(p: PackedTrie, j: int) -> np.ndarray:
    """Queries that see key j: the rest of j's node plus every token of every
    node below it (walking the child lists)."""
    v = int(p.node_id[j])
    if v < 0:
        return np.zeros(0, np.int64)
    parts = [np.arange(j, int(p.node_end[v]) + 1)]
    stack = list(p.nodes[v].children)
    while stack:
        u = stack.pop()
        parts.append(np.arange(int(p.node_start[u]), int(p.node_end[u]) + 1))
        stack.extend(p.nodes[u].children)
    return np.sort(np.concatenate(parts))


def position_ids(mask: np.ndarray) -> np.ndarray:
    """[TT] "打包数据的生成": a token's position id is the number of tokens it
    may attend to under the dense mask, minus one.  Pads (rows with no
    visible token) get 0.  int32 [L]."""
    cnt = mask.sum(axis=1, dtype=np.int64)
    return np.where(cnt > 0, cnt - 1, 0).astype(np.int32)


def tile_classes(mask: np.ndarray, block: int = BLOCK_SIZE) -> np.ndarray:
    """Classification of the block x block tiles of the dense mask, the
    granularity of [TT]'s block mask: 2 = every entry visible (full),
    0 = none visible (empty), 1 = otherwise (partial).  uint8 [nb, nb],
    indexed [query block, key block]."""
    L = mask.shape[0]
    if L % block:
        raise PackError("arg", "mask size must be a multiple of the block size")
    nb = L // block
    t = mask.reshape(nb, block, nb, block)
    full = t.all(axis=(1, 3))
    anyv = t.any(axis=(1, 3))
    return np.where(full, 2, np.where(anyv, 1, 0)).astype(np.uint8)


def accounting(tries: list[PackedTrie], masks: list[np.ndarray], seq_lens) -> dict:
    """[TT] "指标与监控": tree_token_ratio = tokens stored in all tries divided
    by the original token count (the attention-mask sum).  Also the number of
    visible (query, key) pairs under the tree masks, and under independent
    causal attention of every sequence unpacked."""
    tree_tokens = sum(p.n_tokens for p in tries)
    original = int(sum(int(x) for x in seq_lens))
    pairs = [int(m.sum(dtype=np.int64)) for m in masks]
    unpacked = int(sum(int(x) * (int(x) + 1) // 2 for x in seq_lens))
    return {
        "tree_tokens": tree_tokens,
        "original_tokens": original,
        "tree_token_ratio": tree_tokens / original,
        "n_pairs": sum(pairs),
        "n_pairs_per_trie": pairs,
        "unpacked_pairs": unpacked,
    }
