/*
 * tree_attn.h -- C ABI of the MI355X (gfx950) trie-packed tree-attention
 * library (libtreeattn.so).
 *
 * The problem (sources: the AReaL tree-training guide, "AReaL Tree Training
 * 完全指南" on 2kiu.com, sections 树构建流程 / 核心数据结构 / 打包数据的生成 /
 * 两种注意力实现; and the AREAL-DTA paper notes, §3 问题形式化):
 * rollout sequences that share prefixes are packed into compressed prefix
 * tries, flattened in pre-order, so each shared token is stored and computed
 * once.  Each token attends to itself and its ancestors only; its position
 * id is its ancestor count.  Gradients of a shared prefix are the sum over
 * every sequence through it.
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative TREE_E_* code; the message of the
 *     last failure on the calling thread is in tree_last_error().  No C++
 *     exception crosses this boundary.
 *   - Pointers named d_* and the tensors q/k/v/o/lse/dout/dq/dk/dv are DEVICE
 *     pointers owned by the caller.  The library never allocates device
 *     memory; it reports workspace sizes and the caller passes workspaces in.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is enqueued on it; no call synchronises.  Faults inside a
 *     kernel surface at the caller's next synchronisation of that stream.
 *   - Layouts: one packed trie of L tokens (L a multiple of 128) is a batch
 *     of one.  Q, O, dQ, dO are [L, Hq, D] contiguous; K, V, dK, dV are
 *     [L, Hkv, D]; LSE is [Hq, L] float32 (natural log).  dtype is
 *     TREE_DTYPE_BF16 (bf16 tensors, fp32 accumulation; D = 64 or 128) or
 *     TREE_DTYPE_FP32 (fp32 tensors, a slow check mode; D <= 128).  Query
 *     head h reads key/value head h / (Hq / Hkv).
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TREE_ATTN_ABI_VERSION 7

/* status codes */
#define TREE_OK 0
#define TREE_E_MAX_TOKENS (-1)   /* max_tokens_per_mb <= 0 */
#define TREE_E_ALIGN (-2)        /* max_tokens_per_mb not a multiple of block_size */
#define TREE_E_SEQ_TOO_LONG (-3) /* a sequence longer than max_tokens_per_mb */
#define TREE_E_EMPTY_SEQ (-4)    /* a row with no real token */
#define TREE_E_ARG (-5)          /* null pointer, bad size, dims, head ratio or dtype */
#define TREE_E_WORKSPACE (-6)    /* workspace smaller than the reported size */
#define TREE_E_HIP (-7)          /* a HIP launch or runtime call failed */
#define TREE_E_NOMEM (-8)        /* host allocation failed */

#define TREE_DTYPE_BF16 0
#define TREE_DTYPE_FP32 1

/* Block size of the tile grid and of the padding (the guide's BlockMask
 * block, section 两种注意力实现). */
#define TREE_BLOCK 128

/* Version of this ABI (TREE_ATTN_ABI_VERSION). */
int tree_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  The string
 * belongs to the library and stays valid until the thread's next call. */
const char* tree_last_error(void);

/* ------------------------------------------------------------------------
 * Host packer.  Guide, sections 参数背后的源码校验逻辑 (validation),
 * 树构建流程 steps 1-3 (extraction, first-fit-decreasing insertion, chain
 * compression) and 核心数据结构 / 打包数据的生成 (pre-order layout with
 * inclusive node ranges, position ids, tree_token_ratio).
 * ---------------------------------------------------------------------- */
typedef struct tree_pack tree_pack_t; /* opaque, owned by the library */

/* Read-only view of one packed trie.  Every pointer belongs to the
 * tree_pack_t it came from and stays valid until tree_pack_free(). */
typedef struct {
    int64_t n_tokens;            /* real (stored) tokens n                      */
    int64_t L;                   /* padded length, multiple of block_size       */
    int64_t n_nodes;             /* compressed nodes                            */
    int64_t n_seqs;              /* sequences in this trie                      */
    const int32_t* token_ids;    /* [L]  pads = pad_id                          */
    const int32_t* node_id;      /* [L]  pre-order node index, -1 for pads      */
    const int32_t* subtree_end;  /* [L]  inclusive last index of the token's
                                         node's subtree, -1 for pads            */
    const int32_t* node_start;   /* [n_nodes] first token index                 */
    const int32_t* node_end;     /* [n_nodes] last token index (inclusive)      */
    const int32_t* node_parent;  /* [n_nodes] parent node, -1 under the root    */
    const int32_t* seq_ids;      /* [n_seqs] batch rows, insertion order        */
    const int32_t* seq_iv_ptr;   /* [n_seqs+1] CSR offsets into seq_iv          */
    const int32_t* seq_iv;       /* [2*seq_iv_ptr[n_seqs]] (start,end) pairs:
                                    the nodes each sequence passes, root first  */
} tree_trie_view;

typedef struct {
    int64_t n_tries;
    int64_t original_tokens;     /* sum of the attention mask                   */
    int64_t tree_tokens;         /* sum of n_tokens over tries                  */
    double tree_token_ratio;     /* tree_tokens / original_tokens (guide,
                                    section 指标与监控)                          */
    int64_t n_pairs;             /* visible (query,key) pairs, all tries        */
    int64_t unpacked_pairs;      /* sum over sequences of l*(l+1)/2             */
    /* 128x128 tiles of the block mask (guide, section 两种注意力实现), summed
       over tries: full (every query of the tile sees every key), partial
       (some but not all), and the lower-triangular tile count of dense
       causal attention over each trie, nb (nb + 1) / 2 with nb = L / 128.
       The tile-skip rate against dense causal is
       1 - (tiles_full + tiles_partial) / tiles_causal. */
    int64_t tiles_full;
    int64_t tiles_partial;
    int64_t tiles_causal;
} tree_pack_stats_t;

/* Pack a padded batch.  ids [B,S] int32 and mask [B,S] uint8 are HOST
 * row-major arrays; row r's sequence is ids[r][c] for every c with
 * mask[r][c] != 0, in column order.  Sequences are sorted by length,
 * longest first (ties keep row order), and each goes into the first trie
 * (in creation order) whose uncompressed token count plus what it adds
 * stays <= max_tokens_per_mb; otherwise a new trie is opened.  Single-child
 * chains carrying the same sequences are merged; nodes are laid out in
 * pre-order with children in insertion order; each trie is padded to
 * round_up(n, block_size), or to max_tokens_per_mb if pad_to_maximum != 0,
 * with pad_id.  block_size must be 128.  On success *out owns the result
 * (free with tree_pack_free).  Errors: TREE_E_MAX_TOKENS, TREE_E_ALIGN,
 * TREE_E_EMPTY_SEQ, TREE_E_SEQ_TOO_LONG (rows checked in order, empty
 * before too long), TREE_E_ARG, TREE_E_NOMEM; *out is then NULL. */
int tree_pack(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S,
              int64_t max_tokens_per_mb, int32_t block_size, int32_t pad_to_maximum,
              int32_t pad_id, tree_pack_t** out);

/* How tree_pack_ordered assigns sequences to tries. */
#define TREE_PACK_FFD 0    /* first-fit decreasing, as tree_pack */
#define TREE_PACK_PREFIX 1 /* prefix order, see below */

/* tree_pack with a choice of assignment.  TREE_PACK_FFD is tree_pack.
 * TREE_PACK_PREFIX takes the sequences in lexicographic order (token ids
 * compared as integers, a proper prefix first, ties by row): the DFS order
 * of one tree over the whole batch that AREAL-DTA's load-balancing section
 * (负载均衡并行化) partitions.  Each sequence goes into the most recently
 * opened trie if its uncompressed token count plus what the sequence adds
 * stays <= max_tokens_per_mb, otherwise it opens a new trie, so every trie
 * is a contiguous run of that order and keeps a prompt's responses
 * together where first-fit by length spreads them.  Sequences are inserted
 * in that order.  Arguments, layout, ownership and errors are those of
 * tree_pack, plus TREE_E_ARG for an unknown order. */
int tree_pack_ordered(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S,
                      int64_t max_tokens_per_mb, int32_t block_size, int32_t pad_to_maximum,
                      int32_t pad_id, int32_t order, tree_pack_t** out);

/* Number of tries, or -1 if p is NULL. */
int64_t tree_pack_num_tries(const tree_pack_t* p);

/* Fill *v with a view of trie t (0 <= t < num_tries); TREE_E_ARG otherwise. */
int tree_pack_trie(const tree_pack_t* p, int64_t t, tree_trie_view* v);

/* Accounting of the whole pack (guide, section 指标与监控). */
int tree_pack_stats(const tree_pack_t* p, tree_pack_stats_t* s);

/* All tries of a pack laid end to end, for one launch over the whole batch.
 * No attention crosses tries (a subtree never leaves its trie), so the
 * concatenation is itself a valid packed layout: trie t occupies
 * [off_t, off_t + L_t) with off_t the sum of the earlier L, its subtree
 * ends are shifted by off_t and pads stay -1; position ids, tile classes
 * and every attention result restricted to trie t's rows are those of trie
 * t alone, and tiles across tries classify as empty.  Writes the total
 * length to *L_total; when out_se is non-NULL it receives the *L_total
 * concatenated subtree ends and cap (its capacity in int32) must be at
 * least that.  Errors: TREE_E_ARG (NULL pack or L_total, cap too small). */
int tree_pack_concat(const tree_pack_t* p, int32_t* out_se, int64_t cap, int64_t* L_total);

/* Token ids of all tries in the concatenated layout of tree_pack_concat
 * (pads carry the pack's pad id), into out_ids[cap].  Errors: TREE_E_ARG
 * (NULL argument, cap smaller than the total length). */
int tree_pack_concat_ids(const tree_pack_t* p, int32_t* out_ids, int64_t cap);

/* Where each sequence sits in the concatenated layout (guide, section
 * "Log Probability 计算": a sequence's own token order is recovered from
 * the trie, root to leaf, as the pages' get_sequence_tree_indices does).
 * out[r * S + k] = packed position of the k-th real token of batch row r
 * (B, S: the batch shape the pack was built from), -1 for k >= the row's
 * length.  cap is out's capacity in int32 and must be >= B * S.  Errors:
 * TREE_E_ARG (NULL argument, cap too small). */
int tree_pack_row_positions(const tree_pack_t* p, int32_t* out, int64_t cap);

/* Load-balanced split of a batch over K data-parallel workers (AREAL-DTA
 * notes, §4 负载均衡并行化): the rows' real-token sequences are taken in
 * lexicographic order (the DFS order of one prefix tree over all of them;
 * a proper prefix first, equal sequences by row), and cut into at most K
 * contiguous runs minimising the largest run cost C(T) = tokens of the
 * run's prefix tree.  The optimum tau is found by binary search between the
 * longest sequence and the whole tree, each candidate checked by a greedy
 * scan that starts a new run when the next sequence would exceed it; the
 * result is that greedy scan at tau, so runs fill from the left and the
 * last ones may be empty.  Outputs (host memory, caller-owned):
 * out_group[B] = run of each row; *out_max_cost = tau (if non-NULL);
 * out_costs[K] = each run's tree tokens (if non-NULL).  Each worker then
 * packs its rows with tree_pack; workers with fewer tries pad to the
 * maximum count with empty ones (the guide's DP tree-count sync, 打包数据
 * 的生成).  Rows may be empty here.  Errors: TREE_E_ARG (K <= 0, bad shape,
 * NULL input), TREE_E_NOMEM. */
int tree_partition(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S, int32_t K, int32_t* out_group,
                   int64_t* out_max_cost, int64_t* out_costs);

/* Release a pack (NULL is a no-op). */
void tree_pack_free(tree_pack_t* p);

/* ------------------------------------------------------------------------
 * Metadata (device).  Guide, section 打包数据的生成: a token's position id is
 * the number of tokens it may attend to, minus one; the block mask of
 * section 两种注意力实现 is built here as a per-128x128-tile class computed
 * from subtree intervals: key j is visible to query i iff j <= i <= se[j].
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace tree_meta needs for a trie of length L. */
size_t tree_meta_workspace_bytes(int64_t L);

/* From d_se[L] (the trie's subtree_end, copied to the device; real tokens
 * first, pads -1 after them) compute:
 *   d_pos[L]          int32 position ids, pads 0;
 *   d_tile_class[nb*nb] uint8, nb = L/128, row-major [query block][key
 *                     block]: 0 empty, 1 partial, 2 full;
 *   d_ws              the attention kernels' tile lists (row- and
 *                     column-wise nonempty tiles, heaviest-first orders).
 * d_ws must hold tree_meta_workspace_bytes(L) bytes and stay untouched
 * until the attention calls that use it have run.  L % 128 != 0 or
 * L > 2^20 gives TREE_E_ARG. */
int tree_meta(const int32_t* d_se, int64_t L, int32_t* d_pos, uint8_t* d_tile_class,
              void* d_ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Attention (device).  scale must be finite and > 0.  Forward: for query
 * head h and token i,
 *   O_i = softmax_j(scale * q_i . k_j) v_j over j in A(i) = {j : j <= i <= se[j]},
 *   LSE_i = ln sum_{j in A(i)} exp(scale * q_i . k_j);
 * rows with no visible key (pads) get O = 0 and LSE = -inf.  Tiles the
 * metadata marks empty are skipped.  d_se and d_meta_ws are the inputs and
 * the workspace of the tree_meta call for this trie.
 * ---------------------------------------------------------------------- */
int tree_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* d_se, const void* d_meta_ws, int64_t L, int32_t Hq,
                  int32_t Hkv, int32_t D, float scale, int32_t dtype, void* stream);

/* Bytes of device workspace tree_attn_bwd needs: two float rows per query
 * head and token (Delta_i and, for bf16, LSE_i / scale), 2 * L * Hq * 4
 * rounded up to 256.  Returns 0 for L <= 0 or Hq <= 0. */
size_t tree_attn_bwd_workspace_bytes(int64_t L, int32_t Hq, int32_t D, int32_t dtype);

/* Backward of tree_attn_fwd (AREAL-DTA notes, §3 问题形式化: a shared
 * prefix's gradient is accumulated over every sequence through it, which
 * holds here because a shared token is one row of the packed problem).
 * Inputs q, k, v, o, lse (from tree_attn_fwd) and dout; outputs dq [L,Hq,D],
 * dk, dv [L,Hkv,D] in the tensor dtype, fully overwritten (pads get 0).
 * dk/dv of a key/value head sum over its query heads.  d_ws must hold
 * tree_attn_bwd_workspace_bytes() bytes. */
int tree_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  const int32_t* d_se, const void* d_meta_ws, void* d_ws, size_t ws_bytes,
                  int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                  int32_t dtype, void* stream);

/* One phase of tree_attn_bwd, for callers that time or schedule the
 * backward's kernels separately: TREE_BWD_DELTA computes Delta_i =
 * dO_i . O_i (and, for bf16, LSE_i / scale) into d_ws, in an internal
 * layout; TREE_BWD_DKDV writes dk and dv; TREE_BWD_DQ writes dq;
 * TREE_BWD_DQ_DELTA writes dq and leaves in d_ws what a DELTA phase would
 * (for bf16 the dQ kernel computes Delta itself from o and dout; in the
 * fp32 check mode it is the DELTA then the DQ phase).  DKDV and DQ read what
 * a DELTA or DQ_DELTA phase left in the same d_ws, so one of those must
 * precede them on the stream.  TREE_BWD_ALL (same as tree_attn_bwd) runs
 * DQ_DELTA then DKDV for bf16, and DELTA, DKDV, DQ for fp32.  Other arguments
 * and errors as tree_attn_bwd; an unknown phase gives TREE_E_ARG. */
#define TREE_BWD_ALL 0
#define TREE_BWD_DELTA 1
#define TREE_BWD_DKDV 2
#define TREE_BWD_DQ 3
#define TREE_BWD_DQ_DELTA 4
int tree_attn_bwd_phase(int32_t phase, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const int32_t* d_se, const void* d_meta_ws, void* d_ws, size_t ws_bytes,
                        int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                        int32_t dtype, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the
 * backward of tree_attn_bwd (same kernels, same results bit for bit) with its
 * workspace taken from a static array the library owns on each device,
 * TREE_BWD_STATIC_SCRATCH_BYTES long, instead of d_ws.  The array is set up
 * on the first call on a device (the device current on the calling thread,
 * which the stream must belong to) and held until the process ends.  No
 * device memory is allocated or freed.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, threads or
 * graph replays) race and must be serialised by the caller.  Limit:
 * tree_attn_bwd_workspace_bytes(L, Hq, D, dtype) <= TREE_BWD_STATIC_SCRATCH_BYTES,
 * i.e. L * Hq <= 8388608 (L = 262144 at 32 query heads); a larger call fails
 * with TREE_E_ARG before any device work.  Other arguments and errors as
 * tree_attn_bwd (TREE_E_HIP if the array's address cannot be looked up). */
#define TREE_BWD_STATIC_SCRATCH_BYTES (64u << 20)
int tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, const int32_t* d_se,
                          const void* d_meta_ws, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                          int32_t dtype, void* stream);

/* ------------------------------------------------------------------------
 * Depth-first execution (AREAL-DTA notes, §3.1 前缀树的深度优先搜索遍历 and
 * §3.2 系统优化).  The same attention and gradients as tree_attn_fwd +
 * tree_attn_bwd on one trie, computed the way the notes' DFS traversal does:
 * a stack holds the keys/values of the current root-to-node path; entering
 * an internal node pushes its tokens and runs their forward against the
 * stack; leaves run forward and backward at once and are never pushed ("cut
 * tail": no later token attends to them); leaving a node runs its backward,
 * after every sequence below it has added its gradient to the node's keys,
 * and pops it.  Internal nodes and leaves longer than `chunk` tokens run in
 * chunks of at most `chunk` queries.  Device memory (the frame) is bounded by
 * the longest path, not the tree.  Consecutive sibling leaves of at most
 * `chunk` tokens run together in one launch, up to the frame's leaf rows
 * (4 * chunk or the longest leaf, whichever is more): the same computation
 * as visiting them one by one.  bf16 only.
 * ---------------------------------------------------------------------- */
typedef struct {
    int64_t rows;              /* frame length the kernels run on (multiple of 256) */
    int64_t stack_rows;        /* most frame rows the stack occupies (each node from a
                                  128-aligned row) */
    int64_t leaf_rows;         /* most rows one launch of leaves may take: 4 * chunk, or
                                  the longest leaf if longer */
    int64_t peak_stack_tokens; /* most real tokens on the stack at once: the longest
                                  root-to-internal-node path */
    int64_t max_path_tokens;   /* longest root-to-leaf path */
    int64_t chunks;            /* query launches (one forward and one backward each) */
    int64_t leaf_groups;       /* launches of consecutive sibling leaves */
    int64_t max_depth;         /* most internal nodes on the stack */
} tree_dfs_plan_t;

/* Plan of the depth-first execution of one trie, from its HOST node table
 * (tree_trie_view's node_start / node_end / node_parent, n_nodes, and its
 * n_tokens).  chunk must be a positive multiple of 128 (2048 in the notes).
 * Errors: TREE_E_ARG (NULL pointers, a node table that is not the pre-order
 * layout, a stack deeper than 240 internal nodes, a frame longer than
 * 2^20 rows), TREE_E_NOMEM. */
int tree_dfs_plan(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent, int64_t n_nodes,
                  int64_t n_tokens, int32_t chunk, tree_dfs_plan_t* plan);

/* Bytes of device workspace tree_attn_dfs needs for a plan (0 if invalid). */
size_t tree_attn_dfs_workspace_bytes(const tree_dfs_plan_t* plan, int32_t Hq, int32_t Hkv, int32_t D);

/* Forward and backward of one trie by depth-first execution.  The node table
 * is on the HOST (as for tree_dfs_plan); q, k, v, dout, o, lse, dq, dk, dv
 * are DEVICE tensors in the packed layout of tree_attn_fwd / tree_attn_bwd
 * (L rows, bf16, LSE [Hq, L] float32), d_se the trie's subtree ends on the
 * device.  All outputs are fully overwritten (pads: O = dQ = dK = dV = 0,
 * LSE = -inf).  d_ws holds tree_attn_dfs_workspace_bytes(plan) bytes.  The
 * host walks the trie and enqueues many small launches on `stream`; nothing
 * synchronises.  Errors: those of tree_dfs_plan and tree_attn_bwd. */
int tree_attn_dfs(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent, int64_t n_nodes,
                  int64_t n_tokens, const void* q, const void* k, const void* v, const void* dout, void* o,
                  float* lse, void* dq, void* dk, void* dv, const int32_t* d_se, void* d_ws, size_t ws_bytes,
                  int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t chunk, void* stream);

/* ------------------------------------------------------------------------
 * Log-probabilities and entropies of packed logits (device).  Guide,
 * section "Log Probability 计算：树结构的特殊处理": labels cannot come from
 * rolling the packed ids; each sequence's token k + 1 is predicted by the
 * logits at the packed position of its token k (inside a node the next
 * position, at a node's end the row every child's first token reads), and
 * shared prefixes are computed once.  Here the row statistics are computed
 * once per packed row and the per-sequence values are gathered, then laid
 * out per batch row (the pages' merge_packed_tree_results).
 * ---------------------------------------------------------------------- */

/* Per packed row p of logits [L, V] (row-major, dtype TREE_DTYPE_BF16 or
 * TREE_DTYPE_FP32, aligned to its element size; V any size >= 1):
 *   d_lse[p] = ln sum_v exp(logits[p, v]),
 *   d_ent[p] = -sum_v P_v ln P_v with P = softmax(logits[p, :]), 0 ln 0 = 0,
 * both float32 [L], accumulated in float32 in one pass over the row.  A row
 * of -inf gives lse -inf and entropy 0.  L = 0 is a no-op.  Errors:
 * TREE_E_ARG (NULL pointer, bad shape or dtype, misaligned logits),
 * TREE_E_HIP (launch). */
int tree_logits_stats(const void* logits, int64_t L, int64_t V, int32_t dtype, float* d_lse, float* d_ent,
                      void* stream);

/* The gather, for a batch of B rows of width S: with pos = d_row_pos (from
 * tree_pack_row_positions, on the device) and ids = the packed token ids
 * [L] (tree_pack_concat_ids),
 *   d_logp[r, j] = logits[pos[r, j], ids[pos[r, j + 1]]] - d_lse[pos[r, j]],
 *   d_out_ent[r, j] = d_ent[pos[r, j]]
 * for j < (row r's length) - 1, i.e. row r's j-th prediction is that of its
 * token j + 1; every other entry is pad_value.  d_lse / d_ent come from
 * tree_logits_stats on the same logits.  Outputs are float32 [B, S],
 * fully overwritten.  A position outside [0, L) or a token id outside
 * [0, V) yields NaN for that entry (never an access out of range).  B * S
 * = 0 is a no-op.  Errors: TREE_E_ARG (NULL pointer, bad shape or dtype),
 * TREE_E_HIP (launch). */
int tree_gather_logprobs(const void* logits, int64_t L, int64_t V, int32_t dtype, const float* d_lse,
                         const float* d_ent, const int32_t* d_ids, const int32_t* d_row_pos, int64_t B,
                         int64_t S, float pad_value, float* d_logp, float* d_out_ent, void* stream);

/* The same gather over a window of rows, for logits produced chunk by chunk
 * (the guide's chunk_size, 1024 rows by default, bounds peak memory the
 * same way): logits_rows holds packed rows [row0, row0 + n_rows) of the
 * [L, V] logits, row-major.  Entries predicted from a row in the window are
 * written as tree_gather_logprobs writes them; entries predicted from a row
 * outside it are left unchanged; pad entries (pad_value) and entries with
 * a position outside [0, L) (NaN) are written by every call.  So calls whose
 * windows cover [0, L) exactly once, in any order, leave d_logp /
 * d_out_ent equal to one tree_gather_logprobs over the whole logits.  d_lse
 * / d_ent are the whole [L] arrays (tree_logits_stats of each chunk written
 * at d_lse + row0, d_ent + row0).  Errors: those of tree_gather_logprobs,
 * and TREE_E_ARG for a window outside [0, L). */
int tree_gather_logprobs_rows(const void* logits_rows, int64_t row0, int64_t n_rows, int64_t L, int64_t V,
                              int32_t dtype, const float* d_lse, const float* d_ent, const int32_t* d_ids,
                              const int32_t* d_row_pos, int64_t B, int64_t S, float pad_value, float* d_logp,
                              float* d_out_ent, void* stream);

/* ------------------------------------------------------------------------
 * Rotary position embedding by tree position ids (device).  Guide, section
 * 打包数据的生成: position ids are ancestor counts minus one (tree_meta's
 * d_pos), so a shared prefix carries the same positional encoding in every
 * sequence through it; they feed the model's rotary embedding.  The pages do
 * not spell the rotation out; this is the half-split form of the Qwen/Llama
 * models they train: for head vectors x [L, H, D] (D even), position
 * p = d_pos[i], f_j = base^(-2j/D), a_j = p f_j,
 *   y[i,h,j]       = x[i,h,j] cos a_j - x[i,h,j+D/2] sin a_j,
 *   y[i,h,j+D/2]   = x[i,h,j+D/2] cos a_j + x[i,h,j] sin a_j,
 * j < D/2; with inverse != 0 the rotation is by -a_j, which is also the
 * gradient map (dx = inverse rotation of dy).  Angles, sines and cosines are
 * formed in float64, the rotation in float32; dtype TREE_DTYPE_BF16 or
 * TREE_DTYPE_FP32 for both x and y.  y may equal x (in place).  L = 0 is a
 * no-op.  Errors: TREE_E_ARG (NULL pointer, odd or bad D, H, L, base <= 1
 * or not finite, dtype, misalignment), TREE_E_HIP. */
int tree_rope(const void* x, void* y, const int32_t* d_pos, int64_t L, int32_t H, int32_t D, double base,
              int32_t inverse, int32_t dtype, void* stream);

/* The same rotary embedding fused into the attention kernels (bf16): Q is
 * rotated as the forward kernel loads it into registers, K by a table-driven
 * pass into k_rot, and the backward rotates dQ and dK back in its epilogues,
 * so its outputs are gradients with respect to the unrotated q and k.
 *
 * tree_rope_table fills d_tab with (cos, sin) float pairs of p f_j for every
 * position p < P and pair j < D/2 -- float64 angles rounded to float32, the
 * values tree_rope uses -- [P, D/2, 2] float32, tree_rope_table_bytes(P, D)
 * bytes (0 for a bad P or D; D a multiple of 16).  The attention calls need a
 * table with P >= L (every position id is below L).  Errors: TREE_E_ARG,
 * TREE_E_WORKSPACE (table too small), TREE_E_HIP. */
size_t tree_rope_table_bytes(int64_t P, int32_t D);
int tree_rope_table(double base, int64_t P, int32_t D, float* d_tab, size_t tab_bytes, void* stream);

/* tree_attn_fwd on rotated q and k: O = attention(rot(q), rot(k), v), with
 * rot by the position ids d_pos (tree_meta's) and the table d_tab.  Also
 * writes q_rot = rot(q) [L, Hq, D] and k_rot = rot(k) [L, Hkv, D] (bf16), the
 * operands tree_attn_bwd_rope needs.  Other arguments and errors as
 * tree_attn_fwd. */
int tree_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* q_rot, void* k_rot,
                       const int32_t* d_pos, const float* d_tab, size_t tab_bytes, const int32_t* d_se,
                       const void* d_meta_ws, int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                       void* stream);

/* Backward of tree_attn_fwd_rope from its q_rot, k_rot, o, lse: dq and dk
 * are the gradients with respect to the unrotated q and k (the rotation is
 * orthogonal, so each is the inverse rotation of the gradient with respect
 * to its rotated operand, applied before the bf16 rounding), dv as
 * tree_attn_bwd.  Other arguments and errors as tree_attn_bwd. */
int tree_attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, const int32_t* d_pos, const float* d_tab,
                       size_t tab_bytes, const int32_t* d_se, const void* d_meta_ws, void* d_ws, size_t ws_bytes,
                       int64_t L, int32_t Hq, int32_t Hkv, int32_t D, float scale, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TREE_ATTN_H */
