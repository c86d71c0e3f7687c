// Depth-first (DTA) execution of tree attention over one packed trie.
//
// AREAL-DTA notes, §3.1 (前缀树的深度优先搜索遍历) and §3.2 (系统优化): the trie
// is walked depth first while a stack holds the keys/values of the current
// root-to-node path.  Entering an internal node pushes its tokens and runs
// their forward against the stack; a leaf runs forward and backward at once
// and is never pushed (its keys serve no later token); leaving a node runs
// its backward -- every descendant's gradient having been accumulated into its
// keys meanwhile -- and pops it.  Internal nodes and leaves longer than
// `chunk` run in chunks of at most `chunk` query tokens.
//
// On the GPU the stack is a "frame": a layout of Lc rows holding the path's
// node segments (each from a 128-aligned row, in path order) and, above them,
// the leaves being run.  The frame is itself a packed trie (every stack key is
// an ancestor of every later token; the leaves are its branches), so the tree
// kernels run on it unchanged, restricted to the query blocks of one node or
// chunk (fwd / dQ over a block list, dK/dV clipped to that block range and
// accumulating into float32 per-row accumulators that live as long as the
// row is on the stack).  Consecutive sibling leaves run together, up to the
// frame's leaf capacity, so a launch has enough work for the chip; that is
// the same computation as visiting them one by one (they share the stack and
// touch disjoint rows); the leaf rows hold four chunks' worth, so that a leaf
// launch's dK/dV grid has enough key-block pairs.  Memory is bounded by the
// longest path, not the tree.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "device.h"
#include "status.h"

namespace treeattn {
namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Tree {
    const int32_t *start, *end, *parent;
    int64_t n_nodes, n_tokens;
    std::vector<std::vector<int>> kids;
    std::vector<int> roots;
    int64_t size(int v) const { return int64_t(end[v]) - start[v] + 1; }
    bool leaf(int v) const { return kids[size_t(v)].empty(); }
};

int build_tree(const int32_t* s, const int32_t* e, const int32_t* par, int64_t n_nodes, int64_t n_tokens, Tree& t) {
    if (n_nodes <= 0 || n_tokens <= 0 || !s || !e || !par)
        return set_error(TREE_E_ARG, "tree_attn_dfs: empty or NULL node table");
    t.start = s;
    t.end = e;
    t.parent = par;
    t.n_nodes = n_nodes;
    t.n_tokens = n_tokens;
    t.kids.assign(size_t(n_nodes), {});
    t.roots.clear();
    // pre-order node table: contiguous token ranges in node order, and each
    // node's parent on the root path of the node before it (the path is kept
    // as a stack while scanning), so that the parent links describe the tree
    // the layout was written from
    std::vector<int64_t> path;
    for (int64_t v = 0; v < n_nodes; ++v) {
        const int64_t lo = s[v], hi = e[v];
        if (lo != (v == 0 ? 0 : int64_t(e[v - 1]) + 1) || hi < lo || hi >= n_tokens)
            return set_error(TREE_E_ARG, "tree_attn_dfs: node %lld range [%lld, %lld] is not the pre-order layout",
                             (long long)v, (long long)lo, (long long)hi);
        const int64_t p = par[v];
        while (!path.empty() && path.back() != p) path.pop_back();
        if (p >= v || p < -1 || (p >= 0 && path.empty()))
            return set_error(TREE_E_ARG, "tree_attn_dfs: node %lld has parent %lld, not on the pre-order path",
                             (long long)v, (long long)p);
        path.push_back(v);
        (p < 0 ? t.roots : t.kids[size_t(p)]).push_back(int(v));
    }
    if (int64_t(e[n_nodes - 1]) + 1 != n_tokens)
        return set_error(TREE_E_ARG, "tree_attn_dfs: nodes cover %lld tokens, not %lld",
                         (long long)(int64_t(e[n_nodes - 1]) + 1), (long long)n_tokens);
    return TREE_OK;
}

// One walk serves both the plan (sizes only) and the execution.
struct Walk {
    const Tree& t;
    int64_t chunk, leaf_cap;
    struct Seg {
        int node;
        int64_t row0;
    };
    std::vector<Seg> path;
    int64_t top = 0, stack_tokens = 0;
    // plan
    int64_t rows_needed = 0, stack_rows = 0, peak_stack = 0, max_path = 0, chunks = 0, groups = 0;
    int depth_max = 0;

    Walk(const Tree& tr, int64_t ch, int64_t cap) : t(tr), chunk(ch), leaf_cap(cap) {}

    template <class Ex>
    int run(Ex& ex) {
        return siblings(ex, t.roots);
    }

    // Process a sibling list: consecutive leaves in groups, internal nodes
    // depth first (recursion depth = path depth, at most kDfsMaxSegments).
    template <class Ex>
    int siblings(Ex& ex, const std::vector<int>& list) {
        size_t i = 0;
        while (i < list.size()) {
            const int v = list[i];
            if (t.leaf(v)) {
                // a leaf longer than the chunk runs alone, in chunks; shorter
                // consecutive sibling leaves run together in one launch, up to
                // the frame's leaf rows
                size_t j = i + 1;
                int64_t G = t.size(v);
                const bool long_leaf = G > chunk;
                if (!long_leaf)
                    while (j < list.size() && t.leaf(list[j]) && t.size(list[j]) <= chunk &&
                           G + t.size(list[j]) <= leaf_cap)
                        G += t.size(list[j++]);
                for (size_t k = i; k < j; ++k) max_path = std::max(max_path, stack_tokens + t.size(list[k]));
                rows_needed = std::max(rows_needed, top + round_up(G, kBlock));
                const int64_t launch_rows = long_leaf ? chunk : round_up(G, kBlock);
                chunks += (G + launch_rows - 1) / launch_rows;
                ++groups;
                if (int rc = ex.group(*this, t.start[v], G, launch_rows)) return rc;
                i = j;
                continue;
            }
            if (int(path.size()) >= kDfsMaxSegments)
                return set_error(TREE_E_ARG, "tree_attn_dfs: the trie is deeper than %d internal nodes",
                                 kDfsMaxSegments);
            const int64_t n = t.size(v), row0 = top;
            path.push_back({v, row0});
            top += round_up(n, kBlock);
            stack_tokens += n;
            depth_max = std::max(depth_max, int(path.size()));
            peak_stack = std::max(peak_stack, stack_tokens);
            max_path = std::max(max_path, stack_tokens);
            stack_rows = std::max(stack_rows, top);
            rows_needed = std::max(rows_needed, top);
            chunks += (n + chunk - 1) / chunk;
            if (int rc = ex.push(*this, v, row0)) return rc;
            if (int rc = siblings(ex, t.kids[size_t(v)])) return rc;
            if (int rc = ex.pop(*this, v, row0)) return rc;
            path.pop_back();
            top = row0;
            stack_tokens -= n;
            ++i;
        }
        return TREE_OK;
    }
};

struct NoExec {
    int group(Walk&, int64_t, int64_t, int64_t) { return TREE_OK; }
    int push(Walk&, int, int64_t) { return TREE_OK; }
    int pop(Walk&, int, int64_t) { return TREE_OK; }
};

int plan_of(const Tree& t, int32_t chunk, tree_dfs_plan_t* out) {
    if (chunk < kBlock || chunk % kBlock != 0)
        return set_error(TREE_E_ARG, "tree_attn_dfs: chunk %d must be a positive multiple of %d", chunk, kBlock);
    int64_t longest_leaf = 0;
    for (int64_t v = 0; v < t.n_nodes; ++v)
        if (t.leaf(int(v))) longest_leaf = std::max(longest_leaf, t.size(int(v)));
    // leaf rows: four chunks of short leaves per launch (enough key-block
    // pairs for the dK/dV grid to fill the chip), or the longest leaf
    const int64_t cap = round_up(std::max<int64_t>(4 * int64_t(chunk), longest_leaf), kBlock);
    Walk w(t, chunk, cap);
    NoExec none;
    if (int rc = w.run(none)) return rc;
    const int64_t rows = round_up(std::max<int64_t>(w.rows_needed, 2 * kBlock), 2 * kBlock);
    if (rows > kMaxL)
        return set_error(TREE_E_ARG, "tree_attn_dfs: a frame of %lld rows exceeds %lld", (long long)rows,
                         (long long)kMaxL);
    out->rows = rows;
    out->stack_rows = w.stack_rows;
    out->leaf_rows = cap;
    out->peak_stack_tokens = w.peak_stack;
    out->max_path_tokens = w.max_path;
    out->chunks = w.chunks;
    out->leaf_groups = w.groups;
    out->max_depth = w.depth_max;
    return TREE_OK;
}

// Workspace of a frame of `rows` rows, in 256-byte aligned pieces.
struct FrameBufs {
    char *q, *dO, *o, *dq, *k, *v;
    float *acck, *accv, *lse, *bws;
    int32_t *se, *pos, *iota;
    uint8_t* tc;
    void* meta;
    size_t bytes;
};

FrameBufs frame_layout(char* base, int64_t rows, int Hq, int Hkv, int D) {
    FrameBufs f{};
    size_t off = 0;
    auto take = [&](size_t b) {
        char* p = base ? base + off : nullptr;
        off += (b + 255) / 256 * 256;
        return p;
    };
    const size_t qb = size_t(rows) * Hq * D * 2, kb = size_t(rows) * Hkv * D * 2;
    const int64_t nb = rows / kBlock;
    f.q = take(qb);
    f.dO = take(qb);
    f.o = take(qb);
    f.dq = take(qb);
    f.k = take(kb);
    f.v = take(kb);
    f.acck = reinterpret_cast<float*>(take(2 * kb));
    f.accv = reinterpret_cast<float*>(take(2 * kb));
    f.lse = reinterpret_cast<float*>(take(size_t(rows) * Hq * 4));
    f.bws = reinterpret_cast<float*>(take(tree_attn_bwd_workspace_bytes(rows, Hq, D, TREE_DTYPE_BF16)));
    f.se = reinterpret_cast<int32_t*>(take(size_t(rows) * 4));
    f.pos = reinterpret_cast<int32_t*>(take(size_t(rows) * 4));
    f.iota = reinterpret_cast<int32_t*>(take(size_t(nb) * 4));
    f.tc = reinterpret_cast<uint8_t*>(take(size_t(nb) * size_t(nb)));
    f.meta = take(tree_meta_workspace_bytes(rows));
    f.bytes = off;
    return f;
}

// Enqueues the device work of the walk on one stream.
struct Exec {
    const Tree& t;
    const char *q, *k, *v, *dO;  // packed inputs
    char *o, *dq, *dk, *dv;      // packed outputs
    float* lse;
    const int32_t* d_se;
    int64_t L, rows;
    int Hq, Hkv, D;
    float scale;
    int64_t chunk;
    FrameBufs f;
    hipStream_t s;
    int64_t qrow, krow;  // row bytes of Q-like and K-like tensors

    int st(hipError_t e) {
        if (e != hipSuccess) return set_error(TREE_E_HIP, "tree_attn_dfs: HIP error %d (%s)", int(e),
                                              hipGetErrorString(e));
        return TREE_OK;
    }
    AttnShape shape() const { return AttnShape{rows, int(rows / kBlock), Hq, Hkv, D, scale}; }

    // subtree ends and tile lists of the current frame
    int frame(Walk& w, int64_t last_real, int64_t leaf_row0, int64_t leaf_len, int64_t leaf_p0) {
        DfsSegments a{};
        a.n = int(w.path.size());
        a.top_se = int(last_real);
        a.leaf_row0 = int(leaf_row0);
        a.leaf_len = int(leaf_len);
        a.leaf_p0 = int(leaf_p0);
        for (int i = 0; i < a.n; ++i) {
            a.row0[i] = int(w.path[size_t(i)].row0);
            a.len[i] = int(t.size(w.path[size_t(i)].node));
        }
        if (int rc = st(launch_dfs_se(f.se, rows, d_se, a, s))) return rc;
        return st(launch_meta(f.se, rows, f.pos, f.tc, f.meta, s));
    }

    // frame rows [r0, r0 + n) in launches of at most `per` rows (a multiple
    // of 128): forward, and/or backward
    int chunks(int64_t r0, int64_t n, int64_t last_real, bool fwd, bool bwd, int64_t per) {
        const AttnShape sh = shape();
        const MetaPtrs mp = meta_ptrs(f.meta, rows);
        for (int64_t c = r0; c < r0 + n; c += per) {
            const int64_t c1 = std::min(r0 + n, c + per);
            RowSel sel;
            sel.q_list = f.iota + c / kBlock;
            sel.n_q = int((c1 + kBlock - 1) / kBlock - c / kBlock);
            sel.qb_lo = int(c / kBlock);
            sel.qb_hi = int((c1 + kBlock - 1) / kBlock);
            sel.n_wg = int(dkdv_workgroups((last_real + 1 + kChunk - 1) / kChunk));
            sel.dk_acc = f.acck;
            sel.dv_acc = f.accv;
            if (fwd)
                if (int rc = st(launch_fwd_bf16(f.q, f.k, f.v, f.o, f.lse, f.se, mp, sh, s, sel))) return rc;
            if (bwd) {
                if (int rc = st(launch_bwd_bf16(kPhaseDqDelta, f.q, f.k, f.v, f.o, f.lse, f.dO, f.dq, nullptr, nullptr,
                                                f.se, mp, f.bws, sh, s, sel)))
                    return rc;
                if (int rc = st(launch_bwd_bf16(kPhaseDkdv, f.q, f.k, f.v, f.o, f.lse, f.dO, f.dq, nullptr, nullptr,
                                                f.se, mp, f.bws, sh, s, sel)))
                    return rc;
            }
        }
        return TREE_OK;
    }

    // packed rows [p0, p0 + n) -> frame rows from r0 (inputs), and clear the
    // rows' accumulators up to the next block boundary
    int load(int64_t p0, int64_t r0, int64_t n) {
        if (int rc = st(launch_dfs_copy_rows(q, f.q, p0, r0, n, qrow, s))) return rc;
        if (int rc = st(launch_dfs_copy_rows(dO, f.dO, p0, r0, n, qrow, s))) return rc;
        if (int rc = st(launch_dfs_copy_rows(k, f.k, p0, r0, n, krow, s))) return rc;
        if (int rc = st(launch_dfs_copy_rows(v, f.v, p0, r0, n, krow, s))) return rc;
        const int64_t nr = round_up(n, kBlock);
        if (int rc = st(launch_dfs_fill(reinterpret_cast<char*>(f.acck) + r0 * 2 * krow, nr * 2 * krow, 0u, s)))
            return rc;
        return st(launch_dfs_fill(reinterpret_cast<char*>(f.accv) + r0 * 2 * krow, nr * 2 * krow, 0u, s));
    }
    int store_fwd(int64_t r0, int64_t p0, int64_t n) {
        if (int rc = st(launch_dfs_copy_rows(f.o, o, r0, p0, n, qrow, s))) return rc;
        return st(launch_dfs_copy_cols(f.lse, lse, rows, L, r0, p0, n, Hq, s));
    }
    int store_bwd(int64_t r0, int64_t p0, int64_t n) {
        if (int rc = st(launch_dfs_copy_rows(f.dq, dq, r0, p0, n, qrow, s))) return rc;
        const int64_t w = int64_t(Hkv) * D;
        if (int rc = st(launch_dfs_emit(f.acck, dk, r0, p0, n, w, s))) return rc;
        return st(launch_dfs_emit(f.accv, dv, r0, p0, n, w, s));
    }

    int group(Walk& w, int64_t p0, int64_t G, int64_t per) {
        const int64_t r0 = w.top, last = r0 + G - 1;
        if (int rc = load(p0, r0, G)) return rc;
        if (int rc = frame(w, last, r0, G, p0)) return rc;
        if (int rc = chunks(r0, G, last, true, true, per)) return rc;  // a leaf's backward starts at once
        if (int rc = store_fwd(r0, p0, G)) return rc;
        return store_bwd(r0, p0, G);
    }
    int push(Walk& w, int node, int64_t r0) {
        const int64_t n = t.size(node), last = r0 + n - 1;
        if (int rc = load(t.start[node], r0, n)) return rc;
        if (int rc = frame(w, last, 0, 0, 0)) return rc;
        if (int rc = chunks(r0, n, last, true, false, chunk)) return rc;
        return store_fwd(r0, t.start[node], n);
    }
    int pop(Walk& w, int node, int64_t r0) {
        // every branch below has added its gradient to this node's keys
        const int64_t n = t.size(node), last = r0 + n - 1;
        if (int rc = frame(w, last, 0, 0, 0)) return rc;
        if (int rc = chunks(r0, n, last, false, true, chunk)) return rc;
        return store_bwd(r0, t.start[node], n);
    }
};

}  // namespace
}  // namespace treeattn

using namespace treeattn;

extern "C" {

int tree_dfs_plan(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent, int64_t n_nodes,
                  int64_t n_tokens, int32_t chunk, tree_dfs_plan_t* plan) {
    if (!plan) return set_error(TREE_E_ARG, "tree_dfs_plan: plan is NULL");
    try {
        Tree t;
        if (int rc = build_tree(node_start, node_end, node_parent, n_nodes, n_tokens, t)) return rc;
        if (int rc = plan_of(t, chunk, plan)) return rc;
    } catch (const std::bad_alloc&) {
        return set_error(TREE_E_NOMEM, "tree_dfs_plan: out of host memory");
    }
    clear_error();
    return TREE_OK;
}

size_t tree_attn_dfs_workspace_bytes(const tree_dfs_plan_t* plan, int32_t Hq, int32_t Hkv, int32_t D) {
    if (!plan || plan->rows <= 0 || plan->rows % (2 * kBlock) != 0 || plan->rows > kMaxL || Hq <= 0 || Hkv <= 0 ||
        D <= 0)
        return 0;
    return frame_layout(nullptr, plan->rows, Hq, Hkv, D).bytes;
}

int tree_attn_dfs(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent, int64_t n_nodes,
                  int64_t n_tokens, const void* q, const void* k, const void* v, const void* dout, void* o, float* lse,
                  void* dq, void* dk, void* dv, const int32_t* d_se, void* d_ws, size_t ws_bytes, int64_t L,
                  int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t chunk, void* stream) {
    if (int rc = check_attn("tree_attn_dfs", L, Hq, Hkv, D, scale, TREE_DTYPE_BF16)) return rc;
    if (!q || !k || !v || !dout || !o || !lse || !dq || !dk || !dv || !d_se || !d_ws)
        return set_error(TREE_E_ARG, "tree_attn_dfs: NULL device pointer");
    if (n_tokens > L) return set_error(TREE_E_ARG, "tree_attn_dfs: %lld tokens > L = %lld", (long long)n_tokens,
                                       (long long)L);
    try {
        Tree t;
        if (int rc = build_tree(node_start, node_end, node_parent, n_nodes, n_tokens, t)) return rc;
        tree_dfs_plan_t plan{};
        if (int rc = plan_of(t, chunk, &plan)) return rc;
        if (int rc = check_attn("tree_attn_dfs (frame)", plan.rows, Hq, Hkv, D, scale, TREE_DTYPE_BF16)) return rc;
        const size_t need = frame_layout(nullptr, plan.rows, Hq, Hkv, D).bytes;
        if (ws_bytes < need)
            return set_error(TREE_E_WORKSPACE, "tree_attn_dfs: workspace %zu < %zu bytes", ws_bytes, need);
        const hipStream_t s = static_cast<hipStream_t>(stream);
        Exec ex{t,
                static_cast<const char*>(q),
                static_cast<const char*>(k),
                static_cast<const char*>(v),
                static_cast<const char*>(dout),
                static_cast<char*>(o),
                static_cast<char*>(dq),
                static_cast<char*>(dk),
                static_cast<char*>(dv),
                lse,
                d_se,
                L,
                plan.rows,
                Hq,
                Hkv,
                D,
                scale,
                chunk,
                frame_layout(static_cast<char*>(d_ws), plan.rows, Hq, Hkv, D),
                s,
                int64_t(Hq) * D * 2,
                int64_t(Hkv) * D * 2};
        // the frame's inputs start finite (padding rows are read, weighted 0);
        // the packed outputs' padding rows get O = dQ = dK = dV = 0, LSE = -inf
        const size_t qbytes = size_t(plan.rows) * size_t(ex.qrow), kbytes = size_t(plan.rows) * size_t(ex.krow);
        hipError_t e = launch_dfs_fill(ex.f.q, int64_t(qbytes), 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.f.dO, int64_t(qbytes), 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.f.k, int64_t(kbytes), 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.f.v, int64_t(kbytes), 0u, s);
        if (e == hipSuccess) e = launch_dfs_iota(ex.f.iota, int(plan.rows / kBlock), s);
        const int64_t pad = L - n_tokens;
        if (e == hipSuccess) e = launch_dfs_fill(ex.o + n_tokens * ex.qrow, pad * ex.qrow, 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.dq + n_tokens * ex.qrow, pad * ex.qrow, 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.dk + n_tokens * ex.krow, pad * ex.krow, 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill(ex.dv + n_tokens * ex.krow, pad * ex.krow, 0u, s);
        if (e == hipSuccess) e = launch_dfs_fill_cols(lse, L, n_tokens, pad, Hq, -INFINITY, s);
        if (e != hipSuccess)
            return set_error(TREE_E_HIP, "tree_attn_dfs: HIP error %d (%s)", int(e), hipGetErrorString(e));
        Walk w(t, chunk, plan.leaf_rows);
        if (int rc = w.run(ex)) return rc;
    } catch (const std::bad_alloc&) {
        return set_error(TREE_E_NOMEM, "tree_attn_dfs: out of host memory");
    }
    clear_error();
    return TREE_OK;
}

}  // extern "C"
