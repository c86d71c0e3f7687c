// Host trie packer of libtreeattn (tree_pack*).
//
// Follows the AReaL tree-training guide: section 参数背后的源码校验逻辑 for the
// argument checks, section 树构建流程 steps 1-3 for extraction, greedy
// first-fit-decreasing insertion and single-child chain compression, and
// sections 核心数据结构 / 打包数据的生成 for the pre-order layout with inclusive
// node ranges and per-sequence node intervals.  Readings of what the guide
// leaves open: the sort is stable by length (longest first), first fit scans
// tries in creation order with the budget counted in uncompressed tokens,
// children keep insertion order, a chain node merges into its only child
// exactly when no sequence ends at it (which is when both carry the same
// sequences), empty rows are an error, pads get node -1 / subtree end -1.
// tree_pack_ordered adds prefix-order packing: the lexicographic (DFS) order
// of AREAL-DTA's load-balancing section fills tries one after another (next
// fit), so each trie is a contiguous run of that order.
//
// The tries are built directly in compressed (radix) form: a node's tokens
// are a run of one source sequence, referenced by (sequence, start, length),
// and matching walks whole runs with a vectorisable compare instead of one
// lookup per token.  A node is split only where a later sequence branches
// off or ends inside it, so node boundaries are exactly the branch points
// and sequence ends -- the guide's compressed nodes.  Child lookup by first
// token goes through one open-addressing hash table per trie.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <numeric>
#include <vector>

#include "status.h"

namespace {

// ---------------------------------------------------------------------------
// open-addressing map (parent node, first token) -> child node
// ---------------------------------------------------------------------------
class ChildMap {
  public:
    ChildMap() { rehash(256); }

    int32_t find(int32_t parent, int32_t token) const {
        const uint64_t key = pack_key(parent, token);
        for (size_t i = slot(key);; i = (i + 1) & mask_) {
            if (keys_[i] == kEmpty) return -1;
            if (keys_[i] == key) return vals_[i];
        }
    }

    // insert or overwrite
    void set(int32_t parent, int32_t token, int32_t child) {
        const uint64_t key = pack_key(parent, token);
        for (size_t i = slot(key);; i = (i + 1) & mask_) {
            if (keys_[i] == key) {
                vals_[i] = child;
                return;
            }
            if (keys_[i] == kEmpty) break;
        }
        if ((size_ + 1) * 2 > keys_.size()) rehash(keys_.size() * 2);
        put(key, child);
        ++size_;
    }

  private:
    static constexpr uint64_t kEmpty = ~uint64_t(0);
    static uint64_t pack_key(int32_t parent, int32_t token) {
        return (uint64_t(uint32_t(parent)) << 32) | uint32_t(token);
    }
    size_t slot(uint64_t key) const { return size_t((key * 0x9E3779B97F4A7C15ull) >> 20) & mask_; }
    void put(uint64_t key, int32_t v) {
        size_t i = slot(key);
        while (keys_[i] != kEmpty) i = (i + 1) & mask_;
        keys_[i] = key;
        vals_[i] = v;
    }
    void rehash(size_t cap) {
        std::vector<uint64_t> ok;
        std::vector<int32_t> ov;
        ok.swap(keys_);
        ov.swap(vals_);
        keys_.assign(cap, kEmpty);
        vals_.assign(cap, -1);
        mask_ = cap - 1;
        for (size_t i = 0; i < ok.size(); ++i)
            if (ok[i] != kEmpty) put(ok[i], ov[i]);
    }
    std::vector<uint64_t> keys_;
    std::vector<int32_t> vals_;
    size_t mask_ = 0, size_ = 0;
};

// Extracted sequences, concatenated.
struct Seqs {
    std::vector<int32_t> tok;
    std::vector<int64_t> off;  // [B + 1]
    const int32_t* at(int32_t r) const { return tok.data() + off[size_t(r)]; }
    int64_t len(int32_t r) const { return off[size_t(r) + 1] - off[size_t(r)]; }
};

// Number of leading equal elements of a[0..n) and b[0..n).
int64_t common_prefix(const int32_t* a, const int32_t* b, int64_t n) {
    int64_t i = 0;
    while (i + 16 <= n && std::memcmp(a + i, b + i, 16 * sizeof(int32_t)) == 0) i += 16;
    while (i < n && a[i] == b[i]) ++i;
    return i;
}

// Compressed trie.  Node 0 is the root (no tokens).
struct RadixTrie {
    struct Node {
        int32_t row, start, len;    // tokens: seqs.at(row)[start .. start + len)
        int32_t parent;
        int32_t n_end;              // sequences ending at this node's last token
        std::vector<int32_t> kids;  // insertion order
    };
    std::vector<Node> nodes;
    ChildMap map;
    std::vector<int32_t> seq_rows, seq_end;  // insertion order; node holding each sequence's last token
    int64_t tokens = 0;

    RadixTrie() { nodes.push_back({-1, 0, 0, -1, 0, {}}); }

    // Where a walk of s stops: at the end of `node` (mid == -1) or inside
    // child `mid` after `midlen` of its tokens; `matched` tokens of s agree.
    struct Walk {
        int32_t node, mid, midlen;
        int64_t matched;
    };

    Walk walk(const Seqs& S, const int32_t* s, int64_t n) const {
        int32_t node = 0;
        int64_t i = 0;
        for (;;) {
            if (i == n) return {node, -1, 0, i};
            const int32_t c = map.find(node, s[i]);
            if (c < 0) return {node, -1, 0, i};
            const Node& x = nodes[size_t(c)];
            const int64_t lim = std::min<int64_t>(x.len, n - i);
            const int64_t m = 1 + common_prefix(s + i + 1, S.at(x.row) + x.start + 1, lim - 1);
            if (m < x.len) return {node, c, int32_t(m), i + m};
            i += x.len;
            node = c;
        }
    }

    void insert(const Seqs& S, int32_t row, const Walk& w) {
        const int64_t n = S.len(row);
        const int32_t* s = S.at(row);
        int32_t at = w.node;
        if (w.mid >= 0) {  // split child `mid` after `midlen` tokens; the old node keeps the suffix
            const int32_t x = w.mid;
            const int32_t y = int32_t(nodes.size());
            Node pre{nodes[size_t(x)].row, nodes[size_t(x)].start, w.midlen, nodes[size_t(x)].parent, 0, {x}};
            const int32_t par = pre.parent;
            const int32_t first = S.at(pre.row)[pre.start];
            nodes.push_back(std::move(pre));
            Node& X = nodes[size_t(x)];
            X.start += w.midlen;
            X.len -= w.midlen;
            X.parent = y;
            for (auto& k : nodes[size_t(par)].kids)
                if (k == x) k = y;
            map.set(par, first, y);
            map.set(y, S.at(X.row)[X.start], x);
            at = y;
        }
        int32_t end = at;
        if (w.matched < n) {  // new leaf with the rest of s
            end = int32_t(nodes.size());
            nodes.push_back({row, int32_t(w.matched), int32_t(n - w.matched), at, 0, {}});
            nodes[size_t(at)].kids.push_back(end);
            map.set(at, s[w.matched], end);
            tokens += n - w.matched;
        }
        ++nodes[size_t(end)].n_end;
        seq_rows.push_back(row);
        seq_end.push_back(end);
    }
};

struct PackedTrie {
    int64_t n = 0, L = 0;
    std::vector<int32_t> token_ids, node_id, subtree_end;
    std::vector<int32_t> node_start, node_end, node_parent;
    std::vector<int32_t> seq_ids, seq_iv_ptr, seq_iv;
    int64_t n_pairs = 0;
};

// Lay out one trie in pre-order (children in insertion order) and pad.
void flatten(const RadixTrie& t, const Seqs& S, int64_t L, int32_t pad_id, PackedTrie& out) {
    const int64_t n = t.tokens;
    out.n = n;
    out.L = L;
    out.token_ids.assign(size_t(L), pad_id);
    out.node_id.assign(size_t(L), -1);
    out.subtree_end.assign(size_t(L), -1);
    const size_t nn = t.nodes.size();
    std::vector<int32_t> pre_id(nn, -1);    // radix node -> pre-order index
    std::vector<int64_t> depth_end(nn, 0);  // ancestors-or-self count at a node's last token
    struct Frame {
        int32_t node;
        bool exit;
    };
    std::vector<Frame> stack;
    const auto& rk = t.nodes[0].kids;
    for (auto it = rk.rbegin(); it != rk.rend(); ++it) stack.push_back({*it, false});
    int64_t off = 0;
    while (!stack.empty()) {
        const Frame f = stack.back();
        stack.pop_back();
        const auto& x = t.nodes[size_t(f.node)];
        if (f.exit) {  // subtree laid out: its last index is off - 1
            const int32_t id = pre_id[size_t(f.node)];
            std::fill(out.subtree_end.begin() + out.node_start[size_t(id)],
                      out.subtree_end.begin() + out.node_end[size_t(id)] + 1, int32_t(off - 1));
            continue;
        }
        const int32_t me = int32_t(out.node_start.size());
        pre_id[size_t(f.node)] = me;
        const int32_t par = x.parent > 0 ? pre_id[size_t(x.parent)] : -1;
        out.node_start.push_back(int32_t(off));
        out.node_end.push_back(int32_t(off + x.len - 1));
        out.node_parent.push_back(par);
        std::memcpy(out.token_ids.data() + off, S.at(x.row) + x.start, size_t(x.len) * sizeof(int32_t));
        std::fill(out.node_id.begin() + off, out.node_id.begin() + off + x.len, me);
        const int64_t d0 = x.parent > 0 ? depth_end[size_t(x.parent)] : 0;
        depth_end[size_t(f.node)] = d0 + x.len;
        out.n_pairs += int64_t(x.len) * d0 + int64_t(x.len) * (x.len + 1) / 2;
        off += x.len;
        stack.push_back({f.node, true});
        for (auto it = x.kids.rbegin(); it != x.kids.rend(); ++it) stack.push_back({*it, false});
    }

    // per-sequence node intervals, insertion order, root first
    out.seq_ids = t.seq_rows;
    out.seq_iv_ptr.assign(1, 0);
    std::vector<int32_t> path;
    for (size_t k = 0; k < t.seq_rows.size(); ++k) {
        path.clear();
        for (int32_t v = t.seq_end[k]; v > 0; v = t.nodes[size_t(v)].parent) path.push_back(pre_id[size_t(v)]);
        for (auto it = path.rbegin(); it != path.rend(); ++it) {
            out.seq_iv.push_back(out.node_start[size_t(*it)]);
            out.seq_iv.push_back(out.node_end[size_t(*it)]);
        }
        out.seq_iv_ptr.push_back(int32_t(out.seq_iv.size() / 2));
    }
}

// Nonempty 128x128 tiles of one trie, split into full and partial, from the
// subtree ends alone.  Key j is visible to query i iff j <= i <= se[j], and
// subtree intervals are laminar, so key block kb's nonempty tiles are the
// query blocks kb .. max_se / 128 (the diagonal one partial), and the tile
// of query block qb > kb is full exactly when every key of kb is visible to
// every query of qb: min_se >= 128 qb + 127.  Pads (se = -1) sit after the
// real tokens and make their blocks' minimum -1.
void count_tiles(const PackedTrie& t, int64_t& full, int64_t& partial) {
    const int64_t nb = t.L / TREE_BLOCK;
    for (int64_t kb = 0; kb < nb; ++kb) {
        int32_t lo = INT32_MAX, hi = -1;
        for (int64_t j = kb * TREE_BLOCK; j < (kb + 1) * TREE_BLOCK; ++j) {
            lo = std::min(lo, t.subtree_end[size_t(j)]);
            hi = std::max(hi, t.subtree_end[size_t(j)]);
        }
        if (hi < 0) continue;  // no real key
        const int64_t nonempty = hi / TREE_BLOCK - kb + 1;
        const int64_t last_full = lo >= TREE_BLOCK - 1 ? (int64_t(lo) - (TREE_BLOCK - 1)) / TREE_BLOCK : -1;
        const int64_t f = std::max<int64_t>(0, last_full - kb);
        full += f;
        partial += nonempty - f;
    }
}

}  // namespace

struct tree_pack {
    std::vector<PackedTrie> tries;
    tree_pack_stats_t stats{};
    int64_t B = 0, S = 0;  // batch shape the pack was built from
};

extern "C" {

int tree_pack(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S,
              int64_t max_tokens_per_mb, int32_t block_size, int32_t pad_to_maximum,
              int32_t pad_id, tree_pack_t** out) {
    return tree_pack_ordered(ids, mask, B, S, max_tokens_per_mb, block_size, pad_to_maximum, pad_id, TREE_PACK_FFD,
                             out);
}

int tree_pack_ordered(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S,
                      int64_t max_tokens_per_mb, int32_t block_size, int32_t pad_to_maximum,
                      int32_t pad_id, int32_t order_kind, tree_pack_t** out) {
    using treeattn::set_error;
    if (out) *out = nullptr;
    if (!out) return set_error(TREE_E_ARG, "tree_pack: out is NULL");
    if (order_kind != TREE_PACK_FFD && order_kind != TREE_PACK_PREFIX)
        return set_error(TREE_E_ARG, "tree_pack_ordered: unknown order %d", order_kind);
    if (max_tokens_per_mb <= 0)
        return set_error(TREE_E_MAX_TOKENS, "max_tokens_per_mb must be a positive integer (got %lld)",
                         (long long)max_tokens_per_mb);
    if (block_size != TREE_BLOCK)
        return set_error(TREE_E_ARG, "block_size must be %d (got %d)", TREE_BLOCK, block_size);
    if (max_tokens_per_mb % block_size != 0)
        return set_error(TREE_E_ALIGN, "max_tokens_per_mb=%lld is not a multiple of %d",
                         (long long)max_tokens_per_mb, block_size);
    if (max_tokens_per_mb > (int64_t(1) << 30))
        return set_error(TREE_E_ARG, "max_tokens_per_mb=%lld too large", (long long)max_tokens_per_mb);
    if (B < 0 || S < 0 || (B > 0 && S > 0 && (!ids || !mask)))
        return set_error(TREE_E_ARG, "tree_pack: bad batch shape or NULL input");
    try {
        const int64_t M = max_tokens_per_mb;
        Seqs seqs;
        seqs.off.assign(size_t(B) + 1, 0);
        seqs.tok.reserve(size_t(B * S));
        for (int64_t r = 0; r < B; ++r) {
            const int32_t* ir = ids + r * S;
            const uint8_t* mr = mask + r * S;
            for (int64_t c = 0; c < S; ++c)
                if (mr[c]) seqs.tok.push_back(ir[c]);
            seqs.off[size_t(r) + 1] = int64_t(seqs.tok.size());
            const int64_t len = seqs.len(int32_t(r));
            if (len == 0) return set_error(TREE_E_EMPTY_SEQ, "row %lld has no real token", (long long)r);
            if (len > M)
                return set_error(TREE_E_SEQ_TOO_LONG, "row %lld has %lld tokens > max_tokens_per_mb=%lld",
                                 (long long)r, (long long)len, (long long)M);
        }
        const int64_t original = int64_t(seqs.tok.size());
        std::vector<int32_t> order(static_cast<size_t>(B));
        std::iota(order.begin(), order.end(), 0);
        const bool prefix = order_kind == TREE_PACK_PREFIX;
        if (prefix)  // lexicographic (DFS) order, a proper prefix first, ties by row
            std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
                return std::lexicographical_compare(seqs.at(a), seqs.at(a) + seqs.len(a), seqs.at(b),
                                                    seqs.at(b) + seqs.len(b));
            });
        else  // longest first, ties by row
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t a, int32_t b) { return seqs.len(a) > seqs.len(b); });
        std::vector<std::unique_ptr<RadixTrie>> tries;
        for (int32_t r : order) {
            const int64_t n = seqs.len(r);
            RadixTrie* dst = nullptr;
            RadixTrie::Walk w{};
            // first fit over all tries, or (prefix order) the newest one only
            for (size_t k = prefix && !tries.empty() ? tries.size() - 1 : 0; k < tries.size(); ++k) {
                RadixTrie* t = tries[k].get();
                w = t->walk(seqs, seqs.at(r), n);
                if (t->tokens + (n - w.matched) <= M) {
                    dst = t;
                    break;
                }
            }
            if (!dst) {
                tries.emplace_back(new RadixTrie());
                dst = tries.back().get();
                w = {0, -1, 0, 0};
            }
            dst->insert(seqs, r, w);
        }
        std::unique_ptr<struct tree_pack> p(new struct tree_pack());
        p->tries.resize(tries.size());
        int64_t tree_tokens = 0, pairs = 0, unpacked = 0, full = 0, partial = 0, causal = 0;
        for (size_t i = 0; i < tries.size(); ++i) {
            const int64_t n = tries[i]->tokens;
            const int64_t L = pad_to_maximum ? M : (n + block_size - 1) / block_size * block_size;
            flatten(*tries[i], seqs, L, pad_id, p->tries[i]);
            tries[i].reset();
            tree_tokens += n;
            pairs += p->tries[i].n_pairs;
            count_tiles(p->tries[i], full, partial);
            causal += (L / block_size) * (L / block_size + 1) / 2;
        }
        for (int64_t r = 0; r < B; ++r) unpacked += seqs.len(int32_t(r)) * (seqs.len(int32_t(r)) + 1) / 2;
        p->stats.n_tries = int64_t(p->tries.size());
        p->stats.original_tokens = original;
        p->stats.tree_tokens = tree_tokens;
        p->stats.tree_token_ratio = original ? double(tree_tokens) / double(original) : 0.0;
        p->stats.n_pairs = pairs;
        p->stats.unpacked_pairs = unpacked;
        p->stats.tiles_full = full;
        p->stats.tiles_partial = partial;
        p->stats.tiles_causal = causal;
        p->B = B;
        p->S = S;
        *out = p.release();
        treeattn::clear_error();
        return TREE_OK;
    } catch (const std::bad_alloc&) {
        return set_error(TREE_E_NOMEM, "tree_pack: out of host memory");
    } catch (...) {
        return set_error(TREE_E_ARG, "tree_pack: unexpected failure");
    }
}

int64_t tree_pack_num_tries(const tree_pack_t* p) { return p ? int64_t(p->tries.size()) : -1; }

int tree_pack_trie(const tree_pack_t* p, int64_t t, tree_trie_view* v) {
    if (!p || !v || t < 0 || t >= int64_t(p->tries.size()))
        return treeattn::set_error(TREE_E_ARG, "tree_pack_trie: bad pack, view or index %lld", (long long)t);
    const PackedTrie& x = p->tries[size_t(t)];
    v->n_tokens = x.n;
    v->L = x.L;
    v->n_nodes = int64_t(x.node_start.size());
    v->n_seqs = int64_t(x.seq_ids.size());
    v->token_ids = x.token_ids.data();
    v->node_id = x.node_id.data();
    v->subtree_end = x.subtree_end.data();
    v->node_start = x.node_start.data();
    v->node_end = x.node_end.data();
    v->node_parent = x.node_parent.data();
    v->seq_ids = x.seq_ids.data();
    v->seq_iv_ptr = x.seq_iv_ptr.data();
    v->seq_iv = x.seq_iv.data();
    treeattn::clear_error();
    return TREE_OK;
}

int tree_pack_stats(const tree_pack_t* p, tree_pack_stats_t* s) {
    if (!p || !s) return treeattn::set_error(TREE_E_ARG, "tree_pack_stats: NULL argument");
    *s = p->stats;
    treeattn::clear_error();
    return TREE_OK;
}

int tree_pack_concat(const tree_pack_t* p, int32_t* out_se, int64_t cap, int64_t* L_total) {
    if (!p || !L_total) return treeattn::set_error(TREE_E_ARG, "tree_pack_concat: NULL argument");
    int64_t total = 0;
    for (const PackedTrie& x : p->tries) total += x.L;
    *L_total = total;
    if (out_se) {
        if (cap < total)
            return treeattn::set_error(TREE_E_ARG, "tree_pack_concat: capacity %lld < %lld", (long long)cap,
                                       (long long)total);
        int64_t off = 0;
        for (const PackedTrie& x : p->tries) {
            for (int64_t i = 0; i < x.L; ++i) {
                const int32_t s = x.subtree_end[size_t(i)];
                out_se[off + i] = s < 0 ? -1 : int32_t(s + off);
            }
            off += x.L;
        }
    }
    treeattn::clear_error();
    return TREE_OK;
}

int tree_pack_concat_ids(const tree_pack_t* p, int32_t* out_ids, int64_t cap) {
    if (!p || !out_ids) return treeattn::set_error(TREE_E_ARG, "tree_pack_concat_ids: NULL argument");
    int64_t total = 0;
    for (const PackedTrie& x : p->tries) total += x.L;
    if (cap < total)
        return treeattn::set_error(TREE_E_ARG, "tree_pack_concat_ids: capacity %lld < %lld", (long long)cap,
                                   (long long)total);
    int64_t off = 0;
    for (const PackedTrie& x : p->tries) {
        std::copy(x.token_ids.begin(), x.token_ids.end(), out_ids + off);
        off += x.L;
    }
    treeattn::clear_error();
    return TREE_OK;
}

int tree_pack_row_positions(const tree_pack_t* p, int32_t* out, int64_t cap) {
    if (!p || (!out && p->B * p->S > 0))
        return treeattn::set_error(TREE_E_ARG, "tree_pack_row_positions: NULL argument");
    if (cap < p->B * p->S)
        return treeattn::set_error(TREE_E_ARG, "tree_pack_row_positions: capacity %lld < B*S = %lld",
                                   (long long)cap, (long long)(p->B * p->S));
    std::fill(out, out + p->B * p->S, -1);
    int64_t off = 0;
    for (const PackedTrie& x : p->tries) {
        // sequence k of the trie is batch row seq_ids[k]; its tokens are the
        // concatenation of its node intervals, root to leaf
        for (size_t k = 0; k + 1 < x.seq_iv_ptr.size(); ++k) {
            int32_t* row = out + int64_t(x.seq_ids[k]) * p->S;
            int64_t n = 0;
            for (int32_t iv = x.seq_iv_ptr[k]; iv < x.seq_iv_ptr[k + 1]; ++iv)
                for (int32_t i = x.seq_iv[size_t(2 * iv)]; i <= x.seq_iv[size_t(2 * iv + 1)]; ++i)
                    row[n++] = int32_t(off + i);
        }
        off += x.L;
    }
    treeattn::clear_error();
    return TREE_OK;
}

int tree_partition(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S, int32_t K, int32_t* out_group,
                   int64_t* out_max_cost, int64_t* out_costs) {
    using treeattn::set_error;
    if (K <= 0) return set_error(TREE_E_ARG, "tree_partition: K must be positive (got %d)", K);
    if (B < 0 || S < 0 || (B > 0 && (!out_group || (S > 0 && (!ids || !mask)))))
        return set_error(TREE_E_ARG, "tree_partition: bad batch shape or NULL argument");
    try {
        // real tokens of each row, in column order
        std::vector<int64_t> off(size_t(B) + 1, 0);
        std::vector<int32_t> tok;
        tok.reserve(size_t(B * S));
        for (int64_t r = 0; r < B; ++r) {
            for (int64_t c = 0; c < S; ++c)
                if (mask[r * S + c]) tok.push_back(ids[r * S + c]);
            off[size_t(r) + 1] = int64_t(tok.size());
        }
        auto len = [&](int64_t r) { return off[size_t(r) + 1] - off[size_t(r)]; };
        auto at = [&](int64_t r) { return tok.data() + off[size_t(r)]; };
        // lexicographic (DFS) order, a proper prefix first, ties by row
        std::vector<int64_t> order(static_cast<size_t>(B));
        std::iota(order.begin(), order.end(), int64_t(0));
        std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
            return std::lexicographical_compare(at(a), at(a) + len(a), at(b), at(b) + len(b));
        });
        // tokens each sequence adds to the tree of the sequences before it
        std::vector<int64_t> add(static_cast<size_t>(B)), full(static_cast<size_t>(B));
        int64_t lo = 0, hi = 0;
        for (int64_t i = 0; i < B; ++i) {
            const int64_t r = order[size_t(i)], n = len(r);
            int64_t l = 0;
            if (i > 0) {
                const int64_t q = order[size_t(i - 1)], m = std::min(n, len(q));
                const int32_t *x = at(r), *y = at(q);
                while (l < m && x[l] == y[l]) ++l;
            }
            add[size_t(i)] = n - l;
            full[size_t(i)] = n;
            lo = std::max(lo, n);
            hi += n - l;
        }
        // greedy check: groups needed under maximum cost tau (a fresh group
        // costs the sequence's full length)
        auto groups_for = [&](int64_t tau, int32_t* grp) {
            int64_t g = -1, cost = 0;
            for (int64_t i = 0; i < B; ++i) {
                if (g < 0 || cost + add[size_t(i)] > tau) {
                    ++g;
                    cost = full[size_t(i)];
                } else {
                    cost += add[size_t(i)];
                }
                if (grp) grp[order[size_t(i)]] = int32_t(g);
            }
            return g + 1;
        };
        if (B > 0) {
            lo = std::min(lo, hi);
            while (lo < hi) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (groups_for(mid, nullptr) <= K)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            groups_for(lo, out_group);
        }
        if (out_max_cost) *out_max_cost = B > 0 ? lo : 0;
        if (out_costs) {
            std::fill(out_costs, out_costs + K, int64_t(0));
            int64_t pg = -1;
            for (int64_t i = 0; i < B; ++i) {
                const int64_t g = out_group[order[size_t(i)]];
                out_costs[g] += (g == pg) ? add[size_t(i)] : full[size_t(i)];
                pg = g;
            }
        }
        treeattn::clear_error();
        return TREE_OK;
    } catch (const std::bad_alloc&) {
        return set_error(TREE_E_NOMEM, "tree_partition: out of host memory");
    }
}

void tree_pack_free(tree_pack_t* p) { delete p; }

}  // extern "C"
