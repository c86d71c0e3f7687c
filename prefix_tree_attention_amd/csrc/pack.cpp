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
//
// Token tries are flat arrays; child lookup goes through one open-addressing
// hash table per trie keyed by (parent node, token).

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
// open-addressing map (parent node, token) -> child node
// ---------------------------------------------------------------------------
class ChildMap {
  public:
    ChildMap() { rehash(1024); }

    int32_t find(int32_t parent, int32_t token) const {
        const uint64_t key = pack_key(parent, token);
        for (size_t i = slot(key);; i = (i + 1) & mask_) {
            if (keys_[i] == kEmpty) return -1;
            if (keys_[i] == key) return vals_[i];
        }
    }

    void insert(int32_t parent, int32_t token, int32_t child) {
        if ((size_ + 1) * 2 > keys_.size()) rehash(keys_.size() * 2);
        put(pack_key(parent, token), child);
        ++size_;
    }

  private:
    static constexpr uint64_t kEmpty = ~uint64_t(0);
    static uint64_t pack_key(int32_t parent, int32_t token) {
        return (uint64_t(uint32_t(parent)) << 32) | uint32_t(token);
    }
    size_t slot(uint64_t key) const {
        uint64_t h = key * 0x9E3779B97F4A7C15ull;
        return size_t(h >> 20) & mask_;
    }
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

// Uncompressed token trie.  Node 0 is the root (no token).
struct TokenTrie {
    std::vector<int32_t> token, first_child, last_child, next_sibling;
    std::vector<int32_t> n_children, n_end;  // children count; sequences ending here
    ChildMap map;
    std::vector<int32_t> seqs;  // batch rows, insertion order
    int64_t tokens = 0;

    TokenTrie() { add_node(-1, -1); }

    int32_t add_node(int32_t parent, int32_t tok) {
        const int32_t id = int32_t(token.size());
        token.push_back(tok);
        first_child.push_back(-1);
        last_child.push_back(-1);
        next_sibling.push_back(-1);
        n_children.push_back(0);
        n_end.push_back(0);
        if (parent >= 0) {
            if (last_child[parent] < 0)
                first_child[parent] = id;
            else
                next_sibling[last_child[parent]] = id;
            last_child[parent] = id;
            ++n_children[parent];
            map.insert(parent, tok, id);
        }
        return id;
    }

    // tokens an insertion would add = length minus the longest present prefix
    int64_t added(const int32_t* s, int64_t n) const {
        int32_t cur = 0;
        int64_t i = 0;
        for (; i < n; ++i) {
            const int32_t c = map.find(cur, s[i]);
            if (c < 0) break;
            cur = c;
        }
        return n - i;
    }

    void insert(const int32_t* s, int64_t n, int32_t row) {
        int32_t cur = 0;
        for (int64_t i = 0; i < n; ++i) {
            int32_t c = map.find(cur, s[i]);
            if (c < 0) {
                c = add_node(cur, s[i]);
                ++tokens;
            }
            cur = c;
        }
        ++n_end[cur];
        seqs.push_back(row);
    }
};

struct PackedTrie {
    int64_t n = 0, L = 0;
    std::vector<int32_t> token_ids, node_id, subtree_end;
    std::vector<int32_t> node_start, node_end, node_parent;
    std::vector<int32_t> seq_ids, seq_iv_ptr, seq_iv;
    int64_t n_pairs = 0;
};

// Compress, lay out in pre-order and pad one token trie.
void flatten(const TokenTrie& t, const std::vector<std::vector<int32_t>>& seqs, int64_t L,
             int32_t pad_id, PackedTrie& out) {
    const int64_t n = t.tokens;
    out.n = n;
    out.L = L;
    out.token_ids.assign(size_t(L), pad_id);
    out.node_id.assign(size_t(L), -1);
    out.subtree_end.assign(size_t(L), -1);
    std::vector<int32_t> comp_of(t.token.size(), -1);  // token node -> compressed node
    std::vector<int64_t> depth_end;                     // ancestors-or-self count at node end

    // Iterative pre-order walk over compressed nodes.  A frame is a token
    // node starting a compressed node; children are visited in insertion
    // order by pushing them reversed.
    struct Frame {
        int32_t tok_node;
        int32_t parent_comp;
        bool exit;
        int32_t comp;
    };
    std::vector<Frame> stack;
    std::vector<int32_t> kids;
    for (int32_t c = t.first_child[0]; c >= 0; c = t.next_sibling[c]) kids.push_back(c);
    for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back({*it, -1, false, -1});
    int64_t off = 0;
    while (!stack.empty()) {
        Frame f = stack.back();
        stack.pop_back();
        if (f.exit) {  // whole subtree laid out: its last index is off-1
            const int32_t se = int32_t(off - 1);
            for (int64_t i = out.node_start[f.comp]; i <= out.node_end[f.comp]; ++i)
                out.subtree_end[size_t(i)] = se;
            continue;
        }
        const int32_t comp = int32_t(out.node_start.size());
        out.node_start.push_back(int32_t(off));
        out.node_parent.push_back(f.parent_comp);
        int64_t d = f.parent_comp >= 0 ? depth_end[size_t(f.parent_comp)] : 0;
        int32_t cur = f.tok_node;
        for (;;) {
            comp_of[size_t(cur)] = comp;
            out.token_ids[size_t(off)] = t.token[size_t(cur)];
            out.node_id[size_t(off)] = comp;
            ++off;
            ++d;
            out.n_pairs += d;
            // merge into the only child when no sequence ends here
            if (t.n_children[size_t(cur)] == 1 && t.n_end[size_t(cur)] == 0)
                cur = t.first_child[size_t(cur)];
            else
                break;
        }
        out.node_end.push_back(int32_t(off - 1));
        depth_end.push_back(d);
        stack.push_back({cur, f.parent_comp, true, comp});
        kids.clear();
        for (int32_t c = t.first_child[size_t(cur)]; c >= 0; c = t.next_sibling[size_t(c)])
            kids.push_back(c);
        for (auto it = kids.rbegin(); it != kids.rend(); ++it)
            stack.push_back({*it, comp, false, -1});
    }

    // per-sequence node intervals, in insertion order, root first
    out.seq_ids = t.seqs;
    out.seq_iv_ptr.assign(1, 0);
    for (int32_t row : t.seqs) {
        const auto& s = seqs[size_t(row)];
        int32_t cur = 0, last = -1;
        for (int32_t tok : s) {
            cur = t.map.find(cur, tok);
            const int32_t c = comp_of[size_t(cur)];
            if (c != last) {
                out.seq_iv.push_back(out.node_start[size_t(c)]);
                out.seq_iv.push_back(out.node_end[size_t(c)]);
                last = c;
            }
        }
        out.seq_iv_ptr.push_back(int32_t(out.seq_iv.size() / 2));
    }
}

}  // namespace

struct tree_pack {
    std::vector<PackedTrie> tries;
    tree_pack_stats_t stats{};
};

extern "C" {

int tree_pack(const int32_t* ids, const uint8_t* mask, int64_t B, int64_t S,
              int64_t max_tokens_per_mb, int32_t block_size, int32_t pad_to_maximum,
              int32_t pad_id, tree_pack_t** out) {
    using treeattn::set_error;
    if (out) *out = nullptr;
    if (!out) return set_error(TREE_E_ARG, "tree_pack: out is NULL");
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
        std::vector<std::vector<int32_t>> seqs(static_cast<size_t>(B));
        int64_t original = 0;
        for (int64_t r = 0; r < B; ++r) {
            auto& s = seqs[size_t(r)];
            for (int64_t c = 0; c < S; ++c)
                if (mask[r * S + c]) s.push_back(ids[r * S + c]);
            if (s.empty()) return set_error(TREE_E_EMPTY_SEQ, "row %lld has no real token", (long long)r);
            if (int64_t(s.size()) > M)
                return set_error(TREE_E_SEQ_TOO_LONG, "row %lld has %zu tokens > max_tokens_per_mb=%lld",
                                 (long long)r, s.size(), (long long)M);
            original += int64_t(s.size());
        }
        std::vector<int32_t> order(static_cast<size_t>(B));
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
            return seqs[size_t(a)].size() > seqs[size_t(b)].size();
        });
        std::vector<std::unique_ptr<TokenTrie>> tries;
        for (int32_t r : order) {
            const auto& s = seqs[size_t(r)];
            const int64_t n = int64_t(s.size());
            TokenTrie* dst = nullptr;
            for (auto& t : tries)
                if (t->tokens + t->added(s.data(), n) <= M) {
                    dst = t.get();
                    break;
                }
            if (!dst) {
                tries.emplace_back(new TokenTrie());
                dst = tries.back().get();
            }
            dst->insert(s.data(), n, r);
        }
        std::unique_ptr<struct tree_pack> p(new struct tree_pack());
        p->tries.resize(tries.size());
        int64_t tree_tokens = 0, pairs = 0, unpacked = 0;
        for (size_t i = 0; i < tries.size(); ++i) {
            const int64_t n = tries[i]->tokens;
            const int64_t L = pad_to_maximum ? M : (n + block_size - 1) / block_size * block_size;
            flatten(*tries[i], seqs, L, pad_id, p->tries[i]);
            tries[i].reset();
            tree_tokens += n;
            pairs += p->tries[i].n_pairs;
        }
        for (const auto& s : seqs) unpacked += int64_t(s.size()) * (int64_t(s.size()) + 1) / 2;
        p->stats.n_tries = int64_t(p->tries.size());
        p->stats.original_tokens = original;
        p->stats.tree_tokens = tree_tokens;
        p->stats.tree_token_ratio = original ? double(tree_tokens) / double(original) : 0.0;
        p->stats.n_pairs = pairs;
        p->stats.unpacked_pairs = unpacked;
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

void tree_pack_free(tree_pack_t* p) { delete p; }

}  // extern "C"
