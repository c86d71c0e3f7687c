// Internal: device-side types, the metadata workspace layout and the kernel
// launchers of libtreeattn.  Included by the .hip translation units and by
// the C ABI shim.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace treeattn {

constexpr int kBlock = 128;          // tile edge = padding unit
constexpr int64_t kMaxL = 1 << 20;   // largest packed length accepted

// Layout of the tree_meta workspace, in int32 words.  Segments are padded to
// 64 words (256 bytes).  nb = L / 128, T = nb (nb + 1) / 2 bounds the number
// of nonempty tiles (only key block <= query block can be nonempty).
//   hdr      [64]     hdr[0] = L, hdr[1] = nb, hdr[2] = real tokens
//   blk_min  [nb]     min subtree end over each key block (pads: -1)
//   blk_max  [nb]     max subtree end over each key block
//   hist     [L+1]    number of tokens whose subtree ends at each index
//   row_cnt  [nb]     nonempty tiles per query block
//   row_ptr  [nb+1]   CSR offsets into row_ent
//   row_ent  [T]      (key block << 1) | partial, ascending key block
//   col_cnt  [nb]     nonempty tiles per key block
//   col_ptr  [nb+1]
//   col_ent  [T]      (query block << 1) | partial, ascending query block
//   q_order  [nb]     query blocks in descending position (the forward's and
//                     dQ's work order)
//   k_order  [nb]     key blocks, most nonempty tiles first (ties: index)
//   blk_cnt  [nb]     real tokens per block, then their exclusive prefix
//   blk_hsum [nb]     histogram mass per block, then its exclusive prefix
//   hi64     [n64]    max subtree end over each 64-key chunk (pads: -1),
//                     n64 = L / 64
//   g_order  [n64]    the dK/dV kernel's key groups, most 64-query steps
//                     first (ties: index), as first chunk | (chunks - 1) << 14;
//                     hdr[3] holds their number
// Key groups: consecutive chunks with the same hi64 form a run (a node's
// chunks share one subtree end), and each run is cut into groups of at
// most four chunks from its start, so the groups tile the chunks.  A
// group's keys see query steps (64 rows) from its first chunk to
// hi64 / 64 at most.
// If the runs would give more groups starting before the last real chunk
// c_end than ceil(c_end / 4) + ceil(c_end / 16), every chunk is grouped by
// four from chunk 0 instead (ceil(n64 / 4) groups), so a dK/dV launch of
// dkdv_workgroups(c_end) workgroups per key/value head covers every group
// with work (and, at c_end = n64, every group).
constexpr int kChunk = 64;
constexpr int kMaxGroupChunks = 4;
__host__ __device__ inline int64_t dkdv_group_bound(int64_t c_end) { return (c_end + 3) / 4 + (c_end + 15) / 16; }
__host__ __device__ inline int64_t dkdv_workgroups(int64_t c_end) { return dkdv_group_bound(c_end) + 2; }
struct MetaLayout {
    int64_t L, nb, T, n64;
    int64_t hdr, blk_min, blk_max, hist, row_cnt, row_ptr, row_ent, col_cnt, col_ptr, col_ent,
        q_order, k_order, blk_cnt, blk_hsum, hi64, g_order, words;
};

inline int64_t pad64(int64_t w) { return (w + 63) / 64 * 64; }

inline MetaLayout meta_layout(int64_t L) {
    MetaLayout m{};
    m.L = L;
    m.nb = L / kBlock;
    m.T = m.nb * (m.nb + 1) / 2;
    m.n64 = L / kChunk;
    int64_t o = 0;
    m.hdr = o;     o += 64;
    m.blk_min = o; o += pad64(m.nb);
    m.blk_max = o; o += pad64(m.nb);
    m.hist = o;    o += pad64(L + 1);
    m.row_cnt = o; o += pad64(m.nb);
    m.row_ptr = o; o += pad64(m.nb + 1);
    m.row_ent = o; o += pad64(m.T);
    m.col_cnt = o; o += pad64(m.nb);
    m.col_ptr = o; o += pad64(m.nb + 1);
    m.col_ent = o; o += pad64(m.T);
    m.q_order = o; o += pad64(m.nb);
    m.k_order = o; o += pad64(m.nb);
    m.blk_cnt = o; o += pad64(m.nb);
    m.blk_hsum = o; o += pad64(m.nb);
    m.hi64 = o;    o += pad64(m.n64);
    m.g_order = o; o += pad64(m.n64);
    m.words = o;
    return m;
}

// Device pointers into a metadata workspace.
struct MetaPtrs {
    const int32_t* row_ptr;
    const int32_t* row_ent;
    const int32_t* col_ptr;
    const int32_t* col_ent;
    const int32_t* q_order;
    const int32_t* k_order;
    const int32_t* blk_min;
    const int32_t* blk_max;
    const int32_t* hdr;
    const int32_t* hi64;
    const int32_t* g_order;
};

inline MetaPtrs meta_ptrs(const void* ws, int64_t L) {
    const MetaLayout m = meta_layout(L);
    const int32_t* w = static_cast<const int32_t*>(ws);
    return {w + m.row_ptr, w + m.row_ent, w + m.col_ptr, w + m.col_ent, w + m.q_order,
            w + m.k_order, w + m.blk_min, w + m.blk_max, w + m.hdr, w + m.hi64, w + m.g_order};
}

// Backward phases (TREE_BWD_* of the public header).
constexpr int kPhaseAll = 0, kPhaseDelta = 1, kPhaseDkdv = 2, kPhaseDq = 3, kPhaseDqDelta = 4;

// Problem shape shared by the attention launchers.
struct AttnShape {
    int64_t L;
    int nb, Hq, Hkv, D;
    float scale;
};

// Restriction of one attention launch to some query blocks, for the
// depth-first variant, which runs one node's (or one chunk's) queries at a
// time over a stack of its ancestors' keys.  The default runs everything.
struct RowSel {
    const int32_t* q_list = nullptr;  // fwd / dQ: the query blocks to run (null: all, heaviest first)
    int n_q = 0;                      // entries of q_list
    int qb_lo = 0, qb_hi = 1 << 30;   // dK/dV: only query blocks in [qb_lo, qb_hi) contribute
    int n_wg = -1;                    // dK/dV: workgroups per key/value head, each taking every
                                      // n_wg-th key group of the heaviest-first order (-1: nb / 2)
    float* dk_acc = nullptr;          // dK/dV: if set, add scale * dK and dV in float32 to
    float* dv_acc = nullptr;          // these [L, Hkv, D] arrays instead of writing dK / dV
};

// Rotary embedding fused into the attention kernels: Q rotated at the
// forward's register load (and written to q_rot for the backward), dQ and dK
// rotated back in the backward's epilogues; pos = the trie's position ids,
// tab = launch_rope_table's (cos, sin) rows.  The default fuses nothing.
struct RopeArgs {
    const int32_t* pos = nullptr;
    const float* tab = nullptr;
    void* q_rot = nullptr;  // forward only
};

hipError_t launch_meta(const int32_t* se, int64_t L, int32_t* pos, uint8_t* tile_class, void* ws,
                       hipStream_t stream);

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int32_t* se, const MetaPtrs& mp, const AttnShape& sh,
                           hipStream_t stream, const RowSel& sel = RowSel(), const RopeArgs& rope = RopeArgs());
hipError_t launch_bwd_bf16(int phase, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           const int32_t* se, const MetaPtrs& mp, float* delta,
                           const AttnShape& sh, hipStream_t stream, const RowSel& sel = RowSel(),
                           const RopeArgs& rope = RopeArgs());
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const int32_t* se, const MetaPtrs& mp, const AttnShape& sh,
                          hipStream_t stream);
hipError_t launch_bwd_f32(int phase, const float* q, const float* k, const float* v, const float* o,
                          const float* lse, const float* dout, float* dq, float* dk, float* dv,
                          const int32_t* se, const MetaPtrs& mp, float* delta,
                          const AttnShape& sh, hipStream_t stream);

// Depth-first execution: the node segments on the stack of one frame (rows
// [row0, row0 + len) each, subtree end top_se) and the leaf rows being run
// (frame rows [leaf_row0, leaf_row0 + leaf_len) = packed rows from leaf_p0).
constexpr int kDfsMaxSegments = 240;
struct DfsSegments {
    int n, top_se;
    int leaf_row0, leaf_len, leaf_p0;
    int row0[kDfsMaxSegments];
    int len[kDfsMaxSegments];
};
hipError_t launch_dfs_se(int32_t* se, int64_t rows, const int32_t* packed_se, const DfsSegments& a,
                         hipStream_t stream);
hipError_t launch_dfs_copy_rows(const void* src, void* dst, int64_t s0, int64_t d0, int64_t nrows, int64_t row_bytes,
                                hipStream_t stream);
hipError_t launch_dfs_copy_cols(const float* src, float* dst, int64_t Ls, int64_t Ld, int64_t s0, int64_t d0,
                                int64_t n, int H, hipStream_t stream);
hipError_t launch_dfs_fill(void* p, int64_t bytes, uint32_t pattern, hipStream_t stream);
hipError_t launch_dfs_fill_cols(float* p, int64_t L, int64_t i0, int64_t n, int H, float value, hipStream_t stream);
hipError_t launch_dfs_iota(int32_t* p, int n, hipStream_t stream);
hipError_t launch_dfs_emit(const float* acc, void* out, int64_t s0, int64_t d0, int64_t nrows, int64_t width,
                           hipStream_t stream);

hipError_t launch_logits_stats(const void* logits, int64_t L, int64_t V, int dtype, float* lse, float* ent,
                               hipStream_t stream);
hipError_t launch_gather_logprobs(const void* logits, int64_t row0, int64_t n_rows, int64_t L, int64_t V, int dtype,
                                  const float* lse, const float* ent, const int32_t* ids, const int32_t* row_pos,
                                  int64_t B, int64_t S, float pad_value, float* out_logp, float* out_ent,
                                  hipStream_t stream);

hipError_t launch_rope_table(float* tab, int64_t P, int D, double base, hipStream_t stream);
hipError_t launch_rope_tab(const void* x, void* y, const int32_t* pos, const float* tab, int64_t L, int H, int D,
                           hipStream_t stream);
hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t L, int H, int D, double base, int inverse,
                       int dtype, hipStream_t stream);

}  // namespace treeattn
