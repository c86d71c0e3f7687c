// Metadata kernels of libtreeattn (tree_meta): position ids, 128x128 tile
// classes and the tile lists of the attention kernels, all derived from the
// per-token subtree ends se[L] in O(L + nb^2) work spread over one
// workgroup per 128-token block; a single workgroup only scans and sorts
// per-block values.
//
// AReaL tree-training guide, section 打包数据的生成: a token's position id is
// the number of tokens it may attend to, minus one.  Key j is visible to
// query i iff j <= i <= se[j] (the subtree intervals of a pre-order layout
// are laminar), so
//   |A(i)| = #{real j <= i} - #{real j : se[j] < i},
// and the second count is an exclusive prefix sum of a histogram of se.
// For a tile (query block qb, key block kb < qb) with lo/hi the min/max of
// se over the key block (pads count as -1): empty iff hi < 128 qb, full iff
// lo >= 128 qb + 127, else partial.  A diagonal tile is partial iff its
// block holds a real token; tiles above the diagonal are empty.  These rules
// are exact, not conservative.  They also put column kb's nonempty tiles in
// closed form: the contiguous range qb = kb .. hi / 128 (when the block
// holds a real token, hi >= 128 kb), full exactly for kb < qb <=
// (lo - 127) / 128.

#include "device.h"

namespace treeattn {
namespace {

__global__ void meta_init(int32_t* __restrict__ hist, int64_t n_hist, int32_t* __restrict__ hdr, int64_t L,
                          int nb) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_hist; i += stride) hist[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[0] = int32_t(L);
        hdr[1] = nb;
        hdr[2] = 0;
    }
}

// One workgroup per 128-token block: histogram of subtree ends, the block's
// min / max subtree end and its real-token count.
__global__ __launch_bounds__(128) void meta_blocks(const int32_t* __restrict__ se, int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ blk_min, int32_t* __restrict__ blk_max,
                                                   int32_t* __restrict__ blk_cnt, int32_t* __restrict__ hdr,
                                                   int32_t* __restrict__ hi64, int L) {
    const int b = blockIdx.x;
    const int j = b * kBlock + threadIdx.x;
    int s = se[j];
    if (s < -1 || s >= L) s = -1;  // malformed input: treat as a pad, never index out of range
    // one atomic per run of equal subtree ends (a node's tokens share one),
    // so a long shared prefix does not serialise on a single counter
    __shared__ int ss[kBlock];
    ss[threadIdx.x] = s;
    __syncthreads();
    if (s >= 0 && (threadIdx.x == 0 || ss[threadIdx.x - 1] != s)) {
        int run = 1;
        while (threadIdx.x + run < kBlock && ss[threadIdx.x + run] == s) ++run;
        atomicAdd(&hist[s], run);
    }
    int mn = s, mx = s;
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off));
        mx = max(mx, __shfl_xor(mx, off));
    }
    const unsigned long long real = __ballot(s >= 0);
    __shared__ int smn[2], smx[2], sreal[2];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) {
        smn[wave] = mn;
        smx[wave] = mx;
        sreal[wave] = __popcll(real);
        hi64[2 * b + wave] = mx;  // each wave holds one 64-key chunk
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nreal = sreal[0] + sreal[1];
        blk_min[b] = min(smn[0], smn[1]);
        blk_max[b] = max(smx[0], smx[1]);
        blk_cnt[b] = nreal;
        if (nreal) atomicAdd(&hdr[2], nreal);
    }
}

// Class of tile (qb, kb): 0 empty, 1 partial, 2 full; lo / hi are the key
// block's min / max subtree end.
__device__ __forceinline__ int tile_class_of(int qb, int kb, int lo, int hi) {
    if (kb > qb) return 0;
    if (kb == qb) return hi >= 0 ? 1 : 0;
    return hi < qb * kBlock ? 0 : (lo >= qb * kBlock + kBlock - 1 ? 2 : 1);
}

// Sum of one int per thread over the workgroup (blockDim.x a multiple of 64,
// at most 16 waves); `sh` holds >= 16 ints.
__device__ inline int block_sum(int x, int* sh) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = x;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < nw; ++w) t += sh[w];
    return t;
}

// One workgroup per query block: the class of every tile of its row, the
// row's nonempty count, and the block's histogram mass.
__global__ __launch_bounds__(256) void meta_tiles(const int32_t* __restrict__ blk_min,
                                                  const int32_t* __restrict__ blk_max,
                                                  const int32_t* __restrict__ hist, uint8_t* __restrict__ tc,
                                                  int32_t* __restrict__ row_cnt, int32_t* __restrict__ blk_hsum,
                                                  int nb) {
    const int qb = blockIdx.x;
    int cnt = 0;
    for (int kb = threadIdx.x; kb < nb; kb += blockDim.x) {
        const int c = tile_class_of(qb, kb, blk_min[kb], blk_max[kb]);
        tc[int64_t(qb) * nb + kb] = uint8_t(c);
        cnt += c != 0;
    }
    const int hs = threadIdx.x < kBlock ? hist[qb * kBlock + threadIdx.x] : 0;
    __shared__ int sh[16];
    const int rc = block_sum(cnt, sh);
    const int hm = block_sum(hs, sh);
    if (threadIdx.x == 0) {
        row_cnt[qb] = rc;
        blk_hsum[qb] = hm;
    }
}

// Exclusive scan of one value per thread across a 1024-thread workgroup.
// Returns the exclusive prefix; *total receives the sum.  Uses `sh` (>= 17
// long longs of shared memory).
__device__ inline long long block_exclusive_scan(long long x, long long* sh, long long* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    long long inc = x;
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long run = 0;
        for (int w = 0; w < nw; ++w) {
            const long long t = sh[w];
            sh[w] = run;
            run += t;
        }
        sh[nw] = run;
    }
    __syncthreads();
    const long long res = sh[wave] + inc - x;
    *total = sh[nw];
    __syncthreads();
    return res;
}

// Exclusive max-scan of one int per thread across the workgroup, in thread
// order (-1 for thread 0).  Uses `sh` (>= 17 ints of shared memory).
__device__ inline int block_exclusive_max(int x, int* sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int inc = x;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (lane >= off) inc = max(inc, y);
    }
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = -1;
        for (int w = 0; w < nw; ++w) {
            const int v = sh[w];
            sh[w] = run;
            run = max(run, v);
        }
    }
    __syncthreads();
    int ex = __shfl_up(inc, 1);
    if (lane == 0) ex = -1;
    const int res = max(sh[wave], ex);
    __syncthreads();
    return res;
}

// Single workgroup over per-block values: column counts (closed form),
// exclusive prefixes of (real tokens, histogram mass) per block and of
// (row, column) counts (the CSR pointers), the heaviest-first orders and the
// dK/dV kernel's key groups.
__global__ __launch_bounds__(1024) void meta_scan(const int32_t* __restrict__ blk_max,
                                                  int32_t* __restrict__ blk_cnt, int32_t* __restrict__ blk_hsum,
                                                  const int32_t* __restrict__ row_cnt, int32_t* __restrict__ col_cnt,
                                                  int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_ptr,
                                                  int32_t* __restrict__ q_order, int32_t* __restrict__ k_order,
                                                  const int32_t* __restrict__ hi64, int32_t* __restrict__ g_order,
                                                  int32_t* __restrict__ hdr, int nb) {
    __shared__ long long sh[32];
    __shared__ int shi[32];
    const int t = threadIdx.x, nt = blockDim.x;
    const int chunk = (nb + nt - 1) / nt;
    const int a = min(nb, t * chunk), e = min(nb, a + chunk);
    for (int i = a; i < e; ++i) {
        const int hi = blk_max[i];
        col_cnt[i] = hi >= 0 ? min(nb - 1, hi / kBlock) - i + 1 : 0;
    }
    long long total;
    {
        long long r = 0, h = 0;
        for (int i = a; i < e; ++i) {
            r += blk_cnt[i];
            h += blk_hsum[i];
        }
        // pack the two counts (each <= 2^20) into one scan value
        const long long base = block_exclusive_scan((h << 32) | r, sh, &total);
        long long rr = base & 0xffffffffll, hh = base >> 32;
        for (int i = a; i < e; ++i) {
            const int ci = blk_cnt[i], hi = blk_hsum[i];
            blk_cnt[i] = int32_t(rr);
            blk_hsum[i] = int32_t(hh);
            rr += ci;
            hh += hi;
        }
    }
    {
        long long r = 0, c = 0;
        for (int i = a; i < e; ++i) {
            r += row_cnt[i];
            c += col_cnt[i];
        }
        const long long base = block_exclusive_scan((r << 32) | c, sh, &total);
        long long rr = base >> 32, cc = base & 0xffffffffll;
        for (int i = a; i < e; ++i) {
            row_ptr[i] = int32_t(rr);
            col_ptr[i] = int32_t(cc);
            rr += row_cnt[i];
            cc += col_cnt[i];
        }
        if (t == 0) {
            row_ptr[nb] = int32_t(total >> 32);
            col_ptr[nb] = int32_t(total & 0xffffffffll);
        }
    }

    // The forward and dQ take query blocks in descending position: the
    // workgroups in flight on an XCD then hold neighbouring blocks, whose
    // row lists name mostly the same key tiles (read from its L2), and
    // within a trie the later blocks have the longer lists, so long items
    // still start first.  (Heaviest-first over the whole launch spread the
    // blocks in flight over all tries and ran 6-8% slower on GRPO-shaped
    // batches.)  The key-block order is heaviest first, ties by index: the
    // keys ((nb - count) << 13) | index are unique, so sorting them ascending
    // with a bitonic network in LDS gives exactly that order in
    // O(nb log^2 nb) work (nb <= 8192 = 2^13 blocks).
    constexpr int kMaxNb = int(kMaxL / kBlock);
    constexpr int kMaxChunks = int(kMaxL / kChunk);
    static_assert(kMaxNb <= (1 << 13), "block index must fit 13 bits");
    static_assert(kMaxChunks <= (1 << 14), "chunk index must fit 14 bits");
    __shared__ unsigned kk[kMaxNb], kg[kMaxChunks];
    __shared__ unsigned char gflag[kMaxChunks];
    int n = 1;
    while (n < nb) n <<= 1;
    __syncthreads();  // col_cnt written by other threads above
    for (int i = t; i < n; i += nt) kk[i] = i < nb ? (unsigned(nb - col_cnt[i]) << 13) | unsigned(i) : 0xffffffffu;
    __syncthreads();
    for (int k = 2; k <= n; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < n; i += nt) {
                const int p = i ^ j;
                if (p > i) {
                    const unsigned x = kk[i], y = kk[p];
                    if ((x > y) == ((i & k) == 0)) {
                        kk[i] = y;
                        kk[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int i = t; i < nb; i += nt) {
        q_order[i] = nb - 1 - i;
        k_order[i] = int(kk[i] & 0x1fffu);
    }

    // Key groups of the dK/dV kernel: a run of chunks with one subtree-end
    // maximum, cut every four chunks from the run's start.  Each thread
    // walks a contiguous range of chunks, starting from the last run start
    // before it; groups are then compacted in chunk order, keyed
    // ((n64 - steps) << 14) | first chunk with steps = the 64-query steps
    // the group's keys can see (first chunk .. the largest hi64 / 64), and
    // sorted.
    // If that gives more groups starting before c_end (one past the last
    // chunk holding a real token) than dkdv_group_bound(c_end), the chunks
    // are grouped by four from chunk 0 instead, which bounds the dK/dV
    // launch (dkdv_workgroups).
    const int n64 = 2 * nb;
    const int gch = (n64 + nt - 1) / nt;
    const int ga = min(n64, t * gch), ge = min(n64, ga + gch);
    auto run_start = [&](int c) { return c == 0 || hi64[c - 1] != hi64[c]; };
    int last = -1, lreal = 0;
    for (int c = ga; c < ge; ++c) {
        if (run_start(c)) last = c;
        if (hi64[c] >= 0) lreal = c + 1;
    }
    __shared__ int s_cend;
    if (t == 0) s_cend = 0;
    int rs = block_exclusive_max(last, shi);  // (its barriers order s_cend's initialisation)
    if (lreal) atomicMax(&s_cend, lreal);
    __syncthreads();
    const int c_end = s_cend;
    int ng = 0, ngr = 0;
    for (int c = ga; c < ge; ++c) {
        if (run_start(c)) rs = c;
        const bool g = ((c - rs) & (kMaxGroupChunks - 1)) == 0;
        gflag[c] = g;
        ng += g;
        ngr += g && c < c_end;
    }
    long long ngt;
    block_exclusive_scan(ngr, sh, &ngt);
    if (ngt > dkdv_group_bound(c_end)) {
        ng = 0;
        for (int c = ga; c < ge; ++c) {
            const bool g = (c & (kMaxGroupChunks - 1)) == 0;
            gflag[c] = g;
            ng += g;
        }
    }
    const int gbase = int(block_exclusive_scan(ng, sh, &ngt));
    const int n_groups = int(ngt);
    __syncthreads();  // gflag complete (the fallback rewrote it)
    {
        int g = gbase;
        for (int c = ga; c < ge; ++c)
            if (gflag[c]) {
                int hi = hi64[c];  // the group's largest subtree end
                for (int e = c + 1; e < min(n64, c + kMaxGroupChunks) && !gflag[e]; ++e) hi = max(hi, hi64[e]);
                const int steps = hi >= 0 ? hi / kChunk - c + 1 : 0;
                kg[g++] = (unsigned(n64 - steps) << 14) | unsigned(c);
            }
    }
    int ngp = 1;
    while (ngp < n_groups) ngp <<= 1;
    for (int i = n_groups + t; i < ngp; i += nt) kg[i] = 0xffffffffu;
    __syncthreads();
    for (int k = 2; k <= ngp; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < ngp; i += nt) {
                const int p = i ^ j;
                if (p > i) {
                    const unsigned x = kg[i], y = kg[p];
                    if ((x > y) == ((i & k) == 0)) {
                        kg[i] = y;
                        kg[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int i = t; i < n_groups; i += nt) {
        const int c = int(kg[i] & 0x3fffu);
        int m = 1;
        while (m < kMaxGroupChunks && c + m < n64 && !gflag[c + m]) ++m;
        g_order[i] = c | ((m - 1) << 14);
    }
    if (t == 0) hdr[3] = n_groups;
}

// One workgroup (256 threads) per block b: the position ids of its tokens,
// row b's tile list (ascending key blocks) and column b's (closed form).
__global__ __launch_bounds__(256) void meta_lists(const int32_t* __restrict__ se, const int32_t* __restrict__ hist,
                                                  const int32_t* __restrict__ blk_min,
                                                  const int32_t* __restrict__ blk_max,
                                                  const int32_t* __restrict__ blk_roff,
                                                  const int32_t* __restrict__ blk_hoff,
                                                  const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_ptr, int32_t* __restrict__ pos,
                                                  int32_t* __restrict__ row_ent, int32_t* __restrict__ col_ent,
                                                  int L, int nb) {
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const unsigned long long below = (1ull << lane) - 1;
    __shared__ int sh[8];

    // 1) position ids: pos = (#real up to i, inclusive) - (histogram mass
    //    below i) - 1, from the block's exclusive prefixes plus a scan
    //    within the block (waves 0 and 1 hold its 128 tokens)
    if (t < kBlock) {
        const int i = b * kBlock + t;
        const int s = se[i];
        const int real = s >= 0 && s < L;
        const int hv = hist[i];
        int r = real, hx = hv;  // inclusive wave scans
        for (int off = 1; off < 64; off <<= 1) {
            const int ry = __shfl_up(r, off), hy = __shfl_up(hx, off);
            if (lane >= off) {
                r += ry;
                hx += hy;
            }
        }
        if (lane == 63) {
            sh[2 * wave] = r;
            sh[2 * wave + 1] = hx;
        }
        __syncthreads();
        const int r_in = r + (wave ? sh[0] : 0);
        const int h_ex = hx - hv + (wave ? sh[1] : 0);
        pos[i] = real ? blk_roff[b] + r_in - (blk_hoff[b] + h_ex) - 1 : 0;
    } else {
        __syncthreads();
    }

    // 2) row b: nonempty key blocks kb <= b in ascending order, 256 per pass
    {
        int k = row_ptr[b];
        for (int k0 = 0; k0 <= b; k0 += 256) {
            const int kb = k0 + t;
            const int c = kb <= b && kb < nb ? tile_class_of(b, kb, blk_min[kb], blk_max[kb]) : 0;
            const unsigned long long m = __ballot(c != 0);
            __syncthreads();  // sh reuse
            if (lane == 0) sh[wave] = __popcll(m);
            __syncthreads();
            int before = 0, tot = 0;
            for (int w = 0; w < 4; ++w) {
                before += w < wave ? sh[w] : 0;
                tot += sh[w];
            }
            if (c) row_ent[k + before + __popcll(m & below)] = (kb << 1) | (c == 1);
            k += tot;
        }
    }

    // 3) column b: query blocks b .. hi / 128
    {
        const int lo = blk_min[b], hi = blk_max[b];
        if (hi >= 0) {
            const int qmax = min(nb - 1, hi / kBlock), base = col_ptr[b];
            for (int qb = b + t; qb <= qmax; qb += 256) {
                const int c = tile_class_of(qb, b, lo, hi);
                col_ent[base + qb - b] = (qb << 1) | (c == 1);
            }
        }
    }
}

}  // namespace

hipError_t launch_meta(const int32_t* se, int64_t L, int32_t* pos, uint8_t* tile_class, void* ws,
                       hipStream_t stream) {
    const MetaLayout m = meta_layout(L);
    int32_t* w = static_cast<int32_t*>(ws);
    const int nb = int(m.nb);
    meta_init<<<64, 256, 0, stream>>>(w + m.hist, L + 1, w + m.hdr, L, nb);
    meta_blocks<<<nb, kBlock, 0, stream>>>(se, w + m.hist, w + m.blk_min, w + m.blk_max, w + m.blk_cnt, w + m.hdr,
                                          w + m.hi64, int(L));
    meta_tiles<<<nb, 256, 0, stream>>>(w + m.blk_min, w + m.blk_max, w + m.hist, tile_class, w + m.row_cnt,
                                      w + m.blk_hsum, nb);
    meta_scan<<<1, 1024, 0, stream>>>(w + m.blk_max, w + m.blk_cnt, w + m.blk_hsum, w + m.row_cnt, w + m.col_cnt,
                                     w + m.row_ptr, w + m.col_ptr, w + m.q_order, w + m.k_order, w + m.hi64,
                                     w + m.g_order, w + m.hdr, nb);
    meta_lists<<<nb, 256, 0, stream>>>(se, w + m.hist, w + m.blk_min, w + m.blk_max, w + m.blk_cnt, w + m.blk_hsum,
                                      w + m.row_ptr, w + m.col_ptr, pos, w + m.row_ent, w + m.col_ent, int(L), nb);
    return hipGetLastError();
}

}  // namespace treeattn
