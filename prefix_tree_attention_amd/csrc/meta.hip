// Metadata kernels of libtreeattn (tree_meta): position ids, 128x128 tile
// classes and the tile lists of the attention kernels, all derived from the
// per-token subtree ends se[L] in O(L + nb^2) work.
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
// are exact, not conservative.

#include "device.h"

namespace treeattn {
namespace {

__global__ void meta_init(int32_t* __restrict__ hist, int64_t n_hist, int32_t* __restrict__ col_cnt,
                          int nb, int32_t* __restrict__ hdr, int64_t L) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n_hist; i += stride) hist[i] = 0;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nb; i += stride) col_cnt[i] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr[0] = int32_t(L);
        hdr[1] = nb;
        hdr[2] = 0;
    }
}

// One workgroup per 128-token block: histogram of subtree ends and the
// block's min / max subtree end.
__global__ __launch_bounds__(128) void meta_blocks(const int32_t* __restrict__ se, int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ blk_min, int32_t* __restrict__ blk_max,
                                                   int32_t* __restrict__ hdr, int L) {
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
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        blk_min[b] = min(smn[0], smn[1]);
        blk_max[b] = max(smx[0], smx[1]);
        if (sreal[0] + sreal[1]) atomicAdd(&hdr[2], sreal[0] + sreal[1]);
    }
}

// One workgroup per query block: the class of every tile of its row, the
// row's nonempty count, and per-column nonempty counts.
__global__ __launch_bounds__(256) void meta_tiles(const int32_t* __restrict__ blk_min,
                                                  const int32_t* __restrict__ blk_max,
                                                  uint8_t* __restrict__ tc, int32_t* __restrict__ row_cnt,
                                                  int32_t* __restrict__ col_cnt, int nb) {
    const int qb = blockIdx.x;
    const int qlo = qb * kBlock, qhi = qb * kBlock + kBlock - 1;
    int cnt = 0;
    for (int kb = threadIdx.x; kb < nb; kb += blockDim.x) {
        int c;
        if (kb > qb)
            c = 0;
        else if (kb == qb)
            c = blk_max[kb] >= 0 ? 1 : 0;
        else {
            const int lo = blk_min[kb], hi = blk_max[kb];
            c = hi < qlo ? 0 : (lo >= qhi ? 2 : 1);
        }
        tc[int64_t(qb) * nb + kb] = uint8_t(c);
        if (c) {
            ++cnt;
            atomicAdd(&col_cnt[kb], 1);
        }
    }
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    __shared__ int part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) row_cnt[qb] = part[0] + part[1] + part[2] + part[3];
}

// Exclusive scan of one value per thread across a 1024-thread workgroup.
// Returns the exclusive prefix; *total receives the sum.  Uses `sh` (>= 16
// ints of shared memory).
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

// Single workgroup: position ids, CSR pointers and entries, heaviest-first
// orders.
__global__ __launch_bounds__(1024) void meta_finish(const int32_t* __restrict__ se,
                                                    const int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ pos, const uint8_t* __restrict__ tc,
                                                    const int32_t* __restrict__ row_cnt,
                                                    int32_t* __restrict__ row_ptr, int32_t* __restrict__ row_ent,
                                                    const int32_t* __restrict__ col_cnt,
                                                    int32_t* __restrict__ col_ptr, int32_t* __restrict__ col_ent,
                                                    int32_t* __restrict__ q_order, int32_t* __restrict__ k_order,
                                                    int L, int nb) {
    __shared__ long long sh[32];
    const int t = threadIdx.x, nt = blockDim.x;
    long long total;

    // 1) position ids
    {
        const int chunk = (L + nt - 1) / nt;
        const int a = min(L, t * chunk), b = min(L, a + chunk);
        long long lt = 0, re = 0;
        for (int i = a; i < b; ++i) {
            lt += hist[i];
            re += se[i] >= 0 && se[i] < L;
        }
        // pack the two counts (each < 2^21) into one scan value
        const long long base = block_exclusive_scan((lt << 32) | re, sh, &total);
        long long run_lt = base >> 32, run_re = base & 0xffffffffll;
        for (int i = a; i < b; ++i) {
            const bool real = se[i] >= 0 && se[i] < L;
            run_re += real;
            pos[i] = real ? int32_t(run_re - run_lt - 1) : 0;
            run_lt += hist[i];
        }
    }

    // 2) CSR offsets
    {
        const int chunk = (nb + nt - 1) / nt;
        const int a = min(nb, t * chunk), b = min(nb, a + chunk);
        long long r = 0, c = 0;
        for (int i = a; i < b; ++i) {
            r += row_cnt[i];
            c += col_cnt[i];
        }
        const long long base = block_exclusive_scan((r << 32) | c, sh, &total);
        long long rr = base >> 32, cc = base & 0xffffffffll;
        for (int i = a; i < b; ++i) {
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
    __syncthreads();

    // 3) entries, ascending: one wave per row (column), 64 tiles per ballot,
    //    each nonempty tile written at its rank among the nonempty ones
    const int lane = t & 63, wv = t >> 6, nw = nt >> 6;
    const unsigned long long below = (1ull << lane) - 1;
    for (int qb = wv; qb < nb; qb += nw) {
        int k = row_ptr[qb];
        const uint8_t* row = tc + int64_t(qb) * nb;
        for (int k0 = 0; k0 <= qb; k0 += 64) {
            const int kb = k0 + lane;
            const int c = kb <= qb ? row[kb] : 0;
            const unsigned long long m = __ballot(c != 0);
            if (c) row_ent[k + __popcll(m & below)] = (kb << 1) | (c == 1);
            k += __popcll(m);
        }
    }
    for (int kb = wv; kb < nb; kb += nw) {
        int k = col_ptr[kb];
        for (int q0 = kb; q0 < nb; q0 += 64) {
            const int qb = q0 + lane;
            const int c = qb < nb ? tc[int64_t(qb) * nb + kb] : 0;
            const unsigned long long m = __ballot(c != 0);
            if (c) col_ent[k + __popcll(m & below)] = (qb << 1) | (c == 1);
            k += __popcll(m);
        }
    }

    // 4) heaviest-first orders (stable on index), counts staged in LDS
    __shared__ int rc_s[kMaxL / kBlock], cc_s[kMaxL / kBlock];
    for (int i = t; i < nb; i += nt) {
        rc_s[i] = row_cnt[i];
        cc_s[i] = col_cnt[i];
    }
    __syncthreads();
    for (int x = t; x < nb; x += nt) {
        const int rc = rc_s[x], cc = cc_s[x];
        int rq = 0, rk = 0;
        for (int y = 0; y < nb; ++y) {
            const int ry = rc_s[y], cy = cc_s[y];
            rq += (ry > rc) || (ry == rc && y < x);
            rk += (cy > cc) || (cy == cc && y < x);
        }
        q_order[rq] = x;
        k_order[rk] = x;
    }
}

}  // namespace

hipError_t launch_meta(const int32_t* se, int64_t L, int32_t* pos, uint8_t* tile_class, void* ws,
                       hipStream_t stream) {
    const MetaLayout m = meta_layout(L);
    int32_t* w = static_cast<int32_t*>(ws);
    const int nb = int(m.nb);
    meta_init<<<64, 256, 0, stream>>>(w + m.hist, L + 1, w + m.col_cnt, nb, w + m.hdr, L);
    meta_blocks<<<nb, kBlock, 0, stream>>>(se, w + m.hist, w + m.blk_min, w + m.blk_max, w + m.hdr, int(L));
    meta_tiles<<<nb, 256, 0, stream>>>(w + m.blk_min, w + m.blk_max, tile_class, w + m.row_cnt,
                                      w + m.col_cnt, nb);
    meta_finish<<<1, 1024, 0, stream>>>(se, w + m.hist, pos, tile_class, w + m.row_cnt, w + m.row_ptr,
                                       w + m.row_ent, w + m.col_cnt, w + m.col_ptr, w + m.col_ent,
                                       w + m.q_order, w + m.k_order, int(L), nb);
    return hipGetLastError();
}

}  // namespace treeattn
