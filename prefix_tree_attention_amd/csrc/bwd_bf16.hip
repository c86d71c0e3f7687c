// Backward tree attention, bf16 in / fp32 accumulate, gfx950 MFMA.
//
// With P = softmax of the visible scores (recomputed from LSE) and
// Delta_i = dO_i . O_i:
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - Delta_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,
// summed, for dK / dV, over the query heads sharing a key/value head.  A
// shared prefix token is a single key column, so its gradient is the sum
// over every sequence below it (AREAL-DTA notes, §3 问题形式化) with no
// extra work.
//
// Three kernels:
//   delta: Delta for every (token, query head).
//   dkdv:  one workgroup per (128-key block, key/value head); wave w owns
//          keys 32w..32w+31 and keeps K, V, dK^T, dV^T in registers.  It
//          walks the nonempty tiles of its key block (column list) for each
//          query head of the group, 64 queries per step, with Q, dO (rows
//          permuted for the score products) and Q^T, dO^T (for the
//          gradient products) staged in double-buffered LDS.
//            S = Q K^T, dP = dO V^T   (A = Q / dO rows, B = K^T / V^T regs)
//            dV^T += dO^T P, dK^T += Q^T dS   (A = dO^T / Q^T rows, B = P / dS
//            straight from the score accumulators)
//   dq:    one workgroup per (128-query block, query head) like the forward:
//            S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.
// The row permutation that lets a score accumulator serve directly as the
// next product's operand is the forward's: MFMA row 16b + m of a 64-row
// step holds token 32c + 8(m/4) + 4e + (m%4), b = 2c + e.

#include <cmath>

#include "device.h"
#include "mfma.h"

namespace treeattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int perm_row(int tok) {
    const int c = tok >> 5, w = tok & 31;
    return 16 * (2 * c + ((w >> 2) & 1)) + 4 * (w >> 3) + (w & 3);
}

// ---------------------------------------------------------------------------
// staging helpers: a 64-row x D tile of a [token][head][D] tensor
// ---------------------------------------------------------------------------
// "Quad" pattern: thread (qg = tid % 16, ch = tid / 16) loads rows 4qg..4qg+3
// at d-chunk ch; it can write the rows (permuted) and the transpose.
template <int D>
struct Quad {
    u32x4 r[4];
};

template <int D>
__device__ __forceinline__ void quad_load(Quad<D>& x, const bf16* __restrict__ base, int64_t tok_stride, int row0,
                                          int tid) {
    if (tid < 2 * D) {
        const int qg = tid & 15, ch = tid >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) x.r[r] = ld16(base + int64_t(row0 + 4 * qg + r) * tok_stride + 8 * ch);
    }
}

template <int D>
__device__ __forceinline__ void quad_store_rows(const Quad<D>& x, bf16 (*rows)[D + 8], int tid) {
    if (tid < 2 * D) {
        const int qg = tid & 15, ch = tid >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) st16(&rows[perm_row(4 * qg + r)][8 * ch], x.r[r]);
    }
}

template <int D>
__device__ __forceinline__ void quad_store_t(const Quad<D>& x, bf16 (*cols)[kStep + 8], int tid) {
    if (tid < 2 * D) {
        const int qg = tid & 15, ch = tid >> 4;
        u32x2 t[8];
        transpose4x8(x.r, t);
#pragma unroll
        for (int j = 0; j < 8; ++j) st8(&cols[8 * ch + j][4 * qg], t[j]);
    }
}

// "Flat" pattern: 16-byte chunks, consecutive threads along a row.
template <int D>
struct Flat {
    static constexpr int kItems = kStep * (D / 8) / kThreads;
    u32x4 r[kItems];
};

template <int D>
__device__ __forceinline__ void flat_load(Flat<D>& x, const bf16* __restrict__ base, int64_t tok_stride, int row0,
                                          int tid) {
#pragma unroll
    for (int i = 0; i < Flat<D>::kItems; ++i) {
        const int it = tid + kThreads * i;
        x.r[i] = ld16(base + int64_t(row0 + it / (D / 8)) * tok_stride + 8 * (it % (D / 8)));
    }
}

template <int D>
__device__ __forceinline__ void flat_store_rows(const Flat<D>& x, bf16 (*rows)[D + 8], int tid) {
#pragma unroll
    for (int i = 0; i < Flat<D>::kItems; ++i) {
        const int it = tid + kThreads * i;
        st16(&rows[perm_row(it / (D / 8))][8 * (it % (D / 8))], x.r[i]);
    }
}

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_bf16_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                         float* __restrict__ delta, int L, int Hq) {
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= int64_t(L) * Hq) return;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const u32x4 a = ld16(O + r * D + 8 * c), b = ld16(dO + r * D + 8 * c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += bf16_to_float(a[w] & 0xffffu) * bf16_to_float(b[w] & 0xffffu);
            acc += bf16_to_float(a[w] >> 16) * bf16_to_float(b[w] >> 16);
        }
    }
    delta[int64_t(r % Hq) * L + r / Hq] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct DkvSmem {
    bf16 q[2][kStep][D + 8];
    bf16 g[2][kStep][D + 8];
    bf16 qt[2][D][kStep + 8];
    bf16 gt[2][D][kStep + 8];
    float lse2[2][kStep];
    float dl[2][kStep];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dkdv_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, const int32_t* __restrict__ se,
    const int32_t* __restrict__ k_order, const int32_t* __restrict__ col_ptr,
    const int32_t* __restrict__ col_ent, int L, int Hq, int Hkv, float scale_log2, float scale) {
    constexpr int NS = D / 32, NT = D / 16;
    __shared__ DkvSmem<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int rank = blockIdx.x / Hkv, hkv = blockIdx.x % Hkv;
    const int kb = k_order[rank];
    const int G = Hq / Hkv;
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int kw0 = kb * kBlock + 32 * wave;

    // K^T, V^T operands of this wave's 32 keys: lane holds key (kw0 + 16 ks + n)
    bf16x8 kf[2][NS], vf[2][NS];
    int sek[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int key = kw0 + 16 * ks + n;
        sek[ks] = se[key];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kf[ks][s] = __builtin_bit_cast(bf16x8, ld16(K + int64_t(key) * kv_stride + hkv * D + 32 * s + 8 * g));
            vf[ks][s] = __builtin_bit_cast(bf16x8, ld16(V + int64_t(key) * kv_stride + hkv * D + 32 * s + 8 * g));
        }
    }
    f32x4 dk[2][NT], dv[2][NT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int t = 0; t < NT; ++t) dk[ks][t] = dv[ks][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int beg = col_ptr[kb], nsteps = (col_ptr[kb + 1] - beg) * 2 * G;
    // step st: tile col_ent[beg + st / 2G], query half (st / G) % 2, head hkv G + st % G
    Quad<D> pq, pg;
    float plse = 0.f, pdl = 0.f;
    auto load = [&](int st) {
        const int ent = col_ent[beg + st / (2 * G)];
        const int qbase = (ent >> 1) * kBlock + kStep * ((st / G) & 1);
        const int h = hkv * G + st % G;
        quad_load<D>(pq, Q + int64_t(h) * D, q_stride, qbase, tid);
        quad_load<D>(pg, dO + int64_t(h) * D, q_stride, qbase, tid);
        if (tid < kStep) {
            plse = LSE[int64_t(h) * L + qbase + tid] * kLog2e;
            pdl = Delta[int64_t(h) * L + qbase + tid];
        }
    };
    auto store = [&](int buf) {
        quad_store_rows<D>(pq, sm.q[buf], tid);
        quad_store_rows<D>(pg, sm.g[buf], tid);
        quad_store_t<D>(pq, sm.qt[buf], tid);
        quad_store_t<D>(pg, sm.gt[buf], tid);
        if (tid < kStep) {
            sm.lse2[buf][tid] = plse;
            sm.dl[buf][tid] = pdl;
        }
    };
    if (nsteps > 0) {
        load(0);
        store(0);
    }
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int ent = col_ent[beg + st / (2 * G)];
        const int qbase = (ent >> 1) * kBlock + kStep * ((st / G) & 1);
        const bool partial = ent & 1;
        if (st + 1 < nsteps) load(st + 1);

        f32x4 s[2][4], dp[2][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 aq[NS], ag[NS];
#pragma unroll
            for (int x = 0; x < NS; ++x) {
                aq[x] = *reinterpret_cast<const bf16x8*>(&sm.q[buf][16 * b + n][32 * x + 8 * g]);
                ag[x] = *reinterpret_cast<const bf16x8*>(&sm.g[buf][16 * b + n][32 * x + 8 * g]);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f32x4 cs = {0.f, 0.f, 0.f, 0.f}, cd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < NS; ++x) {
                    cs = mfma16x16x32(aq[x], kf[ks][x], cs);
                    cd = mfma16x16x32(ag[x], vf[ks][x], cd);
                }
                s[ks][b] = cs;
                dp[ks][b] = cd;
            }
        }
        // lane's queries for block b = 2c + e: qbase + 32c + 8g + 4e + 0..3
        f32x4 l2[2][2], dl[2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                l2[c][e] = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][32 * c + 8 * g + 4 * e]);
                dl[c][e] = *reinterpret_cast<const f32x4*>(&sm.dl[buf][32 * c + 8 * g + 4 * e]);
            }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int key = kw0 + 16 * ks + n;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float p = fast_exp2(s[ks][b][r] * scale_log2 - l2[b >> 1][b & 1][r]);
                    if (partial) {
                        const int qi = qbase + 32 * (b >> 1) + 8 * g + 4 * (b & 1) + r;
                        p = (key <= qi && qi <= sek[ks]) ? p : 0.f;
                    }
                    s[ks][b][r] = p;
                    dp[ks][b][r] = p * (dp[ks][b][r] - dl[b >> 1][b & 1][r]);
                }
        }
        bf16x8 pb[2][2], db[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                pb[ks][c] = to_bf16x8(s[ks][2 * c], s[ks][2 * c + 1]);
                db[ks][c] = to_bf16x8(dp[ks][2 * c], dp[ks][2 * c + 1]);
            }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 ag = *reinterpret_cast<const bf16x8*>(&sm.gt[buf][16 * t + n][32 * c + 8 * g]);
                const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.qt[buf][16 * t + n][32 * c + 8 * g]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    dv[ks][t] = mfma16x16x32(ag, pb[ks][c], dv[ks][t]);
                    dk[ks][t] = mfma16x16x32(aq, db[ks][c], dk[ks][t]);
                }
            }

        if (st + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }

    // lane holds key (kw0 + 16 ks + n), d = 16 t + 4 g .. +3
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int64_t off = int64_t(kw0 + 16 * ks + n) * kv_stride + hkv * D + 4 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 a = dk[ks][t] * scale, b = dv[ks][t];
            st8(dK + off + 16 * t, u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
            st8(dV + off + 16 * t, u32x2{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
        }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct DqSmem {
    bf16 k[2][kStep][D + 8];
    bf16 v[2][kStep][D + 8];
    bf16 kt[2][D][kStep + 8];
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void dq_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dQ, const int32_t* __restrict__ se, const int32_t* __restrict__ q_order,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv,
    float scale_log2, float scale) {
    constexpr int NS = D / 32, NT = D / 16;
    __shared__ DqSmem<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int rank = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int qb = q_order[rank];
    const int hkv = h / (Hq / Hkv);
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int qrow0 = qb * kBlock + 32 * wave;

    bf16x8 qf[2][NS], gf[2][NS];
    float lse2[2], dlt[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const int qi = qrow0 + 16 * qs + n;
        lse2[qs] = LSE[int64_t(h) * L + qi] * kLog2e;
        dlt[qs] = Delta[int64_t(h) * L + qi];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qf[qs][s] = __builtin_bit_cast(bf16x8, ld16(Q + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
            gf[qs][s] = __builtin_bit_cast(bf16x8, ld16(dO + int64_t(qi) * q_stride + int64_t(h) * D + 32 * s + 8 * g));
        }
    }
    f32x4 dq[2][NT];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < NT; ++t) dq[qs][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int beg = row_ptr[qb], nsteps = 2 * (row_ptr[qb + 1] - beg);
    Quad<D> pk;
    Flat<D> pv;
    auto load = [&](int st) {
        const int kbase = (row_ent[beg + (st >> 1)] >> 1) * kBlock + kStep * (st & 1);
        quad_load<D>(pk, K + hkv * D, kv_stride, kbase, tid);
        flat_load<D>(pv, V + hkv * D, kv_stride, kbase, tid);
    };
    auto store = [&](int buf) {
        quad_store_rows<D>(pk, sm.k[buf], tid);
        quad_store_t<D>(pk, sm.kt[buf], tid);
        flat_store_rows<D>(pv, sm.v[buf], tid);
    };
    if (nsteps > 0) {
        load(0);
        store(0);
    }
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int ent = row_ent[beg + (st >> 1)];
        const int kbase = (ent >> 1) * kBlock + kStep * (st & 1);
        const bool partial = ent & 1;
        if (st + 1 < nsteps) load(st + 1);

        f32x4 s[2][4], dp[2][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 ak[NS], av[NS];
#pragma unroll
            for (int x = 0; x < NS; ++x) {
                ak[x] = *reinterpret_cast<const bf16x8*>(&sm.k[buf][16 * b + n][32 * x + 8 * g]);
                av[x] = *reinterpret_cast<const bf16x8*>(&sm.v[buf][16 * b + n][32 * x + 8 * g]);
            }
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                f32x4 cs = {0.f, 0.f, 0.f, 0.f}, cd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < NS; ++x) {
                    cs = mfma16x16x32(ak[x], qf[qs][x], cs);
                    cd = mfma16x16x32(av[x], gf[qs][x], cd);
                }
                s[qs][b] = cs;
                dp[qs][b] = cd;
            }
        }
        i32x4 sek[2][2];
        if (partial) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                sek[c][0] = *reinterpret_cast<const i32x4*>(se + kbase + 32 * c + 8 * g);
                sek[c][1] = *reinterpret_cast<const i32x4*>(se + kbase + 32 * c + 8 * g + 4);
            }
        }
        bf16x8 db[2][2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            const int qi = qrow0 + 16 * qs + n;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float p = fast_exp2(s[qs][b][r] * scale_log2 - lse2[qs]);
                    if (partial) {
                        const int key = kbase + 32 * (b >> 1) + 8 * g + 4 * (b & 1) + r;
                        p = (key <= qi && qi <= sek[b >> 1][b & 1][r]) ? p : 0.f;
                    }
                    dp[qs][b][r] = p * (dp[qs][b][r] - dlt[qs]);
                }
            db[qs][0] = to_bf16x8(dp[qs][0], dp[qs][1]);
            db[qs][1] = to_bf16x8(dp[qs][2], dp[qs][3]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.kt[buf][16 * t + n][32 * c + 8 * g]);
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) dq[qs][t] = mfma16x16x32(a, db[qs][c], dq[qs][t]);
            }

        if (st + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        bf16* row = dQ + int64_t(qrow0 + 16 * qs + n) * q_stride + int64_t(h) * D + 4 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 a = dq[qs][t] * scale;
            st8(row + 16 * t, u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
        }
    }
}

template <int D>
hipError_t launch_bwd_d(int phase, const bf16* Q, const bf16* K, const bf16* V, const bf16* O, const float* lse,
                        const bf16* dO, bf16* dQ, bf16* dK, bf16* dV, const int32_t* se, const MetaPtrs& mp,
                        float* delta, const AttnShape& sh, hipStream_t stream) {
    const int L = int(sh.L);
    const int64_t rows = int64_t(L) * sh.Hq;
    const float sl2 = sh.scale * kLog2e;
    if (phase == kPhaseAll || phase == kPhaseDelta)
        delta_bf16_kernel<D><<<unsigned((rows + 255) / 256), 256, 0, stream>>>(O, dO, delta, L, sh.Hq);
    if (phase == kPhaseAll || phase == kPhaseDkdv)
        dkdv_bf16_kernel<D><<<unsigned(sh.nb) * unsigned(sh.Hkv), kThreads, 0, stream>>>(
            Q, K, V, dO, lse, delta, dK, dV, se, mp.k_order, mp.col_ptr, mp.col_ent, L, sh.Hq, sh.Hkv, sl2,
            sh.scale);
    if (phase == kPhaseAll || phase == kPhaseDq)
        dq_bf16_kernel<D><<<unsigned(sh.nb) * unsigned(sh.Hq), kThreads, 0, stream>>>(
            Q, K, V, dO, lse, delta, dQ, se, mp.q_order, mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv, sl2, sh.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(int phase, const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, const int32_t* se, const MetaPtrs& mp,
                           float* delta, const AttnShape& sh, hipStream_t stream) {
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    const auto* O = static_cast<const bf16*>(o);
    const auto* G = static_cast<const bf16*>(dout);
    auto* dQ = static_cast<bf16*>(dq);
    auto* dK = static_cast<bf16*>(dk);
    auto* dV = static_cast<bf16*>(dv);
    if (sh.D == 128) return launch_bwd_d<128>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream);
    if (sh.D == 64) return launch_bwd_d<64>(phase, Q, K, V, O, lse, G, dQ, dK, dV, se, mp, delta, sh, stream);
    return hipErrorInvalidValue;
}

}  // namespace treeattn
