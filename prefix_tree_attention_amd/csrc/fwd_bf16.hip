// Forward tree attention, bf16 in / fp32 accumulate, gfx950 MFMA.
//
// What it computes (AReaL tree-training guide, packing figure: a token
// attends to itself and its ancestors only; key j is visible to query i iff
// j <= i <= se[j] in the pre-order layout):
//   O_i = sum_{j in A(i)} softmax_j(scale q_i.k_j) v_j,
//   LSE_i = ln sum_{j in A(i)} exp(scale q_i.k_j).
//
// Work decomposition: one workgroup (4 waves) per (128-query block, query
// head); wave w owns queries 32w..32w+31 of the block as two 16-column MFMA
// groups.  The workgroup walks only the nonempty key tiles of its query
// block (row list of the metadata), 64 keys per pipeline step, with K and
// V^T staged through double-buffered LDS.  Partial tiles apply the
// subtree-interval predicate; full tiles skip it.
//
// Products are computed transposed: S^T = K Q^T (A = K rows from LDS, B =
// Q^T held in registers), O^T = V^T P^T (A = V^T rows from LDS, B = P^T
// taken straight from the S^T accumulators).  Each lane thus owns one query
// column, so softmax statistics need only an in-lane reduction plus two
// cross-lane steps, and the rescaling of O^T is per lane.  For the S^T
// accumulators to be usable as the P^T operand, MFMA row (16b + m) of a
// 64-key step holds key 32c + 8(m/4) + 4e + (m%4) with b = 2c + e; K is
// written to LDS in that row order.  Softmax runs in base 2 with
// scale*log2(e) folded into the scores.

#include <cmath>

#include "device.h"
#include "mfma.h"

namespace treeattn {
namespace {

constexpr int kThreads = 256;
constexpr int kStep = 64;  // keys per pipeline step

// LDS row of key (0..63) within a step, see the file comment.
__device__ __forceinline__ int k_lds_row(int key) {
    const int c = key >> 5, w = key & 31;
    return 16 * (2 * c + ((w >> 2) & 1)) + 4 * (w >> 3) + (w & 3);
}

template <int D>
struct FwdSmem {
    bf16 k[2][kStep][D + 8];   // +16 B per row: conflict-free 16-byte row reads
    bf16 vt[2][D][kStep + 8];  // V transposed: [d][key]
};

template <int D>
struct FwdPrefetch {
    static constexpr int kItems = kStep * (D / 8) / kThreads;  // 16-byte K chunks per thread
    u32x4 k[kItems];
    u32x4 v[4];  // 4 consecutive keys x 8 d of V
};

template <int D>
__device__ __forceinline__ void fwd_load(FwdPrefetch<D>& pf, const bf16* __restrict__ K,
                                         const bf16* __restrict__ V, int64_t tok_stride, int hoff,
                                         int kbase, int tid) {
#pragma unroll
    for (int i = 0; i < FwdPrefetch<D>::kItems; ++i) {
        const int it = tid + kThreads * i;
        const int key = it / (D / 8), ch = it % (D / 8);
        pf.k[i] = ld16(K + int64_t(kbase + key) * tok_stride + hoff + 8 * ch);
    }
    if (tid < 2 * D) {
        const int kg = tid & 15, ch = tid >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) pf.v[r] = ld16(V + int64_t(kbase + 4 * kg + r) * tok_stride + hoff + 8 * ch);
    }
}

template <int D>
__device__ __forceinline__ void fwd_store(const FwdPrefetch<D>& pf, FwdSmem<D>& sm, int buf, int tid) {
#pragma unroll
    for (int i = 0; i < FwdPrefetch<D>::kItems; ++i) {
        const int it = tid + kThreads * i;
        const int key = it / (D / 8), ch = it % (D / 8);
        st16(&sm.k[buf][k_lds_row(key)][8 * ch], pf.k[i]);
    }
    if (tid < 2 * D) {
        const int kg = tid & 15, ch = tid >> 4;
        u32x2 cols[8];
        transpose4x8(pf.v, cols);
#pragma unroll
        for (int j = 0; j < 8; ++j) st8(&sm.vt[buf][8 * ch + j][4 * kg], cols[j]);
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ se,
    const int32_t* __restrict__ q_order, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv, float scale_log2) {
    constexpr int NS = D / 32;  // k-steps of QK^T
    constexpr int NT = D / 16;  // d-blocks of O^T
    __shared__ FwdSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int rank = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int qb = q_order[rank];
    const int hkv = h / (Hq / Hkv);
    const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;
    const int hoff = hkv * D;
    const int qrow0 = qb * kBlock + 32 * wave;  // first query of this wave

    // Q^T operand: lane holds query (qrow0 + 16 qs + n), d = 32 s + 8 g .. +7
    bf16x8 qf[2][NS];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int s = 0; s < NS; ++s)
            qf[qs][s] = __builtin_bit_cast(
                bf16x8, ld16(Q + int64_t(qrow0 + 16 * qs + n) * q_stride + int64_t(h) * D + 32 * s + 8 * g));

    f32x4 oacc[2][NT];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int t = 0; t < NT; ++t) oacc[qs][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    const int beg = row_ptr[qb], nsteps = 2 * (row_ptr[qb + 1] - beg);
    FwdPrefetch<D> pf;
    if (nsteps > 0) {
        fwd_load<D>(pf, K, V, kv_stride, hoff, (row_ent[beg] >> 1) * kBlock, tid);
        fwd_store<D>(pf, sm, 0, tid);
    }
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        const int ent = row_ent[beg + (st >> 1)];
        const int kbase = (ent >> 1) * kBlock + kStep * (st & 1);
        const bool partial = ent & 1;
        if (st + 1 < nsteps) {
            const int ent1 = row_ent[beg + ((st + 1) >> 1)];
            fwd_load<D>(pf, K, V, kv_stride, hoff, (ent1 >> 1) * kBlock + kStep * ((st + 1) & 1), tid);
        }

        // S^T = K Q^T, 4 key blocks of 16 x 2 query groups of 16
        f32x4 sc[2][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 a[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s)
                a[s] = *reinterpret_cast<const bf16x8*>(&sm.k[buf][16 * b + n][32 * s + 8 * g]);
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s) c = mfma16x16x32(a[s], qf[qs][s], c);
                sc[qs][b] = c * scale_log2;
            }
        }

        if (partial) {
            // lane's keys: kbase + 32 c + 8 g + 0..7 for c = 0, 1
            i32x4 sek[2][2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                sek[c][0] = *reinterpret_cast<const i32x4*>(se + kbase + 32 * c + 8 * g);
                sek[c][1] = *reinterpret_cast<const i32x4*>(se + kbase + 32 * c + 8 * g + 4);
            }
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
                const int qi = qrow0 + 16 * qs + n;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kbase + 32 * (b >> 1) + 8 * g + 4 * (b & 1) + r;
                        const int sej = sek[b >> 1][b & 1][r];
                        if (!(key <= qi && qi <= sej)) sc[qs][b][r] = -INFINITY;
                    }
            }
        }

        // online softmax (base 2), one query column per lane
        bf16x8 pb[2][2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            float mx = -INFINITY;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[qs][b][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m_run[qs], mx);
            const float muse = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = fast_exp2(m_run[qs] - muse);
            float rs = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(sc[qs][b][r] - muse);
                    sc[qs][b][r] = p;
                    rs += p;
                }
            l_run[qs] = l_run[qs] * alpha + rs;
            m_run[qs] = mnew;
#pragma unroll
            for (int t = 0; t < NT; ++t) oacc[qs][t] *= alpha;
            pb[qs][0] = to_bf16x8(sc[qs][0], sc[qs][1]);
            pb[qs][1] = to_bf16x8(sc[qs][2], sc[qs][3]);
        }

        // O^T += V^T P^T, 2 key steps of 32 x NT d blocks of 16
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.vt[buf][16 * t + n][32 * c + 8 * g]);
#pragma unroll
                for (int qs = 0; qs < 2; ++qs) oacc[qs][t] = mfma16x16x32(a, pb[qs][c], oacc[qs][t]);
            }

        if (st + 1 < nsteps) fwd_store<D>(pf, sm, buf ^ 1, tid);
        __syncthreads();
    }

    // epilogue: normalise, write O (bf16) and LSE (natural log)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        float l = l_run[qs];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int qi = qrow0 + 16 * qs + n;
        bf16* orow = O + int64_t(qi) * q_stride + int64_t(h) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const f32x4 v = oacc[qs][t] * inv;
            st8(orow + 16 * t + 4 * g, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
        }
        if (g == 0) LSE[int64_t(h) * L + qi] = l > 0.f ? (m_run[qs] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int32_t* se, const MetaPtrs& mp, const AttnShape& sh,
                           hipStream_t stream) {
    const dim3 grid(unsigned(sh.nb) * unsigned(sh.Hq));
    const float sl2 = sh.scale * 1.4426950408889634f;
    const auto* Q = static_cast<const bf16*>(q);
    const auto* K = static_cast<const bf16*>(k);
    const auto* V = static_cast<const bf16*>(v);
    auto* O = static_cast<bf16*>(o);
    if (sh.D == 128)
        fwd_bf16_kernel<128><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, mp.q_order, mp.row_ptr,
                                                             mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2);
    else if (sh.D == 64)
        fwd_bf16_kernel<64><<<grid, kThreads, 0, stream>>>(Q, K, V, O, lse, se, mp.q_order, mp.row_ptr,
                                                            mp.row_ent, int(sh.L), sh.Hq, sh.Hkv, sl2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace treeattn
