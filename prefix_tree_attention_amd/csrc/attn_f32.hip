// fp32 check mode of the tree-attention forward and backward.
//
// Same mathematics and the same metadata (tile lists, subtree-interval
// predicate) as the bf16 MFMA path, in plain fp32 arithmetic with one
// thread per query row (forward, dQ) or key row (dK, dV) and 32-row chunks
// of the other operand staged through LDS.  Written for clarity, not speed:
// it exists so the tile walk can be checked against the oracle at a tight
// tolerance.  Natural-base softmax; scale applied to the scores.

#include <cmath>

#include "device.h"

namespace treeattn {
namespace {

constexpr int kRows = 64;   // rows per workgroup (one thread each)
constexpr int kChunk = 32;  // staged rows of the other operand

template <int D>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, float* __restrict__ O,
                                                        float* __restrict__ LSE, const int32_t* __restrict__ se,
                                                        const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ row_ent, int L, int Hq,
                                                        int Hkv, float scale) {
    __shared__ float ks[kChunk][D + 1], vs[kChunk][D + 1];
    __shared__ int ses[kChunk];
    const int h = blockIdx.y, qb = blockIdx.x >> 1;
    const int qi = qb * kBlock + (blockIdx.x & 1) * kRows + threadIdx.x;
    const int hkv = h / (Hq / Hkv);
    const int64_t qs = int64_t(Hq) * D, kvs = int64_t(Hkv) * D;
    float q[D], o[D];
    for (int d = 0; d < D; ++d) {
        q[d] = Q[qi * qs + h * D + d] * scale;
        o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int e = row_ptr[qb]; e < row_ptr[qb + 1]; ++e) {
        const int kb = row_ent[e] >> 1;
        const bool partial = row_ent[e] & 1;
        for (int c = 0; c < kBlock / kChunk; ++c) {
            const int k0 = kb * kBlock + c * kChunk;
            __syncthreads();
            for (int idx = threadIdx.x; idx < kChunk * D; idx += kRows) {
                const int r = idx / D, d = idx % D;
                ks[r][d] = K[(k0 + r) * kvs + hkv * D + d];
                vs[r][d] = V[(k0 + r) * kvs + hkv * D + d];
            }
            if (threadIdx.x < kChunk) ses[threadIdx.x] = se[k0 + threadIdx.x];
            __syncthreads();
            for (int j = 0; j < kChunk; ++j) {
                const int key = k0 + j;
                if (partial && !(key <= qi && qi <= ses[j])) continue;
                float s = 0.f;
                for (int d = 0; d < D; ++d) s += q[d] * ks[j][d];
                const float mnew = fmaxf(m, s);
                const float alpha = expf(m - mnew);
                const float p = expf(s - mnew);
                l = l * alpha + p;
                for (int d = 0; d < D; ++d) o[d] = o[d] * alpha + p * vs[j][d];
                m = mnew;
            }
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int d = 0; d < D; ++d) O[qi * qs + h * D + d] = o[d] * inv;
    LSE[int64_t(h) * L + qi] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kRows) void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       const float* __restrict__ delta, float* __restrict__ dQ,
                                                       const int32_t* __restrict__ se,
                                                       const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ row_ent, int L, int Hq, int Hkv,
                                                       float scale) {
    __shared__ float ks[kChunk][D + 1], vs[kChunk][D + 1];
    __shared__ int ses[kChunk];
    const int h = blockIdx.y, qb = blockIdx.x >> 1;
    const int qi = qb * kBlock + (blockIdx.x & 1) * kRows + threadIdx.x;
    const int hkv = h / (Hq / Hkv);
    const int64_t qs = int64_t(Hq) * D, kvs = int64_t(Hkv) * D;
    float q[D], g[D], dq[D];
    for (int d = 0; d < D; ++d) {
        q[d] = Q[qi * qs + h * D + d];
        g[d] = dO[qi * qs + h * D + d];
        dq[d] = 0.f;
    }
    const float lse = LSE[int64_t(h) * L + qi], dl = delta[int64_t(h) * L + qi];
    for (int e = row_ptr[qb]; e < row_ptr[qb + 1]; ++e) {
        const int kb = row_ent[e] >> 1;
        const bool partial = row_ent[e] & 1;
        for (int c = 0; c < kBlock / kChunk; ++c) {
            const int k0 = kb * kBlock + c * kChunk;
            __syncthreads();
            for (int idx = threadIdx.x; idx < kChunk * D; idx += kRows) {
                const int r = idx / D, d = idx % D;
                ks[r][d] = K[(k0 + r) * kvs + hkv * D + d];
                vs[r][d] = V[(k0 + r) * kvs + hkv * D + d];
            }
            if (threadIdx.x < kChunk) ses[threadIdx.x] = se[k0 + threadIdx.x];
            __syncthreads();
            for (int j = 0; j < kChunk; ++j) {
                const int key = k0 + j;
                if (partial && !(key <= qi && qi <= ses[j])) continue;
                float s = 0.f, dp = 0.f;
                for (int d = 0; d < D; ++d) {
                    s += q[d] * ks[j][d];
                    dp += g[d] * vs[j][d];
                }
                const float p = expf(s * scale - lse);
                const float ds = p * (dp - dl);
                for (int d = 0; d < D; ++d) dq[d] += ds * ks[j][d];
            }
        }
    }
    for (int d = 0; d < D; ++d) dQ[qi * qs + h * D + d] = dq[d] * scale;
}

// dK (kDK) or dV (!kDK) of one key row per thread, summed over the query
// heads of its key/value head.
template <int D, bool kDK>
__global__ __launch_bounds__(kRows) void dkv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        const float* __restrict__ delta, float* __restrict__ dX,
                                                        const int32_t* __restrict__ se,
                                                        const int32_t* __restrict__ col_ptr,
                                                        const int32_t* __restrict__ col_ent, int L, int Hq,
                                                        int Hkv, float scale) {
    __shared__ float qsm[kChunk][D + 1], gsm[kChunk][D + 1];
    __shared__ float lsm[kChunk], dsm[kChunk];
    const int hkv = blockIdx.y, kb = blockIdx.x >> 1;
    const int kj = kb * kBlock + (blockIdx.x & 1) * kRows + threadIdx.x;
    const int grp = Hq / Hkv;
    const int64_t qs = int64_t(Hq) * D, kvs = int64_t(Hkv) * D;
    const int sej = se[kj];
    float k[D], v[D], acc[D];
    for (int d = 0; d < D; ++d) {
        k[d] = K[kj * kvs + hkv * D + d];
        v[d] = kDK ? V[kj * kvs + hkv * D + d] : 0.f;
        acc[d] = 0.f;
    }
    for (int e = col_ptr[kb]; e < col_ptr[kb + 1]; ++e) {
        const int qb = col_ent[e] >> 1;
        const bool partial = col_ent[e] & 1;
        for (int h = hkv * grp; h < (hkv + 1) * grp; ++h) {
            for (int c = 0; c < kBlock / kChunk; ++c) {
                const int q0 = qb * kBlock + c * kChunk;
                __syncthreads();
                for (int idx = threadIdx.x; idx < kChunk * D; idx += kRows) {
                    const int r = idx / D, d = idx % D;
                    qsm[r][d] = Q[(q0 + r) * qs + h * D + d];
                    gsm[r][d] = dO[(q0 + r) * qs + h * D + d];
                }
                if (threadIdx.x < kChunk) {
                    lsm[threadIdx.x] = LSE[int64_t(h) * L + q0 + threadIdx.x];
                    dsm[threadIdx.x] = delta[int64_t(h) * L + q0 + threadIdx.x];
                }
                __syncthreads();
                for (int i = 0; i < kChunk; ++i) {
                    const int qi = q0 + i;
                    if (partial && !(kj <= qi && qi <= sej)) continue;
                    float s = 0.f;
                    for (int d = 0; d < D; ++d) s += qsm[i][d] * k[d];
                    const float p = expf(s * scale - lsm[i]);
                    if (kDK) {
                        float dp = 0.f;
                        for (int d = 0; d < D; ++d) dp += gsm[i][d] * v[d];
                        const float ds = p * (dp - dsm[i]);
                        for (int d = 0; d < D; ++d) acc[d] += ds * qsm[i][d];
                    } else {
                        for (int d = 0; d < D; ++d) acc[d] += p * gsm[i][d];
                    }
                }
            }
        }
    }
    for (int d = 0; d < D; ++d) dX[kj * kvs + hkv * D + d] = kDK ? acc[d] * scale : acc[d];
}

// delta[h][i] = dO[i,h,:] . O[i,h,:]; one wave per (token, head) row.
__global__ __launch_bounds__(256) void delta_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                                                        float* __restrict__ delta, int L, int Hq, int D) {
    const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= int64_t(L) * Hq) return;
    const int i = int(row / Hq), h = int(row % Hq);
    float acc = 0.f;
    for (int d = lane; d < D; d += 64) acc += O[int64_t(row) * D + d] * dO[int64_t(row) * D + d];
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) delta[int64_t(h) * L + i] = acc;
}

template <int D>
void launch_f32_bwd_d(int phase, const float* q, const float* k, const float* v, const float* dout, const float* lse,
                      const float* delta, float* dq, float* dk, float* dv, const int32_t* se,
                      const MetaPtrs& mp, const AttnShape& sh, hipStream_t stream) {
    const int L = int(sh.L);
    if (phase == kPhaseAll || phase == kPhaseDkdv) {
        dkv_f32_kernel<D, true><<<dim3(2 * sh.nb, sh.Hkv), kRows, 0, stream>>>(
            q, k, v, dout, lse, delta, dk, se, mp.col_ptr, mp.col_ent, L, sh.Hq, sh.Hkv, sh.scale);
        dkv_f32_kernel<D, false><<<dim3(2 * sh.nb, sh.Hkv), kRows, 0, stream>>>(
            q, k, v, dout, lse, delta, dv, se, mp.col_ptr, mp.col_ent, L, sh.Hq, sh.Hkv, sh.scale);
    }
    if (phase == kPhaseAll || phase == kPhaseDq)
        dq_f32_kernel<D><<<dim3(2 * sh.nb, sh.Hq), kRows, 0, stream>>>(q, k, v, dout, lse, delta, dq, se,
                                                                         mp.row_ptr, mp.row_ent, L, sh.Hq, sh.Hkv,
                                                                         sh.scale);
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const int32_t* se, const MetaPtrs& mp, const AttnShape& sh, hipStream_t stream) {
    const dim3 grid(2 * sh.nb, sh.Hq);
    const int L = int(sh.L);
    switch (sh.D) {
        case 32:
            fwd_f32_kernel<32><<<grid, kRows, 0, stream>>>(q, k, v, o, lse, se, mp.row_ptr, mp.row_ent, L, sh.Hq,
                                                            sh.Hkv, sh.scale);
            break;
        case 64:
            fwd_f32_kernel<64><<<grid, kRows, 0, stream>>>(q, k, v, o, lse, se, mp.row_ptr, mp.row_ent, L, sh.Hq,
                                                            sh.Hkv, sh.scale);
            break;
        case 128:
            fwd_f32_kernel<128><<<grid, kRows, 0, stream>>>(q, k, v, o, lse, se, mp.row_ptr, mp.row_ent, L,
                                                             sh.Hq, sh.Hkv, sh.scale);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bwd_f32(int phase, const float* q, const float* k, const float* v, const float* o, const float* lse,
                          const float* dout, float* dq, float* dk, float* dv, const int32_t* se,
                          const MetaPtrs& mp, float* delta, const AttnShape& sh, hipStream_t stream) {
    const int64_t rows = sh.L * sh.Hq;
    if (phase == kPhaseAll || phase == kPhaseDelta || phase == kPhaseDqDelta)
        delta_f32_kernel<<<dim3(unsigned((rows + 3) / 4)), 256, 0, stream>>>(o, dout, delta, int(sh.L), sh.Hq, sh.D);
    if (phase == kPhaseDelta) return hipGetLastError();
    if (phase == kPhaseDqDelta) phase = kPhaseDq;
    switch (sh.D) {
        case 32: launch_f32_bwd_d<32>(phase, q, k, v, dout, lse, delta, dq, dk, dv, se, mp, sh, stream); break;
        case 64: launch_f32_bwd_d<64>(phase, q, k, v, dout, lse, delta, dq, dk, dv, se, mp, sh, stream); break;
        case 128: launch_f32_bwd_d<128>(phase, q, k, v, dout, lse, delta, dq, dk, dv, se, mp, sh, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace treeattn
